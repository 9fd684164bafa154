// Forward pass of packed segment-id masked attention.
//
// Per head, O = softmax(scale * Q K^T over allowed pairs) V and LSE = log of the
// softmax denominator; rows without an allowed key get O = 0, LSE = -inf.  The
// pair predicate is "same seq id, id >= 0" ("Furniture packing, variable length"
// report, implementation part); the kernel visits only the non-empty key tiles
// of its query tile (block sparsity from the seq ids, "LingBot-VA packing"
// report, section 2.2) and applies the elementwise mask only on partial tiles.
//
// bf16 kernels (gfx950 MFMA).  128-wide heads use the ping-pong kernel below
// (8 waves per query tile, MFMA and softmax phases alternating between two
// wave groups); 64-wide heads use the 4-wave kernel described here.
//
// 4-wave kernel: a workgroup of 4 waves owns one 128-row query tile
// of one head; wave w owns query rows 32w..32w+31.  The scores are computed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the query index runs
// along the lanes, so the row max and row sum of the online softmax are
// in-lane reductions plus a single exchange between the two half-waves, the
// per-query rescale of the output is a per-lane multiply, and the fp32 score
// accumulator, converted to bf16, is directly the B operand of
// O^T += V^T P^T (the key order inside each 16-key slice is permuted the same
// way on both operands).  K is staged in LDS row-major and V transposed, in
// 64-key sub-tiles, double-buffered with one barrier per sub-tile; Q stays in
// registers for the whole loop.
//
// fp32 kernel: a plain one-thread-per-query-row loop with K/V staged in LDS,
// exact expf; it serves fp32 inputs (correctness path).
#include <math.h>

#include <type_traits>

#include "pa_common.h"
#include "pa_tile.h"

namespace {

using namespace pa;

// ------------------------------------------------------------------ bf16 MFMA
constexpr int kFwdSub = 64;          // key rows per inner step
constexpr int kFwdTile = 64 * kRowBytes;  // one 64-row LDS tile
constexpr int kFwdStage = 2 * kFwdTile + 256;  // K tile, V tile, 64 key ids
// Rescale threshold (log2 units): the running max is only raised when a new
// score exceeds it by more than this, so exp2 arguments stay <= kLazy and the
// O rescale is skipped for almost every step.
constexpr float kLazy = 8.0f;

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, const int32_t* __restrict__ q_ids,
                const int32_t* __restrict__ kv_ids, int32_t nq, int32_t nkv, int32_t H,
                float s2, const uint8_t* __restrict__ tile_class,
                const int32_t* __restrict__ q_ptr, const int32_t* __restrict__ q_cols,
                const int32_t* __restrict__ q_order, int32_t nkt, uint16_t* __restrict__ o,
                float* __restrict__ lse) {
  constexpr int kDB = D / 32, kKK = D / 16;
  __shared__ __attribute__((aligned(1024))) char st0[kFwdStage];
  __shared__ __attribute__((aligned(1024))) char st1[kFwdStage];

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int hi = lane >> 5, col = lane & 31;
  int work, h;
  block_work(blockIdx.x, H, (nq + 127) / 128, &work, &h);
  const int qt = q_order[work];
  const int beg = q_ptr[qt];
  const int nsub = 2 * (q_ptr[qt + 1] - beg);
  const size_t rs = (size_t)H * D;  // elements between consecutive tokens
  const int hoff = h * D;

  const int qrow = qt * 128 + wv * 32 + col;
  const bool qin = qrow < nq;
  const int qid = qin ? q_ids[qrow] : -1;
  const bool qvalid = qid >= 0;

  bf16x8 qf[kKK];
  {
    const uint16_t* qp = q + (size_t)(qin ? qrow : nq - 1) * rs + hoff + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) qf[kk] = *(const bf16x8*)(qp + 16 * kk);
  }
  const int rb = row_base(lane), tb = tr_base(lane);

  f32x16 oacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  auto stage = [&](int s, char* base) {
    const int kt = q_cols[beg + (s >> 1)];
    const int k0 = kt * 128 + (s & 1) * kFwdSub;
    stage_tile<D, kFwdSub, 4>(k, rs, hoff, k0, nkv, base, wv, lane);
    stage_tile<D, kFwdSub, 4>(v, rs, hoff, k0, nkv, base + kFwdTile, wv, lane);
    if (wv == 0) stage_ids(kv_ids, k0, nkv, base + 2 * kFwdTile, lane);
  };

  if (nsub > 0) stage(0, st0);
  // Two LDS stage arrays and a loop unrolled by two: each step reads one
  // array while the next stage's direct loads fill the other, so the
  // compiler can see that its LDS reads never wait for those loads.
  auto step = [&](int s, const char* base, char* next) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();  // stage s is in LDS; every wave is done with stage s - 1
    if (s + 1 < nsub) stage(s + 1, next);
    const int kt = q_cols[beg + (s >> 1)];
    const bool partial = tile_class_at(tile_class, (size_t)qt * nkt + kt) == 1;

    // S^T = K Q^T: 64 keys (two 32-key blocks) x this wave's 32 queries; lane
    // holds keys 32mb + 8(j/4) + 4hi + j%4 of query `col`
    // K operands of the first key block are all requested before the first
    // MFMA; each slot is refilled for the second block right after its use.
    f32x16 sacc[2];
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[0][j] = sacc[1][j] = 0.f;
    bf16x8 ka[kKK];
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) ka[kk] = lds_row8(base, row_at(rb, kk));
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[kk], sacc[0], 0, 0, 0);
      ka[kk] = lds_row8(base, row_at(rb, kk) + 8192);
    }
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk)
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[kk], sacc[1], 0, 0, 0);
    if (partial) {
      const int32_t* il = (const int32_t*)(base + 2 * kFwdTile);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = mb * 32 + 8 * g + 4 * hi;
          const int4 t4 = *(const int4*)(il + r0);  // -1 past the end of the keys
          // branch-free: bitwise & of the conditions, then a select
          const bool ok0 = qvalid & (t4.x == qid);
          const bool ok1 = qvalid & (t4.y == qid);
          const bool ok2 = qvalid & (t4.z == qid);
          const bool ok3 = qvalid & (t4.w == qid);
          sacc[mb][4 * g + 0] = ok0 ? sacc[mb][4 * g + 0] : -INFINITY;
          sacc[mb][4 * g + 1] = ok1 ? sacc[mb][4 * g + 1] : -INFINITY;
          sacc[mb][4 * g + 2] = ok2 ? sacc[mb][4 * g + 2] : -INFINITY;
          sacc[mb][4 * g + 3] = ok3 ? sacc[mb][4 * g + 3] : -INFINITY;
        }
    }
    // online softmax on raw scores (scale folded into the exp2 argument)
    float mx = sacc[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[mb][j]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * s2;
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazy)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
      m = mnew;
    }
    const float nm = m == -INFINITY ? 0.f : -m;
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int mb = kb >> 1, b0 = (kb & 1) * 8;
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[mb][b0 + e], s2, nm));
        lsum += p[e];
      }
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
      pb[kb] = __builtin_bit_cast(bf16x8, w);
    }
    // O^T += V^T P^T, V^T read transposed from the row-major V tile
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 a = join8(lds_tr4(base + kFwdTile, tr_at(tb, db, 0) + 4096 * kb),
                               lds_tr4(base + kFwdTile, tr_at(tb, db, 1) + 4096 * kb));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb], oacc[db], 0, 0, 0);
      }
    };
  for (int s = 0; s < nsub; s += 2) {
    step(s, st0, st1);
    if (s + 1 < nsub) step(s + 1, st1, st0);
  }

  // epilogue: both half-waves hold partial sums of the same query
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  const bool any = ltot > 0.f;
  const float inv = any ? 1.f / ltot : 0.f;
  if (qin) {
    uint16_t* op = o + (size_t)qrow * rs + hoff;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // rows without an allowed key have an all-zero accumulator and inv = 0
        u32x2 pk;
        pk[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        pk[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *(u32x2*)(op + db * 32 + 8 * g + 4 * hi) = pk;
      }
    if (hi == 0) lse[(size_t)h * nq + qrow] = any ? (m + log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// Ping-pong variant: a workgroup of 8 waves per 128-row query tile.  Wave w
// owns query rows 32(w%4)..+31 and one half of every 128-key tile: waves 0-3
// (group A) keys 0-63, waves 4-7 (group B) keys 64-127, each with its own
// online-softmax state; the two halves are merged at the end.  Work alternates
// in phases separated by barriers: while one group runs its MFMAs (the previous
// tile's PV and this tile's scores) the other runs its softmax on the VALU, and
// the next phase swaps.  Waves w and w+4 sit on the same SIMD (waves are dealt
// to the SIMDs in order), so every SIMD has one MFMA wave and one VALU wave at
// a time instead of two waves that drift into the same phase.
//
// Each group stages only its own half of the K and V tiles (K one tile ahead,
// V one tile behind, two buffers each), one direct load at a time between the
// instructions of its first phase of the step -- group A between its MFMAs,
// group B between its softmax instructions -- so the loads of all eight waves
// never queue up at once in front of the CU's address unit.
constexpr int kPPTile = 128 * kRowBytes;  // one 128-key tile (32 KB)
constexpr int kPPIds = 512;               // 128 key ids after a K tile
constexpr int kPPHalf = 64 * kRowBytes;   // one group's 64 keys of a tile

// Buffer resource over the rows row0 .. n - 1 of a [n][rs] bf16 tensor: reads
// at or past row n return zeros (the hardware's range check), so a tail tile
// needs no clamping.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* g, size_t rs, int row0,
                                                            int n) {
  const uint64_t bytes = row0 < n ? (uint64_t)(n - row0) * rs * 2 : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(g + (size_t)row0 * rs), 0,
                                           (int)(bytes > 0xFFFFFFFFull ? 0xFFFFFFFFull : bytes),
                                           0x00020000);
}

// One direct load of row group `blk` (rows 4 blk .. 4 blk + 3, 1 KB) of a
// 64-row half tile: lane i fetches the 16 bytes that land at offset 16 i of
// the group (the swizzled chunk of its row); `lane_off` is the lane's byte
// offset inside row group 0, which does not depend on blk.  No per-lane address
// arithmetic beyond one add, so it can sit between the MFMAs or VALU
// instructions of a phase.
__device__ __forceinline__ void stage_piece(__amdgpu_buffer_rsrc_t rsrc, uint32_t lane_off,
                                            uint32_t group_bytes, char* half_tile, int blk) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(half_tile + blk * 1024), 16,
                                           lane_off + blk * group_bytes, 0, 0, 0);
}

template <int D>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_pp_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, const int32_t* __restrict__ q_ids,
                   const int32_t* __restrict__ kv_ids, int32_t nq, int32_t nkv, int32_t H,
                   float s2, const uint8_t* __restrict__ tile_class,
                   const int32_t* __restrict__ q_ptr, const int32_t* __restrict__ q_cols,
                   const int32_t* __restrict__ q_order, int32_t nkt, uint16_t* __restrict__ o,
                   float* __restrict__ lse) {
  static_assert(D == 128, "the ping-pong forward is laid out for 128-wide heads");
  constexpr int kDB = D / 32, kKK = D / 16;
  // separate arrays, so the compiler sees that the reads of one buffer never
  // wait for the direct loads into another
  __shared__ __attribute__((aligned(1024))) char kb0[kPPTile + kPPIds];
  __shared__ __attribute__((aligned(1024))) char kb1[kPPTile + kPPIds];
  __shared__ __attribute__((aligned(1024))) char vb0[kPPTile];
  __shared__ __attribute__((aligned(1024))) char vb1[kPPTile];

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int hi = lane >> 5, col = lane & 31;
  const int grp = wv >> 2, wq = wv & 3;
  int work, h;
  block_work(blockIdx.x, H, (nq + 127) / 128, &work, &h);
  const int qt = q_order[work];
  const int beg = q_ptr[qt];
  const int n = q_ptr[qt + 1] - beg;  // key tiles of this query tile
  const size_t rs = (size_t)H * D;
  const int hoff = h * D;
  const int half = grp * kPPHalf;  // this group's 64 keys inside a tile

  const int qrow = qt * 128 + wq * 32 + col;
  const bool qin = qrow < nq;
  const int qid = qin ? q_ids[qrow] : -1;
  const bool qvalid = qid >= 0;

  bf16x8 qf[kKK];
  {
    const uint16_t* qp = q + (size_t)(qin ? qrow : nq - 1) * rs + hoff + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) qf[kk] = *(const bf16x8*)(qp + 16 * kk);
  }
  const int rb = row_base(lane), tb = tr_base(lane);

  f32x16 oacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  f32x16 sacc[2];
  bf16x8 pb[4];

  // Scalar per-tile values are fetched one step ahead, during a softmax phase,
  // and consumed before the next MFMA phase: an outstanding scalar load would
  // force every LDS operand wait in the MFMA phase down to zero.
  // kt_c / kt_n: key tiles t and t + 1; partial_c: tile t needs the mask.
  int kt_c = n > 0 ? q_cols[beg] : 0;
  int kt_n = n > 1 ? q_cols[beg + 1] : 0;
  bool partial_c = n > 0 && tile_class_at(tile_class, (size_t)qt * nkt + kt_c) == 1;

  // This wave's share of the loads of one step: pieces 0-3 are K rows of tile
  // ktk, pieces 4-7 V rows of tile ktv, all in this group's half.
  // Every piece of this wave has row groups blk = wq + 4 j, whose swizzle
  // (4 (lane / 16) + blk % 4 on the chunk) is the same for all four.
  const uint32_t group_bytes = (uint32_t)(4 * rs * 2);
  const uint32_t lane_off =
      (uint32_t)((((size_t)(lane >> 4) * rs + hoff) * 2) +
                 (((lane & 15) ^ (4 * (lane >> 4) + wq)) << 4));
  const auto load_piece = [&](int j, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                              char* kdst, char* vdst) __attribute__((always_inline)) {
    if (j < 4)
      stage_piece(rk, lane_off, group_bytes, kdst + half, wq + 4 * j);
    else
      stage_piece(rv, lane_off, group_bytes, vdst + half, wq + 4 * (j - 4));
  };
  const auto k_rsrc = [&](int kt) { return rows_rsrc(k, rs, kt * 128 + 64 * grp, nkv); };
  const auto v_rsrc = [&](int kt) { return rows_rsrc(v, rs, kt * 128 + 64 * grp, nkv); };
  const auto load_ids = [&](int ktk, char* kdst) __attribute__((always_inline)) {
    if (wq == 0) stage_ids(kv_ids, ktk * 128 + 64 * grp, nkv, kdst + kPPTile + 256 * grp, lane);
  };

  // MFMA phase: O^T += V^T P^T of the previous tile (V from vprev), then
  // S^T = K Q^T of this tile (K from kcur), masked on partial tiles.  With no
  // second MFMA wave on the SIMD, the LDS latency of the operand reads has to
  // hide behind this wave's own MFMAs: the MFMAs go in batches of four, and
  // the reads of batch b + 1 are issued right after the first MFMA of batch b
  // (registers for two batches), pinned in that order by scheduling groups;
  // `hook(b)` (this step's direct loads, or nothing) follows them.
  //   MFMA i <  16: PV, kb = i / 4, db = i % 4 (A = V^T slice, B = pb[kb])
  //   MFMA i >= 16: S,  kk = (i - 16) / 2, mb = (i - 16) % 2 (A = K rows, B = qf[kk])
  // kind: 0 = scores only (first tile), 1 = PV only (after the last tile), 2 = both
  const auto mfma_phase = [&](auto kind, const char* kcur, const char* vprev, bool partial,
                              auto hook) __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    const char* vb = vprev + half;
    const char* kb_ = kcur + half;
    const auto load_op = [&](int i) __attribute__((always_inline)) {
      if (i < 16) {
        const int kb = i >> 2, db = i & 3;
        return join8(lds_tr4(vb, tr_at(tb, db, 0) + 4096 * kb),
                     lds_tr4(vb, tr_at(tb, db, 1) + 4096 * kb));
      }
      const int kk = (i - 16) >> 1, mb = (i - 16) & 1;
      return lds_row8(kb_, row_at(rb, kk) + 8192 * mb);
    };
    const auto do_mfma = [&](int i, bf16x8 a) __attribute__((always_inline)) {
      if (i < 16) {
        const int kb = i >> 2, db = i & 3;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb], oacc[db], 0, 0, 0);
      } else {
        const int kk = (i - 16) >> 1, mb = (i - 16) & 1;
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[mb], 0, 0, 0);
      }
    };
    constexpr int first = K == 0 ? 16 : 0, last = K == 1 ? 16 : 32;
    if (K != 1) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[0][j] = sacc[1][j] = 0.f;
    }
    bf16x8 op[2][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) op[0][e] = load_op(first + e);
    if (first < 16)
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    else
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int b = first; b < last; b += 4) {
      const int cur = ((b - first) >> 2) & 1;
      do_mfma(b, op[cur][0]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (b + 4 < last) {
#pragma unroll
        for (int e = 0; e < 4; ++e) op[cur ^ 1][e] = load_op(b + 4 + e);
        if (b + 4 < 16)
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
      hook((b - first) >> 2);
#pragma unroll
      for (int e = 1; e < 4; ++e) do_mfma(b + e, op[cur][e]);
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    }
    if (K != 1 && partial) {
      const int32_t* il = (const int32_t*)(kcur + kPPTile) + 64 * grp;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int4 t4 = *(const int4*)(il + mb * 32 + 8 * g + 4 * hi);  // -1 past the end
          const bool ok0 = qvalid & (t4.x == qid);
          const bool ok1 = qvalid & (t4.y == qid);
          const bool ok2 = qvalid & (t4.z == qid);
          const bool ok3 = qvalid & (t4.w == qid);
          sacc[mb][4 * g + 0] = ok0 ? sacc[mb][4 * g + 0] : -INFINITY;
          sacc[mb][4 * g + 1] = ok1 ? sacc[mb][4 * g + 1] : -INFINITY;
          sacc[mb][4 * g + 2] = ok2 ? sacc[mb][4 * g + 2] : -INFINITY;
          sacc[mb][4 * g + 3] = ok3 ? sacc[mb][4 * g + 3] : -INFINITY;
        }
    }
  };

  // softmax phase: online softmax of the scores, P as bf16 MFMA operands;
  // `hook(j)`, j = 0..7, places this step's direct loads between the exp blocks
  const auto softmax_phase = [&](auto hook) __attribute__((always_inline)) {
    float mx = sacc[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[mb][j]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * s2;
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazy)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
      m = mnew;
    }
    const float nm = m == -INFINITY ? 0.f : -m;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int mb = kb >> 1, b0 = (kb & 1) * 8;
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[mb][b0 + e], s2, nm));
        lsum += p[e];
      }
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
      pb[kb] = __builtin_bit_cast(bf16x8, w);
      hook(2 * kb);
      hook(2 * kb + 1);
    }
    // the results exist here: keeps the compiler from sinking the softmax
    // past the barrier that ends the phase, into the MFMA phase that uses it
    asm volatile("" ::"v"(pb[0]), "v"(pb[1]), "v"(pb[2]), "v"(pb[3]), "v"(lsum));
  };

  // Group A runs, per key tile t, the MFMA phase t (PV of tile t - 1, scores
  // of tile t) and then the softmax of tile t; group B the softmax of tile
  // t - 1 and then the MFMA phase t, so the groups are one phase apart.  Each
  // step has two barriers: a plain one between its phases (it only keeps the
  // groups in step; no buffer changes hands there; the scheduling fences keep
  // each phase's instructions on its side) and one after the wait for the
  // step's loads (K of tile t + 1, V of tile t), which the next step reads.
  // A barrier that only orders the waves: no wait for outstanding loads (each
  // group waits for its own loads where it needs them), and no instruction or
  // memory access crosses it.
  const auto barrier = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  int kt_nn = 0, partial_n = 0;
  // next step's scalars: fetched at the start of a softmax phase ...
  const auto fetch_next = [&](int t) __attribute__((always_inline)) {
    kt_nn = t + 2 < n ? q_cols[beg + t + 2] : 0;
    partial_n = t + 1 < n ? tile_class_at(tile_class, (size_t)qt * nkt + kt_n) == 1 : 0;
  };
  // ... and in registers by its end
  const auto land_next = [&]() __attribute__((always_inline)) {
    asm volatile("" ::"s"(kt_nn), "s"(partial_n));
  };
  const auto rotate = [&]() __attribute__((always_inline)) {
    kt_c = kt_n;
    kt_n = kt_nn;
    partial_c = partial_n;
  };
  const auto no_hook = [](int) {};
  // K of tile t + 1 (the last step re-reads tile t into the unused buffer)
  const auto ktk_of = [&](int t) { return t + 1 < n ? kt_n : kt_c; };
  // MFMA phase t with this group's loads for step t + 1 (K of tile t + 1, V of
  // tile t) between its MFMAs: each group issues its loads in its own MFMA
  // phase, so the address unit sees the two groups' loads in alternate phases
  const auto mfma_with_loads = [&](int t, auto kind, const char* kcur, char* knext,
                                   const char* vprev, char* vcur) __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    if (K != 1) {
      const int ktk = ktk_of(t);
      const auto rk = k_rsrc(ktk), rv = v_rsrc(kt_c);
      load_ids(ktk, knext);
      mfma_phase(kind, kcur, vprev, partial_c, [&](int b) __attribute__((always_inline)) {
        if (K == 2) {
          load_piece(b, rk, rv, knext, vcur);
        } else {
          load_piece(2 * b, rk, rv, knext, vcur);
          load_piece(2 * b + 1, rk, rv, knext, vcur);
        }
      });
    } else {
      mfma_phase(kind, kcur, vprev, partial_c, no_hook);
    }
  };
  // group A: MFMA phase t (its loads land by the end of the step), softmax t
  const auto step_a = [&](int t, auto kind, const char* kcur, char* knext, const char* vprev,
                          char* vcur) __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    mfma_with_loads(t, kind, kcur, knext, vprev, vcur);
    barrier();
    fetch_next(t);
    if (K != 1) softmax_phase(no_hook);
    land_next();
    rotate();
    wait_vmem();
    barrier();
  };
  // group B: softmax t - 1 (then its loads of the previous step have landed),
  // MFMA phase t
  const auto step_b = [&](int t, auto kind, const char* kcur, char* knext, const char* vprev,
                          char* vcur) __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    fetch_next(t);
    if (K != 0) softmax_phase(no_hook);
    land_next();
    wait_vmem();
    barrier();
    mfma_with_loads(t, kind, kcur, knext, vprev, vcur);
    rotate();
    barrier();
  };
  using First = std::integral_constant<int, 0>;
  using Last = std::integral_constant<int, 1>;
  using Mid = std::integral_constant<int, 2>;
  if (n > 0) {
    load_ids(kt_c, kb0);
    const auto rk = k_rsrc(kt_c);
#pragma unroll
    for (int j = 0; j < 4; ++j) load_piece(j, rk, rk, kb0, vb0);
  }
  wait_vmem();
  __syncthreads();
  // steps t = 0 .. n: the first computes scores only, the last PV only; the
  // middle ones alternate the buffer pairs
  char* const vlast = (n & 1) ? vb0 : vb1;  // V of tile n - 1
  if (grp == 0) {
    if (n > 0) {
      step_a(0, First{}, kb0, kb1, vb1, vb0);
      for (int t = 1; t < n; t += 2) {
        step_a(t, Mid{}, kb1, kb0, vb0, vb1);
        if (t + 1 < n) step_a(t + 1, Mid{}, kb0, kb1, vb1, vb0);
      }
      step_a(n, Last{}, kb0, kb1, vlast, vb0);
    }
  } else {
    if (n > 0) {
      step_b(0, First{}, kb0, kb1, vb1, vb0);
      for (int t = 1; t < n; t += 2) {
        step_b(t, Mid{}, kb1, kb0, vb0, vb1);
        if (t + 1 < n) step_b(t + 1, Mid{}, kb0, kb1, vb1, vb0);
      }
      step_b(n, Last{}, kb0, kb1, vlast, vb0);
    }
  }

  // merge: group B hands (O, running max, partial sum) to its group-A partner,
  // whose lanes hold the same (query, column) elements
  static_assert((16 * kDB + 2) * 64 * 4 <= kPPTile, "one wave's partial fits a buffer");
  float* xo = (float*)(wq == 0 ? kb0 : wq == 1 ? kb1 : wq == 2 ? vb0 : vb1);
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) xo[(16 * db + j) * 64 + lane] = oacc[db][j];
    xo[16 * kDB * 64 + lane] = m;
    xo[(16 * kDB + 1) * 64 + lane] = lsum;
  }
  __syncthreads();
  if (grp == 1) return;
  {
    const float mb_ = xo[16 * kDB * 64 + lane];
    const float lb = xo[(16 * kDB + 1) * 64 + lane];
    const float mn = fmaxf(m, mb_);
    const float ca = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    const float cb = mb_ == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mb_ - mn);
    lsum = lsum * ca + lb * cb;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        oacc[db][j] = oacc[db][j] * ca + xo[(16 * db + j) * 64 + lane] * cb;
    m = mn;
  }
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  const bool any = ltot > 0.f;
  const float inv = any ? 1.f / ltot : 0.f;
  if (qin) {
    uint16_t* op = o + (size_t)qrow * rs + hoff;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pk;
        pk[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        pk[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *(u32x2*)(op + db * 32 + 8 * g + 4 * hi) = pk;
      }
    if (hi == 0) lse[(size_t)h * nq + qrow] = any ? (m + log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// ------------------------------------------------------------------ fp32
constexpr int kF32Sub = 32;  // key rows staged per step

template <int D>
__global__ void __launch_bounds__(128)
fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
               const float* __restrict__ v, const int32_t* __restrict__ q_ids,
               const int32_t* __restrict__ kv_ids, int32_t nq, int32_t nkv, int32_t H,
               float scale, int32_t bq, int32_t bkv, const uint8_t* __restrict__ tile_class,
               const int32_t* __restrict__ q_ptr, const int32_t* __restrict__ q_cols,
               const int32_t* __restrict__ q_order, int32_t nkt, float* __restrict__ o,
               float* __restrict__ lse) {
  __shared__ float ks[kF32Sub][D];
  __shared__ float vs[kF32Sub][D];
  __shared__ int32_t is[kF32Sub];
  const int tid = threadIdx.x;
  const int work = blockIdx.x / H, h = blockIdx.x - work * H;
  const int qt = q_order[work];
  const size_t rs = (size_t)H * D;
  const int qrow = qt * bq + tid;
  const bool qin = tid < bq && qrow < nq;
  const int qtag = qin ? query_tag(q_ids[qrow]) : kPadQuery;
  float qr[D], acc[D];
  for (int d = 0; d < D; ++d) {
    qr[d] = qin ? q[(size_t)qrow * rs + h * D + d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int e = q_ptr[qt]; e < q_ptr[qt + 1]; ++e) {
    const int kt = q_cols[e];
    const bool partial = tile_class[(size_t)qt * nkt + kt] == 1;
    const int kend = min(kt * bkv + bkv, nkv);
    for (int k0 = kt * bkv; k0 < kend; k0 += kF32Sub) {
      const int n = min(kF32Sub, kend - k0);
      __syncthreads();
      for (int x = tid; x < kF32Sub * D; x += blockDim.x) {
        const int r = x / D, d = x % D;
        const int kr = min(k0 + r, nkv - 1);
        ks[r][d] = k[(size_t)kr * rs + h * D + d];
        vs[r][d] = v[(size_t)kr * rs + h * D + d];
      }
      for (int r = tid; r < kF32Sub; r += blockDim.x)
        is[r] = k0 + r < nkv ? key_tag(kv_ids[k0 + r]) : kPadKey;
      __syncthreads();
      for (int r = 0; r < n; ++r) {
        if (partial && is[r] != qtag) continue;
        float sc = 0.f;
        for (int d = 0; d < D; ++d) sc = fmaf(qr[d], ks[r][d], sc);
        sc *= scale;
        const float mn = fmaxf(m, sc);
        const float corr = expf(m - mn);
        const float p = expf(sc - mn);
        l = l * corr + p;
        for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[r][d], acc[d] * corr);
        m = mn;
      }
    }
  }
  if (qin) {
    const bool any = l > 0.f;
    for (int d = 0; d < D; ++d) o[(size_t)qrow * rs + h * D + d] = any ? acc[d] / l : 0.f;
    lse[(size_t)h * nq + qrow] = any ? m + logf(l) : -INFINITY;
  }
}

}  // namespace

namespace pa {

// Shared argument checks of the forward and backward entry points.
int32_t check_attn_args(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads, int32_t head_dim,
                        const pa_block_mask* mask) {
  if (!mask) return PA_ERR_NULL;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_HEADDIM;
  if (nq < 1 || nkv < 1 || heads < 1) return PA_ERR_SHAPE;
  if ((int64_t)nq * heads * head_dim > ((int64_t)1 << 40)) return PA_ERR_SHAPE;
  if (mask->nq != nq || mask->nkv != nkv) return PA_ERR_MASK_MISMATCH;
  if (mask->nq_tiles != (nq + mask->block_q - 1) / mask->block_q ||
      mask->nkv_tiles != (nkv + mask->block_kv - 1) / mask->block_kv)
    return PA_ERR_MASK_MISMATCH;
  if (dtype == PA_BF16) {
    if (mask->block_q != 128 || mask->block_kv != 128) return PA_ERR_MASK_MISMATCH;
  } else {
    const auto ok = [](int b) { return b == 32 || b == 64 || b == 128; };
    if (!ok(mask->block_q) || !ok(mask->block_kv)) return PA_ERR_MASK_MISMATCH;
  }
  if (!mask->tile_class || !mask->q_ptr || !mask->q_cols || !mask->kv_ptr || !mask->kv_rows ||
      !mask->q_order || !mask->kv_order)
    return PA_ERR_NULL;
  if ((int64_t)mask->nq_tiles * heads > INT32_MAX || (int64_t)mask->nkv_tiles * heads > INT32_MAX)
    return PA_ERR_SHAPE;
  return PA_OK;
}

}  // namespace pa

extern "C" int32_t attn_packed_fwd(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                                   int32_t head_dim, float scale, const void* q, const void* k,
                                   const void* v, const int32_t* q_seq_id,
                                   const int32_t* kv_seq_id, const pa_block_mask* mask, void* o,
                                   float* lse, void* stream) {
  int32_t st = pa::check_attn_args(dtype, nq, nkv, heads, head_dim, mask);
  if (st != PA_OK) return st;
  if (!q || !k || !v || !q_seq_id || !kv_seq_id || !o || !lse) return PA_ERR_NULL;
  if (!pa::aligned16(q) || !pa::aligned16(k) || !pa::aligned16(v) || !pa::aligned16(o))
    return PA_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(mask->nq_tiles * heads);
  if (dtype == PA_BF16) {
    const float s2 = scale * pa::kLog2e;
    if (head_dim == 128)
      hipLaunchKernelGGL(fwd_bf16_pp_kernel<128>, grid, dim3(512), 0, s, (const uint16_t*)q,
                         (const uint16_t*)k, (const uint16_t*)v, q_seq_id, kv_seq_id, nq, nkv,
                         heads, s2, mask->tile_class, mask->q_ptr, mask->q_cols, mask->q_order,
                         mask->nkv_tiles, (uint16_t*)o, lse);
    else
      hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, dim3(256), 0, s, (const uint16_t*)q,
                         (const uint16_t*)k, (const uint16_t*)v, q_seq_id, kv_seq_id, nq, nkv,
                         heads, s2, mask->tile_class, mask->q_ptr, mask->q_cols, mask->q_order,
                         mask->nkv_tiles, (uint16_t*)o, lse);
  } else {
    const dim3 block(mask->block_q);
    if (head_dim == 128)
      hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, s, (const float*)q, (const float*)k,
                         (const float*)v, q_seq_id, kv_seq_id, nq, nkv, heads, scale,
                         mask->block_q, mask->block_kv, mask->tile_class, mask->q_ptr,
                         mask->q_cols, mask->q_order, mask->nkv_tiles, (float*)o, lse);
    else
      hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, s, (const float*)q, (const float*)k,
                         (const float*)v, q_seq_id, kv_seq_id, nq, nkv, heads, scale,
                         mask->block_q, mask->block_kv, mask->tile_class, mask->q_ptr,
                         mask->q_cols, mask->q_order, mask->nkv_tiles, (float*)o, lse);
  }
  return pa::launch_status();
}
