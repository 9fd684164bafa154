// Forward pass of packed segment-id masked attention.
//
// Per head, O = softmax(scale * Q K^T over allowed pairs) V and LSE = log of the
// softmax denominator; rows without an allowed key get O = 0, LSE = -inf.  The
// pair predicate is "same seq id, id >= 0" ("Furniture packing, variable length"
// report, implementation part); the kernel visits only the non-empty key tiles
// of its query tile (block sparsity from the seq ids, "LingBot-VA packing"
// report, section 2.2) and applies the elementwise mask only on partial tiles.
//
// bf16 kernels (gfx950 MFMA).  128-wide heads use the paired ping-pong kernel
// below (8 waves per pair of query tiles, MFMA and softmax phases alternating
// between two wave groups); 64-wide heads use the 4-wave kernel described here.
// Both compute in the same layout.
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
#include <limits.h>
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
    mx = half_max(mx) * s2;
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
  const float ltot = half_sum(lsum);
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

// Paired ping-pong variant: a workgroup of 8 waves per PAIR of query tiles,
// the tiles at positions 2w and 2w + 1 of the longest-first order (equal or
// nearly equal key lists: for contiguous segments, two tiles of one segment).
// Group A (waves 0-3) owns the first tile, group B (waves 4-7) the second,
// wave w query rows 32(w%4)..+31 of its group's tile, each over all keys.  Both
// groups walk the same 64-key sub-tiles, one phase apart (A: MFMA phase then
// softmax; B: softmax then MFMA phase; one workgroup barrier per step, at its
// end), so each K/V sub-tile staged in LDS
// serves 256 query rows: half the staging traffic per flop of one tile per
// workgroup.  The sub-tiles walk the pair's list of the block mask: the key
// tiles one of the two query tiles has work with, ascending; a tile in the
// walk that is not in a group's list is fully masked for that group (class 0).
constexpr int kPrSub = 64 * kRowBytes;  // one 64-key sub-tile (16 KB)

template <int D>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_pair_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, const int32_t* __restrict__ q_ids,
                     const int32_t* __restrict__ kv_ids, int32_t nq, int32_t nkv, int32_t H,
                     float s2, const int32_t* __restrict__ q_order,
                     const int32_t* __restrict__ pair_off, const int32_t* __restrict__ pair_len,
                     const int32_t* __restrict__ pair_ent, uint16_t* __restrict__ o,
                     float* __restrict__ lse) {
  static_assert(D == 128, "the paired forward is laid out for 128-wide heads");
  constexpr int kDB = D / 32, kKK = D / 16;
  __shared__ __attribute__((aligned(1024))) char kb0[kPrSub + 256];
  __shared__ __attribute__((aligned(1024))) char kb1[kPrSub + 256];
  __shared__ __attribute__((aligned(1024))) char kb2[kPrSub + 256];
  __shared__ __attribute__((aligned(1024))) char vb0[kPrSub];
  __shared__ __attribute__((aligned(1024))) char vb1[kPrSub];
  __shared__ __attribute__((aligned(1024))) char vb2[kPrSub];

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int hi = lane >> 5, col = lane & 31;
  const int grp = wv >> 2, wq = wv & 3;
  const int nqt = (nq + 127) / 128;
  int work, h;
  block_work(blockIdx.x, H, (nqt + 1) / 2, &work, &h);
  const int qpair[2] = {q_order[2 * work], 2 * work + 1 < nqt ? q_order[2 * work + 1] : -1};
  const int qmine = qpair[grp];  // -1: no tile (odd tile count), no rows, all masked
  // The key walk: the pair's list from the block mask -- every key tile one of
  // the two query tiles has an allowed pair with, ascending, each entry the key
  // tile with both tiles' classes beside it; two 64-key sub-steps per tile.
  const int32_t* const pent = pair_ent + pair_off[work];
  const int n = 2 * pair_len[work];
  const size_t rs = (size_t)H * D;
  const int hoff = h * D;

  const int qrow = qmine * 128 + wq * 32 + col;
  const bool qin = qmine >= 0 && qrow < nq;
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

  // Walk entries as scalars: ent(s) is the entry of sub-step s (clamped to the
  // last one); the first key row of sub-step s comes from its entry, and the id
  // mask is needed unless this group's tile is full for that key tile (class 2;
  // partial, empty or no tile at all need it).  e1, e2 hold the entries of
  // sub-steps s + 1 and s + 2 at step s; the entry of s + 3 is fetched during
  // the step's VALU phase and waited for only at its end.
  const auto ent = [&](int s) { return pent[(s < n ? s : n - 1) >> 1]; };
  const auto k0_of = [&](int e, int s) {
    return (e & 0xFFFF) * 128 + 64 * ((s < n ? s : n - 1) & 1);
  };
  const int csh = 16 + 8 * grp;
  const auto needs_mask = [&](int e) { return ((e >> csh) & 0xFF) != 2; };
  int e1 = 0, e2 = 0, e3 = 0;
  bool partial_c = false;
  if (n > 0) {
    partial_c = needs_mask(ent(0));
    e1 = ent(1);
    e2 = ent(2);
  }

  // Group A stages the K sub-tiles (and their ids, by wave 0), group B the V
  // sub-tiles: 16 row groups over a group's four waves (row groups wq + 4 j,
  // one swizzle for all four).
  const uint32_t group_bytes = (uint32_t)(4 * rs * 2);
  const uint32_t lane_off =
      (uint32_t)((((size_t)(lane >> 4) * rs + hoff) * 2) +
                 (((lane & 15) ^ (4 * (lane >> 4) + wq)) << 4));
  // rows row0 .. nkv - 1 of a K or V tensor (reads past them return zeros)
  const auto rows = [&](const uint16_t* g, int row0) {
    const uint64_t bytes = row0 < nkv ? (uint64_t)(nkv - row0) * rs * 2 : 0;
    return raw_rsrc(g + (size_t)row0 * rs, bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes);
  };
  const auto load_piece = [&](int j, u32x4_t r, char* dst) __attribute__((always_inline)) {
    const int blk = wq + 4 * j;
    dma_b128(r, lane_off + blk * group_bytes, lds_address(dst + blk * 1024));
  };

  // MFMA phase: O^T += V^T P^T of the previous sub-tile (V from vprev), then
  // S^T = K Q^T of this one (K from kcur), masked unless the tile is full for
  // this group.  With no second MFMA wave on the SIMD, the LDS latency of the
  // operand reads has to hide behind this wave's own MFMAs: the MFMAs go in
  // batches of four, and the reads of batch b + 1 are issued right after the
  // first MFMA of batch b (registers for two batches), pinned in that order by
  // scheduling groups.
  //   MFMA i <  16: PV, kb = i / 4, db = i % 4 (A = V^T slice, B = pb[kb])
  //   MFMA i >= 16: S,  kk = (i - 16) / 2, mb = (i - 16) % 2 (A = K rows, B = qf[kk])
  // kind: 0 = scores only (first sub-tile), 1 = PV only (after the last), 2 = both
  const auto mfma_phase = [&](auto kind, const char* kcur, const char* vprev, bool partial)
                              __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    const auto load_op = [&](int i) __attribute__((always_inline)) {
      if (i < 16) {
        const int kb = i >> 2, db = i & 3;
        return join8(lds_tr4(vprev, tr_at(tb, db, 0) + 4096 * kb),
                     lds_tr4(vprev, tr_at(tb, db, 1) + 4096 * kb));
      }
      const int kk = (i - 16) >> 1, mb = (i - 16) & 1;
      return lds_row8(kcur, row_at(rb, kk) + 8192 * mb);
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
#pragma unroll
      for (int e = 1; e < 4; ++e) do_mfma(b + e, op[cur][e]);
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    }
    if (K != 1 && partial) {
      const int32_t* il = (const int32_t*)(kcur + kPrSub);
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

  const auto softmax_phase = [&]() __attribute__((always_inline)) {
    float mx = sacc[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[mb][j]);
    mx = half_max(mx) * s2;
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
    }
    // the results exist here: keeps the compiler from sinking the softmax
    // past the end of the phase, into the MFMA phase that uses it
    asm volatile("" ::"v"(pb[0]), "v"(pb[1]), "v"(pb[2]), "v"(pb[3]), "v"(lsum));
  };

  const auto barrier = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Between a group's two phases only a scheduling fence: no LDS buffer is
  // written in a step that another wave reads in it, and each group's own
  // results stay in its registers, so one barrier per step suffices.
  const auto fence = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  int partial_n = 0;
  const auto fetch_next = [&](int s) __attribute__((always_inline)) {
    const int t = s + 3 < n ? s + 3 : n - 1;
    e3 = sload_issue(pent + (t >> 1));  // lands at the end of the VALU phase
    partial_n = s + 1 < n ? needs_mask(e1) : 0;
  };
  const auto land_next = [&]() __attribute__((always_inline)) {
    sload_wait(e3);
    asm volatile("" ::"s"(partial_n));
    e1 = e2;
    e2 = e3;
  };
  // Three buffers each for K and V: sub-tile s sits in kb[s % 3] / vb[s % 3].
  // Step s stages K(s + 2) (group A) and V(s + 1) (group B), each group at the
  // start of its softmax phase; each wave waits for its previous step's
  // loads at the end of step s + 1, so a load has two steps to land.  Past the
  // last sub-tile the loads re-read sub-tile n - 1 into the free buffer, which
  // keeps the per-step load count (and so the partial waits) fixed.
  // Each wave of group A stages 16 of the sub-tile's 64 key ids (one load
  // with 16 active lanes), so every wave of a group issues the same number of
  // loads per step.  A sub-tile inside the keys takes the buffer form; the
  // tail one the per-lane form, which gives keys past the end the id -1.
  const u32x4_t ids_rsrc = raw_rsrc(kv_ids, (uint32_t)nkv * 4u);
  const auto load_ids = [&](int k0, char* kdst) __attribute__((always_inline)) {
    if ((lane >> 4) == wq) {
      const int i = k0 + lane;
      if (k0 + 64 <= nkv)
        dma_b32_buf(ids_rsrc, (uint32_t)i * 4u, lds_address(kdst + kPrSub));
      else
        dma_b32(i < nkv ? kv_ids + i : &kNoId, lds_address(kdst + kPrSub));
    }
  };
  // wait until only this step's loads are outstanding (loads finish in order):
  // group A issues 5 per step (4 K pieces + ids), group B 4 (V pieces)
  const auto wait_prev_a = [&](auto kind) __attribute__((always_inline)) {
    if (decltype(kind)::value == 1)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x0F75);  // vmcnt(5)
  };
  const auto wait_prev_b = [&](auto kind) __attribute__((always_inline)) {
    if (decltype(kind)::value == 1)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
  };
  // Each group issues its direct loads at the start of its softmax phase: the
  // other group is then in its MFMA phase, reading LDS at full rate, and loads
  // issued by an MFMA-phase wave stalled it (measured).
  // group A: MFMA phase s, then loads of K(s + 2) and softmax s
  const auto step_a = [&](int s, auto kind, const char* kcur, const char* vprev, char* kload)
                          __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    mfma_phase(kind, kcur, vprev, partial_c);
    fence();
    if (K != 1) {
      const int k0n = k0_of(e2, s + 2);
      const auto rk = rows(k, k0n);
      load_ids(k0n, kload);
#pragma unroll
      for (int j = 0; j < 4; ++j) load_piece(j, rk, kload);
    }
    fetch_next(s);
    if (K != 1) softmax_phase();
    land_next();
    partial_c = partial_n;
    wait_prev_a(kind);
    barrier();
  };
  // group B: loads of V(s + 1) and softmax s - 1, then MFMA phase s
  const auto step_b = [&](int s, auto kind, const char* kcur, const char* vprev, char* vload)
                          __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    if (K != 1) {
      const auto rv = rows(v, k0_of(e1, s + 1));
#pragma unroll
      for (int j = 0; j < 4; ++j) load_piece(j, rv, vload);
    }
    fetch_next(s);
    if (K != 0) softmax_phase();
    land_next();
    fence();
    mfma_phase(kind, kcur, vprev, partial_c);
    partial_c = partial_n;
    wait_prev_b(kind);
    barrier();
  };
  using First = std::integral_constant<int, 0>;
  using Last = std::integral_constant<int, 1>;
  using Mid = std::integral_constant<int, 2>;
  // prologue: K(0) -> kb0, K(1) -> kb1 (group A), V(0) -> vb0 (group B)
  if (n > 0) {
    if (grp == 0) {
      const int k00 = k0_of(ent(0), 0), k01 = k0_of(e1, 1);
      const auto r0 = rows(k, k00), r1 = rows(k, k01);
      load_ids(k00, kb0);
      load_ids(k01, kb1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        load_piece(j, r0, kb0);
        load_piece(j, r1, kb1);
      }
    } else {
      const auto r0 = rows(v, k0_of(ent(0), 0));
#pragma unroll
      for (int j = 0; j < 4; ++j) load_piece(j, r0, vb0);
    }
  }
  wait_vmem();
  __syncthreads();
  if (n > 0) {
    // buffers of step s (r = s % 3): kcur kb[r], vprev vb[(r + 2) % 3],
    // K load into kb[(r + 2) % 3], V load into vb[(r + 1) % 3]
    char* const vlast = (n - 1) % 3 == 0 ? vb0 : (n - 1) % 3 == 1 ? vb1 : vb2;
    if (grp == 0) {
      step_a(0, First{}, kb0, vb2, kb2);
      for (int s = 1; s < n; s += 3) {
        step_a(s, Mid{}, kb1, vb0, kb0);
        if (s + 1 < n) step_a(s + 1, Mid{}, kb2, vb1, kb1);
        if (s + 2 < n) step_a(s + 2, Mid{}, kb0, vb2, kb2);
      }
      step_a(n, Last{}, kb0, vlast, kb2);
    } else {
      step_b(0, First{}, kb0, vb2, vb1);
      for (int s = 1; s < n; s += 3) {
        step_b(s, Mid{}, kb1, vb0, vb2);
        if (s + 1 < n) step_b(s + 1, Mid{}, kb2, vb1, vb0);
        if (s + 2 < n) step_b(s + 2, Mid{}, kb0, vb2, vb1);
      }
      step_b(n, Last{}, kb0, vlast, vb0);
    }
  }

  const float ltot = half_sum(lsum);
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
      !mask->q_order || !mask->kv_order || !mask->pair_off || !mask->pair_len || !mask->pair_ent)
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
      hipLaunchKernelGGL(fwd_bf16_pair_kernel<128>, dim3((mask->nq_tiles + 1) / 2 * heads),
                         dim3(512), 0, s, (const uint16_t*)q,
                         (const uint16_t*)k, (const uint16_t*)v, q_seq_id, kv_seq_id, nq, nkv,
                         heads, s2, mask->q_order, mask->pair_off, mask->pair_len,
                         mask->pair_ent, (uint16_t*)o, lse);
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
