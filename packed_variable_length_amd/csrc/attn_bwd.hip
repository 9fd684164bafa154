// Backward pass of packed segment-id masked attention.
//
// Gradients of O = P V, P = softmax(scale * Q K^T over allowed pairs), with
// upstream dO (the standard softmax-attention gradient):
//   Delta_i = sum_d dO_id O_id          (row sums, fp32)
//   P_ij    = exp(scale * q_i.k_j - LSE_i) on allowed pairs, 0 elsewhere
//   dS_ij   = P_ij (dO_i.v_j - Delta_i)
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// Allowed pairs and block sparsity as in the forward ("Furniture packing,
// variable length" report, implementation part; "LingBot-VA packing" report,
// section 2.2); rows with no allowed pair get exact zero gradients.
//
// Two launches, none with atomics:
//   dq          query-major: first the row terms of its queries, Delta =
//               rowsum(dO * O) and LSE in log2 units (+inf on rows without an
//               allowed key, so exp2 gives P = 0 there), written for dkdv; then
//               S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T (query index
//               on the lanes).  For 64-wide heads and fp32 a separate
//               HBM-bound preprocess kernel computes the row terms first.
//   dkdv        key-major, one 128-row key tile per workgroup: S = Q K^T,
//               P (packed to bf16 at once), dP = dO V^T, dS from the bf16 P,
//               dV^T += dO^T P, dK^T += Q^T dS (key index on the lanes, dK and
//               dV accumulated in registers; sized to fit two waves per SIMD)
// Splitting dQ from dK/dV recomputes S and dP once more (14 instead of 10
// d*pairs flops per head) but needs no fp32 atomics, no zero-filled accumulator
// and no conversion pass, and is deterministic.
//
// The bf16 kernels stage K/V (dq) or Q/dO (dkdv) tiles in swizzled LDS with
// direct global->LDS loads; the operands whose contraction runs across rows
// (K^T, Q^T, dO^T) are read with ds_read_b64_tr_b16 from the same row-major
// tiles (see pa_tile.h).
#include <math.h>
#include <limits.h>

#include <mutex>
#include <type_traits>

#include "pa_common.h"
#include "pa_tile.h"

namespace {

using namespace pa;

// ------------------------------------------------------------------ preprocess
template <typename T>
__device__ __forceinline__ void load16(const T* p, float* out);

template <>
__device__ __forceinline__ void load16<uint16_t>(const uint16_t* p, float* out) {
  const u32x4 a = *(const u32x4*)p, b = *(const u32x4*)(p + 8);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    out[2 * w] = bf16_bits_to_f32(a[w] & 0xFFFFu);
    out[2 * w + 1] = bf16_bits_to_f32(a[w] >> 16);
    out[8 + 2 * w] = bf16_bits_to_f32(b[w] & 0xFFFFu);
    out[8 + 2 * w + 1] = bf16_bits_to_f32(b[w] >> 16);
  }
}
template <>
__device__ __forceinline__ void load16<float>(const float* p, float* out) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x4 a = *(const f32x4*)(p + 4 * w);
    out[4 * w] = a[0];
    out[4 * w + 1] = a[1];
    out[4 * w + 2] = a[2];
    out[4 * w + 3] = a[3];
  }
}

// Block = 256 / (D/16) consecutive query rows of one head (D/16 threads per
// row, 16 elements each), so both outputs are written coalesced.
template <typename T, int D>
__global__ void __launch_bounds__(256)
preprocess_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                  const float* __restrict__ lse, int32_t nq, int32_t H,
                  float* __restrict__ delta, float* __restrict__ lse2) {
  constexpr int kPer = D / 16;          // threads per row
  constexpr int kRows = 256 / kPer;     // rows per block
  const int h = blockIdx.x % H;
  const int i = (blockIdx.x / H) * kRows + threadIdx.x / kPer;
  const int part = threadIdx.x % kPer;
  float acc = 0.f;
  if (i < nq) {
    float a[16], b[16];
    const size_t off = ((size_t)i * H + h) * D + part * 16;
    load16<T>(o + off, a);
    load16<T>(dout + off, b);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc = fmaf(a[e], b[e], acc);
  }
#pragma unroll
  for (int s = kPer / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (i < nq && part == 0) {
    delta[(size_t)h * nq + i] = acc;
    const float l = lse[(size_t)h * nq + i];
    lse2[(size_t)h * nq + i] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// ------------------------------------------------------------------ bf16 dq
constexpr int kTile64 = 64 * kRowBytes;
constexpr int kDqStage = 2 * kTile64 + 256;  // K tile, V tile, 64 key ids

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
dq_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
               const float* __restrict__ delta, const float* __restrict__ lse2,
               const int32_t* __restrict__ q_ids, const int32_t* __restrict__ kv_ids,
               int32_t nq, int32_t nkv, int32_t H, float s2, float scale,
               const uint8_t* __restrict__ tile_class, const int32_t* __restrict__ q_ptr,
               const int32_t* __restrict__ q_cols, const int32_t* __restrict__ q_order,
               int32_t nkt, uint16_t* __restrict__ dq) {
  constexpr int kDB = D / 32, kKK = D / 16;
  __shared__ __attribute__((aligned(1024))) char st0[kDqStage];
  __shared__ __attribute__((aligned(1024))) char st1[kDqStage];
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int hi = lane >> 5, col = lane & 31;
  int work, h;
  block_work(blockIdx.x, H, (nq + 127) / 128, &work, &h);
  const int qt = q_order[work];
  const int beg = q_ptr[qt];
  const int nsub = 2 * (q_ptr[qt + 1] - beg);
  const size_t rs = (size_t)H * D;
  const int hoff = h * D;

  const int qrow = qt * 128 + wv * 32 + col;
  const bool qin = qrow < nq;
  const int qc = qin ? qrow : nq - 1;
  const int qid = qin ? q_ids[qrow] : -1;
  const bool qvalid = qid >= 0;
  const float nl2 = -lse2[(size_t)h * nq + qc];  // -inf on rows without a key: P = 0
  const float dlt = delta[(size_t)h * nq + qc];

  bf16x8 qf[kKK], df[kKK];
  {
    const uint16_t* qp = q + (size_t)qc * rs + hoff + 8 * hi;
    const uint16_t* dp = dout + (size_t)qc * rs + hoff + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      qf[kk] = *(const bf16x8*)(qp + 16 * kk);
      df[kk] = *(const bf16x8*)(dp + 16 * kk);
    }
  }
  const int rb = row_base(lane), tb = tr_base(lane);
  f32x16 acc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;

  auto stage = [&](int s, char* base) {
    const int kt = q_cols[beg + (s >> 1)];
    const int k0 = kt * 128 + (s & 1) * 64;
    stage_tile<D, 64, 4>(k, rs, hoff, k0, nkv, base, wv, lane);
    stage_tile<D, 64, 4>(v, rs, hoff, k0, nkv, base + kTile64, wv, lane);
    if (wv == 0) stage_ids(kv_ids, k0, nkv, base + 2 * kTile64, lane);
  };

  if (nsub > 0) stage(0, st0);
  // Two LDS stage arrays and a loop unrolled by two: each step reads one
  // array while the next stage's direct loads fill the other, so the
  // compiler can see that its LDS reads never wait for those loads.
  auto step = [&](int s, const char* base, char* next) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (s + 1 < nsub) stage(s + 1, next);
    const int kt = q_cols[beg + (s >> 1)];
    const bool partial = tile_class_at(tile_class, (size_t)qt * nkt + kt) == 1;
    const int32_t* il = (const int32_t*)(base + 2 * kTile64);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {  // 32 keys at a time
      f32x16 st, dpt;  // S^T, dP^T: keys 32mb + 8(j/4) + 4hi + j%4 x query `col`
#pragma unroll
      for (int j = 0; j < 16; ++j) st[j] = dpt[j] = 0.f;
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) {
        const int ro = row_at(rb, kk) + 8192 * mb;
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(base, ro), qf[kk], st, 0, 0, 0);
        dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(base + kTile64, ro), df[kk], dpt,
                                                       0, 0, 0);
      }
      float p[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(st[j], s2, nl2));
      if (partial) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = mb * 32 + 8 * g + 4 * hi;
          const int4 t4 = *(const int4*)(il + r0);  // -1 past the end of the keys
          p[4 * g + 0] = (qvalid & (t4.x == qid)) ? p[4 * g + 0] : 0.f;
          p[4 * g + 1] = (qvalid & (t4.y == qid)) ? p[4 * g + 1] : 0.f;
          p[4 * g + 2] = (qvalid & (t4.z == qid)) ? p[4 * g + 2] : 0.f;
          p[4 * g + 3] = (qvalid & (t4.w == qid)) ? p[4 * g + 3] : 0.f;
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 8 * kb + 2 * e;
          w[e] = pack_bf16x2(p[j] * (dpt[j] - dlt), p[j + 1] * (dpt[j + 1] - dlt));
        }
        const bf16x8 dsb = __builtin_bit_cast(bf16x8, w);
        // dQ^T += K^T dS^T over keys 32mb + 16kb .. +15
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const int o2 = 8192 * mb + 4096 * kb;
          const bf16x8 a = join8(lds_tr4(base, tr_at(tb, db, 0) + o2), lds_tr4(base, tr_at(tb, db, 1) + o2));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb, acc[db], 0, 0, 0);
        }
      }
    }
    };
  for (int s = 0; s < nsub; s += 2) {
    step(s, st0, st1);
    if (s + 1 < nsub) step(s + 1, st1, st0);
  }
  if (qin) {
    uint16_t* op = dq + (size_t)qrow * rs + hoff;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale);
        pk[1] = pack_bf16x2(acc[db][4 * g + 2] * scale, acc[db][4 * g + 3] * scale);
        *(u32x2*)(op + db * 32 + 8 * g + 4 * hi) = pk;
      }
  }
}

// ------------------------------------------------------------------ bf16 dq, paired
// 128-wide heads: a workgroup of 8 waves per pair of query tiles (positions 2w
// and 2w + 1 of the longest-first order), one per wave group, like the
// forward's paired kernel, walking the pair's list of the block mask.  Both groups walk the same 64-key sub-tiles one
// phase apart: group A runs the MFMA phase of sub-tile s (dQ^T += K^T dS^T of
// s - 1, then S^T = K Q^T and dP^T = V dO^T of s) and then the VALU phase of
// s (P = exp2(S s2 - LSE2), dS = P (dP - Delta)); group B the VALU phase of
// s - 1 and then the MFMA phase of s; one workgroup barrier per step.  K(s) is
// read in two steps (S of s, dQ of s), so K and V each get four LDS buffers;
// sub-tiles are staged two steps ahead by the group in its VALU phase (A: K
// and ids, B: V).
constexpr int kDqSub = 64 * kRowBytes;  // one 64-key sub-tile (16 KB)

template <int D>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
dq_bf16_pair_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                    const uint16_t* __restrict__ o, const float* __restrict__ lse,
                    float* __restrict__ delta, float* __restrict__ lse2,
                    const int32_t* __restrict__ q_ids, const int32_t* __restrict__ kv_ids,
                    int32_t nq, int32_t nkv, int32_t H, float s2, float scale,
                    const int32_t* __restrict__ q_order, const int32_t* __restrict__ pair_off,
                    const int32_t* __restrict__ pair_len, const int32_t* __restrict__ pair_ent,
                    uint16_t* __restrict__ dq) {
  static_assert(D == 128, "the paired dQ kernel is laid out for 128-wide heads");
  constexpr int kDB = D / 32, kKK = D / 16;
  __shared__ __attribute__((aligned(1024))) char kb0[kDqSub + 256];
  __shared__ __attribute__((aligned(1024))) char kb1[kDqSub + 256];
  __shared__ __attribute__((aligned(1024))) char kb2[kDqSub + 256];
  __shared__ __attribute__((aligned(1024))) char kb3[kDqSub + 256];
  __shared__ __attribute__((aligned(1024))) char vb0[kDqSub];
  __shared__ __attribute__((aligned(1024))) char vb1[kDqSub];
  __shared__ __attribute__((aligned(1024))) char vb2[kDqSub];
  __shared__ __attribute__((aligned(1024))) char vb3[kDqSub];

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int hi = lane >> 5, col = lane & 31;
  const int grp = wv >> 2, wq = wv & 3;
  const int nqt = (nq + 127) / 128;
  int work, h;
  block_work(blockIdx.x, H, (nqt + 1) / 2, &work, &h);
  const int qpair[2] = {q_order[2 * work], 2 * work + 1 < nqt ? q_order[2 * work + 1] : -1};
  const int qmine = qpair[grp];  // -1: no tile (odd tile count), no rows, all masked
  // the key walk: the pair's list from the block mask (key tiles one of the two
  // query tiles has work with, ascending, both classes beside each tile)
  const int32_t* const pent = pair_ent + pair_off[work];
  const int n = 2 * pair_len[work];  // 64-key sub-steps
  const size_t rs = (size_t)H * D;
  const int hoff = h * D;

  const int qrow = qmine * 128 + wq * 32 + col;
  const bool qin = qmine >= 0 && qrow < nq;
  const int qc = qin ? qrow : nq - 1;
  const int qid = qin ? q_ids[qrow] : -1;
  const bool qvalid = qid >= 0;

  bf16x8 qf[kKK], df[kKK];
  {
    const uint16_t* qp = q + (size_t)qc * rs + hoff + 8 * hi;
    const uint16_t* dp = dout + (size_t)qc * rs + hoff + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      qf[kk] = *(const bf16x8*)(qp + 16 * kk);
      df[kk] = *(const bf16x8*)(dp + 16 * kk);
    }
  }
  // The row terms of the softmax gradient for this lane's query, from its O
  // and dO rows (the lane holds half of the row; the other half is in lane
  // l ^ 32): Delta = sum_d dO O (fp32), and the LSE in log2 units (+inf on rows
  // without an allowed key, so that exp2 gives P = 0).  Written once per query
  // for the dK/dV stage, which reads them from the workspace.
  float dlt, nl2;
  {
    const uint16_t* op = o + (size_t)qc * rs + hoff + 8 * hi;
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      const bf16x8 ov = *(const bf16x8*)(op + 16 * kk);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)df[kk][e], (float)ov[e], part);
    }
    dlt = half_sum(part);
    const float l = lse[(size_t)h * nq + qc];
    const float l2 = l == -INFINITY ? INFINITY : l * kLog2e;
    nl2 = -l2;
    if (qin && hi == 0) {
      delta[(size_t)h * nq + qrow] = dlt;
      lse2[(size_t)h * nq + qrow] = l2;
    }
  }
  const int rb = row_base(lane), tb = tr_base(lane);
  f32x16 acc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;
  f32x16 st[2], dpt[2];  // S^T, dP^T of the current sub-tile (keys 32mb + ...)
  bf16x8 dsb[4];         // dS^T of the previous one, as MFMA operands (16 keys each)

  // walk entries as scalars, as in the paired forward: e1, e2 hold the entries
  // of sub-steps s + 1 and s + 2 at step s; the entry of s + 3 is fetched in
  // the step's VALU phase and landed at its end
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

  const uint32_t group_bytes = (uint32_t)(4 * rs * 2);
  const uint32_t lane_off =
      (uint32_t)((((size_t)(lane >> 4) * rs + hoff) * 2) +
                 (((lane & 15) ^ (4 * (lane >> 4) + wq)) << 4));
  const auto rows = [&](const uint16_t* g, int row0) {
    const uint64_t bytes = row0 < nkv ? (uint64_t)(nkv - row0) * rs * 2 : 0;
    return raw_rsrc(g + (size_t)row0 * rs, bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes);
  };
  const auto load_piece = [&](int j, u32x4_t r, char* dst) __attribute__((always_inline)) {
    const int blk = wq + 4 * j;
    dma_b128(r, lane_off + blk * group_bytes, lds_address(dst + blk * 1024));
  };
  // (buffer form inside the keys; the tail sub-tile takes the per-lane form,
  // which gives keys past the end the id -1)
  const auto load_ids = [&](int k0, char* kdst) __attribute__((always_inline)) {
    // the lane index recomputed here (mbcnt) rather than kept live across the loop
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    if ((ln >> 4) == wq) {
      const int i = k0 + ln;
      if (k0 + 64 <= nkv)
        dma_b32_buf(raw_rsrc(kv_ids, (uint32_t)nkv * 4u), (uint32_t)i * 4u,
                    lds_address(kdst + kDqSub));
      else
        dma_b32(i < nkv ? kv_ids + i : &kNoId, lds_address(kdst + kDqSub));
    }
  };

  // MFMA phase: dQ^T += K^T dS^T of the previous sub-tile (K^T read transposed
  // from kprev), then S^T = K Q^T and dP^T = V dO^T of this one (kcur, vcur),
  // masked unless the tile is full for this group; MFMAs in batches of four
  // with the next batch's operand reads in flight.
  //   MFMA i <  16: dQ, kb = i / 4, db = i % 4 (A = K^T slice, B = dsb[kb])
  //   MFMA i >= 16: j = i - 16, kk = j / 4, mb = j % 2, V rows if j % 4 >= 2 (S/dP)
  // kind: 0 = S/dP only (first sub-tile), 1 = dQ only (after the last), 2 = both
  const auto mfma_phase = [&](auto kind, const char* kcur, const char* kprev, const char* vcur,
                              bool partial) __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    const auto load_op = [&](int i) __attribute__((always_inline)) {
      if (i < 16) {
        const int kb = i >> 2, db = i & 3;
        return join8(lds_tr4(kprev, tr_at(tb, db, 0) + 4096 * kb),
                     lds_tr4(kprev, tr_at(tb, db, 1) + 4096 * kb));
      }
      const int j = i - 16, kk = j >> 2, mb = j & 1;
      return lds_row8((j & 2) ? vcur : kcur, row_at(rb, kk) + 8192 * mb);
    };
    const auto do_mfma = [&](int i, bf16x8 a) __attribute__((always_inline)) {
      if (i < 16) {
        const int kb = i >> 2, db = i & 3;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[kb], acc[db], 0, 0, 0);
      } else {
        // the first contraction step starts from zero: S^T and dP^T are not
        // live before it (registers for the dQ part of the phase)
        const int j = i - 16, kk = j >> 2, mb = j & 1;
        const f32x16 zero = {};
        if (j & 2)
          dpt[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, df[kk], kk ? dpt[mb] : zero, 0, 0, 0);
        else
          st[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], kk ? st[mb] : zero, 0, 0, 0);
      }
    };
    constexpr int first_i = K == 0 ? 16 : 0, last_i = K == 1 ? 16 : 48;
    bf16x8 op[2][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) op[0][e] = load_op(first_i + e);
    if (first_i < 16)
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    else
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int b = first_i; b < last_i; b += 4) {
      const int cur = ((b - first_i) >> 2) & 1;
      do_mfma(b, op[cur][0]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (b + 4 < last_i) {
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
      const int32_t* il = (const int32_t*)(kcur + kDqSub);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int4 t4 = *(const int4*)(il + mb * 32 + 8 * g + 4 * hi);  // -1 past the end
          st[mb][4 * g + 0] = (qvalid & (t4.x == qid)) ? st[mb][4 * g + 0] : -INFINITY;
          st[mb][4 * g + 1] = (qvalid & (t4.y == qid)) ? st[mb][4 * g + 1] : -INFINITY;
          st[mb][4 * g + 2] = (qvalid & (t4.z == qid)) ? st[mb][4 * g + 2] : -INFINITY;
          st[mb][4 * g + 3] = (qvalid & (t4.w == qid)) ? st[mb][4 * g + 3] : -INFINITY;
        }
    }
  };

  // VALU phase: P = exp2(S s2 - LSE2) (0 on masked scores), dS = P (dP - Delta)
  const auto valu_phase = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int mb = kb >> 1, b0 = (kb & 1) * 8;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = b0 + 2 * e;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(st[mb][j], s2, nl2));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(st[mb][j + 1], s2, nl2));
        w[e] = pack_bf16x2(p0 * (dpt[mb][j] - dlt), p1 * (dpt[mb][j + 1] - dlt));
      }
      dsb[kb] = __builtin_bit_cast(bf16x8, w);
    }
    // the results exist here: keeps the compiler from sinking this phase past
    // its end, into the MFMA phase that uses it
    asm volatile("" ::"v"(dsb[0]), "v"(dsb[1]), "v"(dsb[2]), "v"(dsb[3]));
  };

  // The barrier that ends a step also sets the issue priority for the phase it
  // opens (as does the fence at mid-step): the wave in its MFMA phase gets the
  // higher one (by default the older wave of a SIMD wins every arbitration,
  // stretching the other wave's phases of both kinds).
  const auto barrier_mfma = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_setprio(2);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  const auto barrier_valu = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_setprio(0);
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
  // Loads of step s: K(s + 2) and its ids (group A, 5 per wave), V(s + 2)
  // (group B, 4 per wave), issued at the start of the group's VALU phase and
  // waited for at the end of step s + 1 (loads finish in order).
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
  const auto step_a = [&](int s, auto kind, const char* kcur, const char* kprev,
                          const char* vcur, char* kload) __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    mfma_phase(kind, kcur, kprev, vcur, partial_c);
    fence();
    __builtin_amdgcn_s_setprio(0);
    if (K != 1) {
      const int k0n = k0_of(e2, s + 2);
      const auto rk = rows(k, k0n);
      load_ids(k0n, kload);
#pragma unroll
      for (int j = 0; j < 4; ++j) load_piece(j, rk, kload);
    }
    fetch_next(s);
    if (K != 1) valu_phase();
    land_next();
    partial_c = partial_n;
    wait_prev_a(kind);
    barrier_mfma();
  };
  const auto step_b = [&](int s, auto kind, const char* kcur, const char* kprev,
                          const char* vcur, char* vload) __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    if (K != 1) {
      const auto rv = rows(v, k0_of(e2, s + 2));
#pragma unroll
      for (int j = 0; j < 4; ++j) load_piece(j, rv, vload);
    }
    fetch_next(s);
    if (K != 0) valu_phase();
    land_next();
    fence();
    __builtin_amdgcn_s_setprio(2);
    mfma_phase(kind, kcur, kprev, vcur, partial_c);
    partial_c = partial_n;
    wait_prev_b(kind);
    barrier_valu();
  };
  using First = std::integral_constant<int, 0>;
  using Last = std::integral_constant<int, 1>;
  using Mid = std::integral_constant<int, 2>;
  // prologue: K(0), K(1) (group A), V(0), V(1) (group B)
  if (n > 0) {
    const int k00 = k0_of(ent(0), 0), k01 = k0_of(e1, 1);
    if (grp == 0) {
      const auto r0 = rows(k, k00), r1 = rows(k, k01);
      load_ids(k00, kb0);
      load_ids(k01, kb1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        load_piece(j, r0, kb0);
        load_piece(j, r1, kb1);
      }
    } else {
      const auto r0 = rows(v, k00), r1 = rows(v, k01);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        load_piece(j, r0, vb0);
        load_piece(j, r1, vb1);
      }
    }
  }
  wait_vmem();
  __syncthreads();
  if (grp == 0) __builtin_amdgcn_s_setprio(2);  // group A opens with its MFMA phase
  if (n > 0) {
    // step s (r = s % 4): kcur kb[r], kprev kb[(r + 3) % 4], vcur vb[r],
    // loads into kb[(r + 2) % 4] / vb[(r + 2) % 4]
    const int rl = (n - 1) & 3;
    const char* const klast = rl == 0 ? kb0 : rl == 1 ? kb1 : rl == 2 ? kb2 : kb3;
    if (grp == 0) {
      step_a(0, First{}, kb0, kb3, vb0, kb2);
      for (int s = 1; s < n; s += 4) {
        step_a(s, Mid{}, kb1, kb0, vb1, kb3);
        if (s + 1 < n) step_a(s + 1, Mid{}, kb2, kb1, vb2, kb0);
        if (s + 2 < n) step_a(s + 2, Mid{}, kb3, kb2, vb3, kb1);
        if (s + 3 < n) step_a(s + 3, Mid{}, kb0, kb3, vb0, kb2);
      }
      step_a(n, Last{}, kb0, klast, vb0, kb2);
    } else {
      step_b(0, First{}, kb0, kb3, vb0, vb2);
      for (int s = 1; s < n; s += 4) {
        step_b(s, Mid{}, kb1, kb0, vb1, vb3);
        if (s + 1 < n) step_b(s + 1, Mid{}, kb2, kb1, vb2, vb0);
        if (s + 2 < n) step_b(s + 2, Mid{}, kb3, kb2, vb3, vb1);
        if (s + 3 < n) step_b(s + 3, Mid{}, kb0, kb3, vb0, vb2);
      }
      step_b(n, Last{}, kb0, klast, vb0, vb2);
    }
  }
  if (qin) {
    uint16_t* op = dq + (size_t)qrow * rs + hoff;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale);
        pk[1] = pack_bf16x2(acc[db][4 * g + 2] * scale, acc[db][4 * g + 3] * scale);
        *(u32x2*)(op + db * 32 + 8 * g + 4 * hi) = pk;
      }
  }
}

// ------------------------------------------------------------------ bf16 dk, dv
constexpr int kKvStage = 2 * kTile64 + 3 * 256;  // Q tile, dO tile, ids, lse2, delta

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
dkdv_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                 const float* __restrict__ delta, const float* __restrict__ lse2,
                 const int32_t* __restrict__ q_ids, const int32_t* __restrict__ kv_ids,
                 int32_t nq, int32_t nkv, int32_t H, float s2, float scale,
                 const uint8_t* __restrict__ tile_class, const int32_t* __restrict__ kv_ptr,
                 const int32_t* __restrict__ kv_rows, const int32_t* __restrict__ kv_order,
                 int32_t nkt, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  constexpr int kDB = D / 32, kKK = D / 16;
  __shared__ __attribute__((aligned(1024))) char st0[kKvStage];
  __shared__ __attribute__((aligned(1024))) char st1[kKvStage];
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int hi = lane >> 5, col = lane & 31;
  int work, h;
  block_work(blockIdx.x, H, nkt, &work, &h);
  const int kt = kv_order[work];
  const int beg = kv_ptr[kt];
  const int nsub = 2 * (kv_ptr[kt + 1] - beg);
  const size_t rs = (size_t)H * D;
  const int hoff = h * D;

  const int krow = kt * 128 + wv * 32 + col;
  const bool kin = krow < nkv;
  const int kc = kin ? krow : nkv - 1;
  const int kid = kin ? kv_ids[krow] : -1;
  const bool kvalid = kid >= 0;

  bf16x8 kf[kKK], vf[kKK];
  {
    const uint16_t* kp = k + (size_t)kc * rs + hoff + 8 * hi;
    const uint16_t* vp = v + (size_t)kc * rs + hoff + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      kf[kk] = *(const bf16x8*)(kp + 16 * kk);
      vf[kk] = *(const bf16x8*)(vp + 16 * kk);
    }
  }
  const int rb = row_base(lane), tb = tr_base(lane);
  f32x16 dka[kDB], dva[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) dka[db][j] = dva[db][j] = 0.f;

  auto stage = [&](int s, char* base) {
    const int qt = kv_rows[beg + (s >> 1)];
    const int q0 = qt * 128 + (s & 1) * 64;
    stage_tile<D, 64, 4>(q, rs, hoff, q0, nq, base, wv, lane);
    stage_tile<D, 64, 4>(dout, rs, hoff, q0, nq, base + kTile64, wv, lane);
    if (wv == 1) stage_ids(q_ids, q0, nq, base + 2 * kTile64, lane);
    if (wv == 2) stage_words(lse2 + (size_t)h * nq, q0, nq, base + 2 * kTile64 + 256, lane);
    if (wv == 3) stage_words(delta + (size_t)h * nq, q0, nq, base + 2 * kTile64 + 512, lane);
  };

  if (nsub > 0) stage(0, st0);
  // Two LDS stage arrays and a loop unrolled by two: each step reads one
  // array while the next stage's direct loads fill the other, so the
  // compiler can see that its LDS reads never wait for those loads.
  auto step = [&](int s, const char* base, char* next) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (s + 1 < nsub) stage(s + 1, next);
    const int qt = kv_rows[beg + (s >> 1)];
    const bool partial = tile_class_at(tile_class, (size_t)qt * nkt + kt) == 1;
    const int32_t* qi = (const int32_t*)(base + 2 * kTile64);
    const float* l2 = (const float*)(base + 2 * kTile64 + 256);
    const float* dl = (const float*)(base + 2 * kTile64 + 512);
    int rbi = rb, tbi = tb;
    asm volatile("" : "+v"(rbi), "+v"(tbi));  // recompute operand offsets here, not hoisted
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {  // 32 queries at a time
      // S, then P packed to bf16 at once (frees S); then dP and dS from the bf16 P
      f32x16 acc;  // queries 32mb + 8(j/4) + 4hi + j%4 x key `col`
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(base, row_at(rbi, kk) + 8192 * mb),
                                                      kf[kk], acc, 0, 0, 0);
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = mb * 32 + 8 * g + 4 * hi;
        const f32x4 l4 = *(const f32x4*)(l2 + r0);
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(acc[4 * g + e], s2, -l4[e]));
        if (partial) {
          const int4 t4 = *(const int4*)(qi + r0);  // -1 past the end of the queries
          p[0] = (kvalid & (t4.x == kid)) ? p[0] : 0.f;
          p[1] = (kvalid & (t4.y == kid)) ? p[1] : 0.f;
          p[2] = (kvalid & (t4.z == kid)) ? p[2] : 0.f;
          p[3] = (kvalid & (t4.w == kid)) ? p[3] : 0.f;
        }
        u32x4 wp = __builtin_bit_cast(u32x4, pb[g >> 1]);
        const int w0 = (g & 1) * 2;
        wp[w0] = pack_bf16x2(p[0], p[1]);
        wp[w0 + 1] = pack_bf16x2(p[2], p[3]);
        pb[g >> 1] = __builtin_bit_cast(bf16x8, wp);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            lds_row8(base + kTile64, row_at(rbi, kk) + 8192 * mb), vf[kk], acc, 0, 0, 0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = mb * 32 + 8 * g + 4 * hi;
        const f32x4 d4 = *(const f32x4*)(dl + r0);
        const u32x4 wp = __builtin_bit_cast(u32x4, pb[g >> 1]);
        const int w0 = (g & 1) * 2;
        const float p0 = bf16_bits_to_f32(wp[w0] & 0xFFFFu), p1 = bf16_bits_to_f32(wp[w0] >> 16);
        const float p2 = bf16_bits_to_f32(wp[w0 + 1] & 0xFFFFu), p3 = bf16_bits_to_f32(wp[w0 + 1] >> 16);
        u32x4 wd = __builtin_bit_cast(u32x4, dsb[g >> 1]);
        wd[w0] = pack_bf16x2(p0 * (acc[4 * g] - d4[0]), p1 * (acc[4 * g + 1] - d4[1]));
        wd[w0 + 1] = pack_bf16x2(p2 * (acc[4 * g + 2] - d4[2]), p3 * (acc[4 * g + 3] - d4[3]));
        dsb[g >> 1] = __builtin_bit_cast(bf16x8, wd);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over queries 32mb + 16kb .. +15
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int o2 = 8192 * mb + 4096 * kb;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const bf16x8 ao = join8(lds_tr4(base + kTile64, tr_at(tbi, db, 0) + o2),
                                  lds_tr4(base + kTile64, tr_at(tbi, db, 1) + o2));
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, pb[kb], dva[db], 0, 0, 0);
          const bf16x8 aq = join8(lds_tr4(base, tr_at(tbi, db, 0) + o2),
                                  lds_tr4(base, tr_at(tbi, db, 1) + o2));
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, dsb[kb], dka[db], 0, 0, 0);
        }
      }
    }
    };
  for (int s = 0; s < nsub; s += 2) {
    step(s, st0, st1);
    if (s + 1 < nsub) step(s + 1, st1, st0);
  }
  if (kin) {
    uint16_t* kp = dk + (size_t)krow * rs + hoff;
    uint16_t* vp = dv + (size_t)krow * rs + hoff;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 a, b;
        a[0] = pack_bf16x2(dka[db][4 * g] * scale, dka[db][4 * g + 1] * scale);
        a[1] = pack_bf16x2(dka[db][4 * g + 2] * scale, dka[db][4 * g + 3] * scale);
        b[0] = pack_bf16x2(dva[db][4 * g], dva[db][4 * g + 1]);
        b[1] = pack_bf16x2(dva[db][4 * g + 2], dva[db][4 * g + 3]);
        *(u32x2*)(kp + db * 32 + 8 * g + 4 * hi) = a;
        *(u32x2*)(vp + db * 32 + 8 * g + 4 * hi) = b;
      }
  }
}

// ------------------------------------------------------------------ bf16 dk, dv, split waves
// 128-wide heads: a workgroup of 8 waves per 128-key tile; waves w and w + 4
// (one SIMD) share keys 32w .. 32w + 31 and split the work: the P wave holds K
// and the dV accumulator (S = Q K^T, P = exp2(S s2 - LSE2), dV^T += dO^T P),
// the D wave holds V and the dK accumulator (dP = dO V^T, dS = P (dP - Delta),
// dK^T += Q^T dS), with P handed over through LDS.  Each wave thus carries
// half of the one-wave kernel's registers (room to keep its operand reads
// ahead of its MFMAs), and the two alternate one phase apart per 64-query
// sub-step s:
//   first half:  P wave MFMAs (dV of s - 1, S of s); D wave VALU (dS of s - 1)
//   second half: P wave VALU (P of s, into LDS);     D wave MFMAs (dK of s - 1, dP of s)
// so each SIMD holds one MFMA wave and one VALU wave at a time.  Only the end
// of a step is a workgroup barrier; the hand-over of P is guarded pairwise (see
// wait_xch / post_xch).  Sub-tile s (Q, dO, ids, LSE2, Delta) is read from the
// first half of step s to the second half of step s + 1: four LDS stages,
// staged two steps ahead by direct loads from inline assembly.  The
// 32 row groups of a sub-tile are spread over all eight waves, and each wave
// issues its loads one at a time between MFMAs or VALU work: a burst of direct
// loads at a phase start stalls the issuing waves for hundreds of cycles.  A
// wave's VALU phase also reads the first two operand batches of its next MFMA
// phase, so that phase starts on MFMAs, not on LDS latency.
constexpr int kSpSub = 64 * kRowBytes;                // one 64-query tile (16 KB)
constexpr int kSpStage = 2 * kSpSub + 3 * 256;        // Q, dO, ids, LSE2, Delta
constexpr int kSpIds = 2 * kSpSub, kSpLse = kSpIds + 256, kSpDelta = kSpLse + 256;

// Number of dK/dV waves whose hand-over wait ran out (their dv rows are NaN),
// since the library was loaded or the count was last reset; one per device.
// Incremented with a vector atomic by lane 0 of such a wave.
__device__ int32_t g_handover_failures = 0;

template <int D>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
dkdv_bf16_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                       const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                       const float* __restrict__ delta, const float* __restrict__ lse2,
                       const int32_t* __restrict__ q_ids, const int32_t* __restrict__ kv_ids,
                       int32_t nq, int32_t nkv, int32_t H, float s2, float scale,
                       const uint8_t* __restrict__ tile_class,
                       const int32_t* __restrict__ kv_ptr, const int32_t* __restrict__ kv_rows,
                       const int32_t* __restrict__ kv_order, int32_t nkt,
                       uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int32_t spin_limit) {
  static_assert(D == 128, "the split dK/dV kernel is laid out for 128-wide heads");
  constexpr int kDB = D / 32, kKK = D / 16;
  __shared__ __attribute__((aligned(1024))) char st0[kSpStage];
  __shared__ __attribute__((aligned(1024))) char st1[kSpStage];
  __shared__ __attribute__((aligned(1024))) char st2[kSpStage];
  __shared__ __attribute__((aligned(1024))) char st3[kSpStage];
  __shared__ __attribute__((aligned(1024))) char xch[4 * 4096];  // P, per key block
  __shared__ int xdone[4];  // per wave pair: last step whose P the D wave has read

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int hi = lane >> 5, col = lane & 31;
  const int grp = wv >> 2, wq = wv & 3;  // grp 0: P wave, 1: D wave
  int work, h;
  block_work(blockIdx.x, H, nkt, &work, &h);
  const int kt = kv_order[work];
  const int beg = kv_ptr[kt];
  const int n = 2 * (kv_ptr[kt + 1] - beg);  // 64-query sub-steps
  const size_t rs = (size_t)H * D;
  const int hoff = h * D;

  const int krow = kt * 128 + wq * 32 + col;
  const bool kin = krow < nkv;
  const int kc = kin ? krow : nkv - 1;
  const int kid = kin ? kv_ids[krow] : -1;
  const bool kvalid = kid >= 0;

  bf16x8 kvf[kKK];  // K rows (P wave) or V rows (D wave) of this lane's key
  {
    const uint16_t* src = (grp == 0 ? k : v) + (size_t)kc * rs + hoff + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) kvf[kk] = *(const bf16x8*)(src + 16 * kk);
  }
  const int rb = row_base(lane), tb = tr_base(lane);
  f32x16 gacc[kDB];  // dV^T (P wave) or dK^T (D wave)
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) gacc[db][j] = 0.f;
  f32x16 sc[2];  // S (P wave) or dP (D wave) of the current sub-tile
  bf16x8 ob[4];  // P (P wave) or dS (D wave) as MFMA operands, 16 queries each
  char* const xb = xch + wq * 4096;

  // Per-step scalars, fetched a step ahead in a VALU phase (an outstanding
  // scalar load would force every LDS operand wait of an MFMA phase to zero):
  // at step s, qt_l is the query tile of sub-step s + 2 (the one this step
  // loads) and qt_p that of s + 1; the step issues the loads of the query tile
  // of s + 3 and of the class word of (qt_p, kt) -- independent of each other,
  // both landed at the end of the VALU phase.
  const auto last_sub = [&](int s) { return s < n ? s : n - 1; };
  const auto qt_of = [&](int s) { return kv_rows[beg + (last_sub(s) >> 1)]; };
  const auto q0_of = [&](int s, int qt) { return qt * 128 + 64 * (last_sub(s) & 1); };
  int qt_l = n > 0 ? qt_of(2) : 0, qt_p = n > 0 ? qt_of(1) : 0;
  bool partial_c = n > 0 && tile_class_at(tile_class, (size_t)qt_of(0) * nkt + kt) != 2;
  int qt_nl = 0, partial_n = 0, cword = 0, csh = 0, s_next = 0;
  const auto fetch_next = [&](int s) __attribute__((always_inline)) {
    qt_nl = sload_issue(kv_rows + beg + (last_sub(s + 3) >> 1));
    const size_t idx = (size_t)qt_p * nkt + kt;
    cword = sload_issue((const int32_t*)tile_class + (idx >> 2));
    csh = 8 * (int)(idx & 3);
    s_next = s + 1;
  };
  const auto land_next = [&]() __attribute__((always_inline)) {
    sload_wait2(qt_nl, cword);
    partial_n = s_next < n ? (((cword >> csh) & 0xFF) != 2) : 0;
    asm volatile("" ::"s"(qt_nl), "s"(partial_n));
  };
  const auto rotate = [&]() __attribute__((always_inline)) {
    qt_p = qt_l;
    qt_l = qt_nl;
    partial_c = partial_n;
  };

  // direct loads: 16 row groups of a 64-row tile over a group's four waves
  const uint32_t group_bytes = (uint32_t)(4 * rs * 2);
  const uint32_t lane_off =
      (uint32_t)((((size_t)(lane >> 4) * rs + hoff) * 2) +
                 (((lane & 15) ^ (4 * (lane >> 4) + wq)) << 4));
  const auto rows = [&](const uint16_t* g, int row0) {
    const uint64_t bytes = row0 < nq ? (uint64_t)(nq - row0) * rs * 2 : 0;
    return raw_rsrc(g + (size_t)row0 * rs, bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes);
  };
  // every wave stages 4 of a sub-tile's 32 row groups (2 of Q, 2 of dO): row
  // groups wq + 4 (2 grp + j) of each, piece j in the step's phase j, so the
  // direct loads of a step spread over all eight waves and both phases
  // rsrc[t]: descriptor over the rows of Q (t = 0) or dO (t = 1) from the step's
  // first query on, built once per step (rebuilding it for every load cost 4 %)
  const auto load_one = [&](const u32x4_t* rsrc, int t, int j, char* stage)
                            __attribute__((always_inline)) {
    const int blk = wq + 4 * (2 * grp + j);
    dma_b128(rsrc[t], lane_off + blk * group_bytes, lds_address(stage + t * kSpSub + blk * 1024));
  };
  const auto step_rsrc = [&](int q0, u32x4_t* rsrc) __attribute__((always_inline)) {
    rsrc[0] = rows(q, q0);
    rsrc[1] = rows(dout, q0);
    asm volatile("" ::"s"(rsrc[0]), "s"(rsrc[1]));
  };
  const auto load_piece = [&](int j, int q0, char* stage) __attribute__((always_inline)) {
    u32x4_t r[2];
    step_rsrc(q0, r);
    load_one(r, 0, j, stage);
    load_one(r, 1, j, stage);
  };
  // D wave wq stages the ids (0), LSE2 (1) or Delta (2, and again 3) of 64 queries
  // (so each D wave issues 5 loads per step, each P wave 4): the buffer form
  // inside the queries, the per-lane form for the tail sub-tile (ids -1 past
  // the end)
  const auto load_words = [&](int q0, char* stage) __attribute__((always_inline)) {
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int i = q0 + ln;
    const uint32_t dst = lds_address(stage + (wq == 0 ? kSpIds : wq == 1 ? kSpLse : kSpDelta));
    if (q0 + 64 <= nq) {
      const void* base = wq == 0 ? (const void*)q_ids : (const void*)((wq == 1 ? lse2 : delta) + (size_t)h * nq);
      dma_b32_buf(raw_rsrc(base, (uint32_t)nq * 4u), (uint32_t)i * 4u, dst);
    } else {
      const void* src;
      if (wq == 0)
        src = i < nq ? q_ids + i : &kNoId;
      else
        src = (wq == 1 ? lse2 : delta) + (size_t)h * nq + min(i, nq - 1);
      dma_b32(src, dst);
    }
  };

  // MFMA phase: gacc += tsrc^T ob over the previous sub-tile (dV^T += dO^T P or
  // dK^T += Q^T dS; tsrc read transposed), then sc = rsrc K^T / rsrc V^T over
  // this one (rsrc = Q or dO rows), in batches of four MFMAs with the next
  // batch's operand reads in flight.
  //   MFMA i <  16: kb = i / 4, db = i % 4 (A = tsrc^T slice, B = ob[kb])
  //   MFMA i >= 16: j = i - 16, kk = j / 2, mb = j % 2 (A = rsrc rows, B = kvf[kk])
  // kind: 0 = rows part only (first sub-tile), 1 = transposed part only, 2 = both
  const auto load_op = [&](int i, const char* tsrc, const char* rsrc) __attribute__((always_inline)) {
    if (i < 16) {
      const int kb = i >> 2, db = i & 3;
      return join8(lds_tr4(tsrc, tr_at(tb, db, 0) + 4096 * kb),
                   lds_tr4(tsrc, tr_at(tb, db, 1) + 4096 * kb));
    }
    const int j = i - 16, kk = j >> 1, mb = j & 1;
    return lds_row8(rsrc, row_at(rb, kk) + 8192 * mb);
  };
  bf16x8 op[3][4];  // operand ring: two batches of reads in flight
  // the first two batches of an MFMA phase, read during the wave's VALU phase
  const auto prefetch = [&](auto kind, const char* tsrc, const char* rsrc)
                            __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    constexpr int first_i = K == 0 ? 16 : 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) op[e >> 2][e & 3] = load_op(first_i + e, tsrc, rsrc);
  };
  // hook(i) runs after the reads issued with batch i (a place for a direct load:
  // issued between MFMAs, a wave's loads never queue up behind a burst)
  const auto mfma_phase = [&](auto kind, const char* tsrc, const char* rsrc, auto hook)
                              __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    const auto do_mfma = [&](int i, bf16x8 a) __attribute__((always_inline)) {
      if (i < 16) {
        const int kb = i >> 2, db = i & 3;
        gacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ob[kb], gacc[db], 0, 0, 0);
      } else {
        const int j = i - 16, kk = j >> 1, mb = j & 1;
        const f32x16 zero = {};
        sc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kvf[kk], kk ? sc[mb] : zero, 0, 0, 0);
      }
    };
    constexpr int first_i = K == 0 ? 16 : 0, last_i = K == 1 ? 16 : 32;
#pragma unroll
    for (int b = first_i; b < last_i; b += 4) {
      const int cur = ((b - first_i) >> 2) % 3;
      do_mfma(b, op[cur][0]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (b + 8 < last_i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) op[(cur + 2) % 3][e] = load_op(b + 8 + e, tsrc, rsrc);
        if (b + 8 < 16)
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
      hook((b - first_i) >> 2);
#pragma unroll
      for (int e = 1; e < 4; ++e) do_mfma(b + e, op[cur][e]);
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    }
  };

  // The per-query words a VALU phase needs (LSE2 for P, Delta for dS) are read
  // into registers at the end of the wave's MFMA phase, and the mask is applied
  // to S there: with the other wave's operand reads in the LDS queue, every
  // LDS read left in a VALU phase costs its full latency.
  f32x4 qw[8];  // LSE2 (P wave) or Delta (D wave) of queries 32mb + 8g + 4hi .. +3
  const auto read_words = [&](const char* stage, int off) __attribute__((always_inline)) {
    const float* w = (const float*)(stage + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) qw[i] = *(const f32x4*)(w + (i >> 2) * 32 + 8 * (i & 3) + 4 * hi);
  };
  const auto mask_scores = [&](const char* stage) __attribute__((always_inline)) {
    const int32_t* qi = (const int32_t*)(stage + kSpIds);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int4 t4 = *(const int4*)(qi + mb * 32 + 8 * g + 4 * hi);  // -1 past the end
        sc[mb][4 * g + 0] = (kvalid & (t4.x == kid)) ? sc[mb][4 * g + 0] : -INFINITY;
        sc[mb][4 * g + 1] = (kvalid & (t4.y == kid)) ? sc[mb][4 * g + 1] : -INFINITY;
        sc[mb][4 * g + 2] = (kvalid & (t4.z == kid)) ? sc[mb][4 * g + 2] : -INFINITY;
        sc[mb][4 * g + 3] = (kvalid & (t4.w == kid)) ? sc[mb][4 * g + 3] : -INFINITY;
      }
  };
  // The two waves of a pair meet once per step (the barrier that ends it), so
  // the P wave must not overwrite the hand-over buffer with P of step s before
  // its D wave has read P of step s - 1 there: the D wave posts each step it
  // has read (release), the P wave waits for it (acquire) before writing --
  // normally long done.  The wait is bounded (spin_limit polls), so it ends on
  // every path; a wait that runs out marks the wave, which then writes NaN
  // instead of its dV rows, so a broken hand-over cannot pass unnoticed.
  int xstep = 0;  // the step whose P this wave writes / reads next
  bool xfail = false;
  const auto wait_xch = [&]() __attribute__((always_inline)) {
    if (xstep > 0) {
      int tries = 0;
      for (; tries < spin_limit; ++tries) {
        const int done = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(&xdone[wq], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (done >= xstep) break;
        __builtin_amdgcn_s_sleep(1);
      }
      xfail |= tries >= spin_limit;
    }
  };
  const auto post_xch = [&]() __attribute__((always_inline)) {
    if (lane == 0) __hip_atomic_store(&xdone[wq], xstep, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  // P wave VALU phase: P = exp2(S s2 - LSE2) (0 on masked scores), packed to
  // bf16 (queries 32mb + 8(j/4) + 4hi + j%4 of the lane's key), handed over
  const auto p_phase = [&](auto mid) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (mb == 1) mid();
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = qw[4 * mb + g];
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sc[mb][4 * g + e], s2, -l4[e]));
        const int kb = 2 * mb + (g >> 1), w0 = (g & 1) * 2;
        u32x4 wp = __builtin_bit_cast(u32x4, ob[kb]);
        wp[w0] = pack_bf16x2(p[0], p[1]);
        wp[w0 + 1] = pack_bf16x2(p[2], p[3]);
        ob[kb] = __builtin_bit_cast(bf16x8, wp);
      }
    }
    wait_xch();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) *(bf16x8*)(xb + kb * 1024 + lane * 16) = ob[kb];
    // The D wave reads this P right after the barrier that ends the step, and
    // s_barrier does not wait for a wave's outstanding LDS writes: wait for
    // them here (LDS counter only, so the step's direct loads stay in flight).
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  // D wave VALU phase: dS = P (dP - Delta) from the handed-over P (same lanes)
  const auto ds_phase = [&](auto mid) __attribute__((always_inline)) {
    u32x4 wps[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) wps[kb] = *(const u32x4*)(xb + kb * 1024 + lane * 16);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb == 2) mid();
      const u32x4 wp = wps[kb];
      const int mb = kb >> 1;
      u32x4 wd;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int g = 2 * (kb & 1) + h2;
        const f32x4 d4 = qw[4 * mb + g];
        const int w0 = 2 * h2;
        const float p0 = bf16_bits_to_f32(wp[w0] & 0xFFFFu), p1 = bf16_bits_to_f32(wp[w0] >> 16);
        const float p2 = bf16_bits_to_f32(wp[w0 + 1] & 0xFFFFu), p3 = bf16_bits_to_f32(wp[w0 + 1] >> 16);
        wd[w0] = pack_bf16x2(p0 * (sc[mb][4 * g] - d4[0]), p1 * (sc[mb][4 * g + 1] - d4[1]));
        wd[w0 + 1] = pack_bf16x2(p2 * (sc[mb][4 * g + 2] - d4[2]), p3 * (sc[mb][4 * g + 3] - d4[3]));
      }
      ob[kb] = __builtin_bit_cast(bf16x8, wd);
    }
  };
  const auto pin_ob = [&]() __attribute__((always_inline)) {
    asm volatile("" ::"v"(ob[0]), "v"(ob[1]), "v"(ob[2]), "v"(ob[3]));
  };

  const auto fence = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // The barrier that ends a step also sets the issue priority for the phase it
  // opens (as does the fence at mid-step): the wave in its MFMA phase gets the
  // higher one (by default the older wave of a SIMD wins every arbitration,
  // stretching the other wave's phases of both kinds).
  const auto barrier_mfma = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_setprio(2);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  const auto barrier_valu = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_setprio(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  using First = std::integral_constant<int, 0>;
  using Last = std::integral_constant<int, 1>;
  using Mid = std::integral_constant<int, 2>;
  // step s: cur = stage of s, prev = stage of s - 1, ld = stage of s + 2
  // (sub-tile s + 2 is staged during step s; each wave waits for its loads of
  // step s at the end of step s + 1: they finish in order)
  const auto step_p = [&](int s, auto kind, const char* cur, const char* prev, char* ld)
                          __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    xstep = s;
    const int q0 = q0_of(s + 2, qt_l);
    u32x4_t rs2[2];
    if (K != 1) step_rsrc(q0, rs2);
    constexpr int nbat = K == 2 ? 8 : 4;
    // dV (dO^T of s - 1), S (Q of s); piece 0 of s + 2 issued between MFMAs
    mfma_phase(kind, prev + kSpSub, cur, [&](int i) __attribute__((always_inline)) {
      if (K != 1 && i == 1) load_one(rs2, 0, 0, ld);
      if (K != 1 && i == nbat - 2) load_one(rs2, 1, 0, ld);
    });
    if (K != 1) {
      read_words(cur, kSpLse);
      if (partial_c) mask_scores(cur);
    }
    fence();
    __builtin_amdgcn_s_setprio(0);
    if (K != 1) prefetch(Mid{}, cur + kSpSub, cur);  // dV of s in step s + 1 (rows not yet used)
    if (K != 1) load_one(rs2, 0, 1, ld);
    fetch_next(s);
    if (K != 1) p_phase([&]() __attribute__((always_inline)) { load_one(rs2, 1, 1, ld); });
    pin_ob();
    land_next();
    rotate();
    if (K == 1)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4): this step's loads may stay
    barrier_mfma();
  };
  const auto step_d = [&](int s, auto kind, const char* cur, const char* prev, char* ld)
                          __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    xstep = s;
    const int q0 = q0_of(s + 2, qt_l);
    u32x4_t rs2[2];
    if (K != 1) step_rsrc(q0, rs2);
    constexpr int nbat = K == 2 ? 8 : 4;
    if (K != 1) load_one(rs2, 0, 0, ld);
    if (K != 0) {
      ds_phase([&]() __attribute__((always_inline)) {
        if (K != 1) load_one(rs2, 1, 0, ld);
      });
      pin_ob();    // dS done (and its waits for the P reads) before what follows
      post_xch();  // P of step s - 1 read: the P wave may write that of step s
    } else {
      load_one(rs2, 1, 0, ld);
    }
    // after the hand-over's LDS accesses, whose waits would otherwise also
    // wait for these scalar loads
    fetch_next(s);
    if (K != 1) load_words(q0, ld);
    prefetch(kind, prev, cur + kSpSub);
    pin_ob();
    fence();
    __builtin_amdgcn_s_setprio(2);
    // dK (Q^T of s - 1), dP (dO of s); piece 1 of s + 2 issued between MFMAs
    mfma_phase(kind, prev, cur + kSpSub, [&](int i) __attribute__((always_inline)) {
      if (K != 1 && i == 1) load_one(rs2, 0, 1, ld);
      if (K != 1 && i == nbat - 2) load_one(rs2, 1, 1, ld);
    });
    if (K != 1) read_words(cur, kSpDelta);  // Delta of s, for dS in the next step
    // the scalars land here, after the MFMA phase: their wait (lgkmcnt(0))
    // placed before it would also drain the prefetched operand reads
    land_next();
    rotate();
    if (K == 1)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x0F75);  // vmcnt(5)
    barrier_valu();
  };
  if (tid < 4) xdone[tid] = 0;
  // prologue: sub-tiles 0 and 1 into stages 0 and 1
  if (n > 0) {
    const int qa = qt_of(0), qb = qt_of(1);
    const int q00 = q0_of(0, qa), q01 = q0_of(1, qb);
    load_piece(0, q00, st0);
    load_piece(1, q00, st0);
    load_piece(0, q01, st1);
    load_piece(1, q01, st1);
    if (grp == 1) {
      load_words(q00, st0);
      load_words(q01, st1);
    }
  }
  wait_vmem();
  __syncthreads();
  if (grp == 0) __builtin_amdgcn_s_setprio(2);  // the P wave opens with its MFMA phase
  if (n > 0) {
    // step s (r = s % 4): cur st[r], prev st[(r + 3) % 4], loads into st[(r + 2) % 4]
    const int rl = (n - 1) & 3;
    char* const slast = rl == 0 ? st0 : rl == 1 ? st1 : rl == 2 ? st2 : st3;
    if (grp == 0) {
      prefetch(First{}, st3, st0);
      step_p(0, First{}, st0, st3, st2);
      for (int s = 1; s < n; s += 4) {
        step_p(s, Mid{}, st1, st0, st3);
        if (s + 1 < n) step_p(s + 1, Mid{}, st2, st1, st0);
        if (s + 2 < n) step_p(s + 2, Mid{}, st3, st2, st1);
        if (s + 3 < n) step_p(s + 3, Mid{}, st0, st3, st2);
      }
      step_p(n, Last{}, st0, slast, st2);
    } else {
      step_d(0, First{}, st0, st3, st2);
      for (int s = 1; s < n; s += 4) {
        step_d(s, Mid{}, st1, st0, st3);
        if (s + 1 < n) step_d(s + 1, Mid{}, st2, st1, st0);
        if (s + 2 < n) step_d(s + 2, Mid{}, st3, st2, st1);
        if (s + 3 < n) step_d(s + 3, Mid{}, st0, st3, st2);
      }
      step_d(n, Last{}, st0, slast, st2);
    }
  }
  if (xfail && lane == 0)
    __hip_atomic_fetch_add(&g_handover_failures, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (kin) {
    uint16_t* gp = (grp == 0 ? dv : dk) + (size_t)krow * rs + hoff;
    const float f = grp == 0 ? 1.f : scale;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 a;
        a[0] = pack_bf16x2(gacc[db][4 * g] * f, gacc[db][4 * g + 1] * f);
        a[1] = pack_bf16x2(gacc[db][4 * g + 2] * f, gacc[db][4 * g + 3] * f);
        if (xfail) a[0] = a[1] = 0x7FC07FC0u;  // bf16 quiet NaN pair
        *(u32x2*)(gp + db * 32 + 8 * g + 4 * hi) = a;
      }
  }
}

// ------------------------------------------------------------------ fp32
constexpr int kF32Sub = 32;

// one thread per query row; K/V rows staged in LDS
template <int D>
__global__ void __launch_bounds__(128)
dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
              const float* __restrict__ v, const float* __restrict__ dout,
              const float* __restrict__ lse, const float* __restrict__ delta,
              const int32_t* __restrict__ q_ids, const int32_t* __restrict__ kv_ids, int32_t nq,
              int32_t nkv, int32_t H, float scale, int32_t bq, int32_t bkv,
              const uint8_t* __restrict__ tile_class, const int32_t* __restrict__ q_ptr,
              const int32_t* __restrict__ q_cols, const int32_t* __restrict__ q_order,
              int32_t nkt, float* __restrict__ dq) {
  __shared__ float ks[kF32Sub][D];
  __shared__ float vs[kF32Sub][D];
  __shared__ int32_t is[kF32Sub];
  const int tid = threadIdx.x;
  const int work = blockIdx.x / H, h = blockIdx.x - work * H;
  const int qt = q_order[work];
  const size_t rs = (size_t)H * D;
  const int qrow = qt * bq + tid;
  const bool qin = qrow < nq;
  const int qc = qin ? qrow : nq - 1;
  const int qtag = qin ? query_tag(q_ids[qrow]) : kPadQuery;
  const float l = lse[(size_t)h * nq + qc];
  const float dl = delta[(size_t)h * nq + qc];
  const bool live = qin && l != -INFINITY;
  float qr[D], dr[D], acc[D];
  for (int d = 0; d < D; ++d) {
    qr[d] = q[(size_t)qc * rs + h * D + d];
    dr[d] = dout[(size_t)qc * rs + h * D + d];
    acc[d] = 0.f;
  }
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
      if (!live) continue;
      for (int r = 0; r < n; ++r) {
        if (partial && is[r] != qtag) continue;
        float sc = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          sc = fmaf(qr[d], ks[r][d], sc);
          dp = fmaf(dr[d], vs[r][d], dp);
        }
        const float p = expf(sc * scale - l);
        const float dsv = p * (dp - dl);
        for (int d = 0; d < D; ++d) acc[d] = fmaf(dsv, ks[r][d], acc[d]);
      }
    }
  }
  if (qin)
    for (int d = 0; d < D; ++d) dq[(size_t)qrow * rs + h * D + d] = live ? acc[d] * scale : 0.f;
}

// one thread per key row; Q/dO rows, LSE, Delta and tags staged in LDS
template <int D>
__global__ void __launch_bounds__(128)
dkdv_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                const float* __restrict__ v, const float* __restrict__ dout,
                const float* __restrict__ lse, const float* __restrict__ delta,
                const int32_t* __restrict__ q_ids, const int32_t* __restrict__ kv_ids,
                int32_t nq, int32_t nkv, int32_t H, float scale, int32_t bq, int32_t bkv,
                const uint8_t* __restrict__ tile_class, const int32_t* __restrict__ kv_ptr,
                const int32_t* __restrict__ kv_rows, const int32_t* __restrict__ kv_order,
                int32_t nkt, float* __restrict__ dk, float* __restrict__ dv) {
  __shared__ float qs[kF32Sub][D];
  __shared__ float ds_[kF32Sub][D];
  __shared__ float ls[kF32Sub], dls[kF32Sub];
  __shared__ int32_t ts[kF32Sub];
  const int tid = threadIdx.x;
  const int work = blockIdx.x / H, h = blockIdx.x - work * H;
  const int kt = kv_order[work];
  const size_t rs = (size_t)H * D;
  const int krow = kt * bkv + tid;
  const bool kin = krow < nkv;
  const int kc = kin ? krow : nkv - 1;
  const int ktag = kin ? key_tag(kv_ids[krow]) : kPadKey;
  float kr_[D], vr[D], ka[D], va[D];
  for (int d = 0; d < D; ++d) {
    kr_[d] = k[(size_t)kc * rs + h * D + d];
    vr[d] = v[(size_t)kc * rs + h * D + d];
    ka[d] = va[d] = 0.f;
  }
  for (int e = kv_ptr[kt]; e < kv_ptr[kt + 1]; ++e) {
    const int qt = kv_rows[e];
    const bool partial = tile_class[(size_t)qt * nkt + kt] == 1;
    const int qend = min(qt * bq + bq, nq);
    for (int q0 = qt * bq; q0 < qend; q0 += kF32Sub) {
      const int n = min(kF32Sub, qend - q0);
      __syncthreads();
      for (int x = tid; x < kF32Sub * D; x += blockDim.x) {
        const int r = x / D, d = x % D;
        const int qr = min(q0 + r, nq - 1);
        qs[r][d] = q[(size_t)qr * rs + h * D + d];
        ds_[r][d] = dout[(size_t)qr * rs + h * D + d];
      }
      for (int r = tid; r < kF32Sub; r += blockDim.x) {
        const int qr = q0 + r;
        ls[r] = qr < nq ? lse[(size_t)h * nq + qr] : -INFINITY;
        dls[r] = qr < nq ? delta[(size_t)h * nq + qr] : 0.f;
        ts[r] = qr < nq ? query_tag(q_ids[qr]) : kPadQuery;
      }
      __syncthreads();
      if (!kin) continue;
      for (int r = 0; r < n; ++r) {
        if (ls[r] == -INFINITY) continue;
        if (partial && ts[r] != ktag) continue;
        float sc = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          sc = fmaf(qs[r][d], kr_[d], sc);
          dp = fmaf(ds_[r][d], vr[d], dp);
        }
        const float p = expf(sc * scale - ls[r]);
        const float dsv = p * (dp - dls[r]);
        for (int d = 0; d < D; ++d) {
          va[d] = fmaf(p, ds_[r][d], va[d]);
          ka[d] = fmaf(dsv, qs[r][d], ka[d]);
        }
      }
    }
  }
  if (kin)
    for (int d = 0; d < D; ++d) {
      dk[(size_t)krow * rs + h * D + d] = ka[d] * scale;
      dv[(size_t)krow * rs + h * D + d] = va[d];
    }
}

template <typename T, int D>
void launch_preprocess(const void* o, const void* dout, const float* lse, int32_t nq, int32_t H,
                       float* delta, float* lse2, hipStream_t s) {
  constexpr int kRows = 256 / (D / 16);
  const int64_t blocks = (int64_t)((nq + kRows - 1) / kRows) * H;
  hipLaunchKernelGGL((preprocess_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s,
                     (const T*)o, (const T*)dout, lse, nq, H, delta, lse2);
}

// Bound of the dK/dV kernel's hand-over wait, in polls of about 64 cycles each
// (2^20: tens of milliseconds, against a normal wait of none).  Tests lower it
// through pa_test_set_handover_spin_limit.
int32_t g_xch_spin_limit = 1 << 20;

// Launches one stage of the backward: 0 = the row terms alone (preprocess),
// 1 = the row terms and dQ (for bf16 128-wide heads one kernel does both), 2 =
// dK/dV.  `ws` holds Delta [H][nq] followed by LSE*log2(e) [H][nq]; stage 1
// writes them, stage 2 reads them.
int32_t bwd_stage(int stage, int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                  int32_t head_dim, float scale, const void* q, const void* k, const void* v,
                  const void* o, const void* dout, const float* lse, const int32_t* q_seq_id,
                  const int32_t* kv_seq_id, const pa_block_mask* mask, void* dq, void* dk,
                  void* dv, float* ws, hipStream_t s) {
  const dim3 gq(mask ? mask->nq_tiles * heads : 1), gk(mask ? mask->nkv_tiles * heads : 1);
  const dim3 gq2(mask ? (mask->nq_tiles + 1) / 2 * heads : 1);  // pairs of query tiles
  const float s2 = scale * pa::kLog2e;
  const bool bf = dtype == PA_BF16;
  float* delta = ws;
  float* lse2 = ws + (size_t)heads * nq;
#define PA_BWD_STAGES(D)                                                                         \
  if (stage == 0) {                                                                              \
    if (bf) launch_preprocess<uint16_t, D>(o, dout, lse, nq, heads, delta, lse2, s);             \
    else launch_preprocess<float, D>(o, dout, lse, nq, heads, delta, lse2, s);                   \
  } else if (stage == 1) {                                                                       \
    /* the paired bf16 kernel computes the row terms itself; the others read */                  \
    /* them from the workspace, filled by the preprocess first */                                \
    if (!(bf && D == 128)) {                                                                     \
      if (bf) launch_preprocess<uint16_t, D>(o, dout, lse, nq, heads, delta, lse2, s);           \
      else launch_preprocess<float, D>(o, dout, lse, nq, heads, delta, lse2, s);                 \
    }                                                                                            \
    if (bf && D == 128)                                                                          \
      hipLaunchKernelGGL(dq_bf16_pair_kernel<128>, gq2, dim3(512), 0, s, (const uint16_t*)q,     \
                         (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,          \
                         (const uint16_t*)o, lse, delta, lse2, q_seq_id, kv_seq_id, nq, nkv,     \
                         heads, s2, scale, mask->q_order, mask->pair_off, mask->pair_len,        \
                         mask->pair_ent, (uint16_t*)dq);                                         \
    else if (bf)                                                                                 \
      hipLaunchKernelGGL(dq_bf16_kernel<D>, gq, dim3(256), 0, s, (const uint16_t*)q,             \
                         (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, delta,   \
                         lse2, q_seq_id, kv_seq_id, nq, nkv, heads, s2, scale,                   \
                         mask->tile_class, mask->q_ptr, mask->q_cols, mask->q_order,             \
                         mask->nkv_tiles, (uint16_t*)dq);                                        \
    else                                                                                         \
      hipLaunchKernelGGL(dq_f32_kernel<D>, gq, dim3(mask->block_q), 0, s, (const float*)q,       \
                         (const float*)k, (const float*)v, (const float*)dout, lse, delta,       \
                         q_seq_id, kv_seq_id, nq, nkv, heads, scale, mask->block_q,              \
                         mask->block_kv, mask->tile_class, mask->q_ptr, mask->q_cols,            \
                         mask->q_order, mask->nkv_tiles, (float*)dq);                            \
  } else {                                                                                       \
    if (bf && D == 128)                                                                          \
      hipLaunchKernelGGL(dkdv_bf16_split_kernel<128>, gk, dim3(512), 0, s, (const uint16_t*)q,   \
                         (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, delta,   \
                         lse2, q_seq_id, kv_seq_id, nq, nkv, heads, s2, scale,                   \
                         mask->tile_class, mask->kv_ptr, mask->kv_rows, mask->kv_order,          \
                         mask->nkv_tiles, (uint16_t*)dk, (uint16_t*)dv, g_xch_spin_limit);       \
    else if (bf)                                                                                 \
      hipLaunchKernelGGL(dkdv_bf16_kernel<D>, gk, dim3(256), 0, s, (const uint16_t*)q,           \
                         (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, delta,   \
                         lse2, q_seq_id, kv_seq_id, nq, nkv, heads, s2, scale,                   \
                         mask->tile_class, mask->kv_ptr, mask->kv_rows, mask->kv_order,          \
                         mask->nkv_tiles, (uint16_t*)dk, (uint16_t*)dv);                         \
    else                                                                                         \
      hipLaunchKernelGGL(dkdv_f32_kernel<D>, gk, dim3(mask->block_kv), 0, s, (const float*)q,    \
                         (const float*)k, (const float*)v, (const float*)dout, lse, delta,       \
                         q_seq_id, kv_seq_id, nq, nkv, heads, scale, mask->block_q,              \
                         mask->block_kv, mask->tile_class, mask->kv_ptr, mask->kv_rows,          \
                         mask->kv_order, mask->nkv_tiles, (float*)dk, (float*)dv);               \
  }
  if (head_dim == 128) {
    PA_BWD_STAGES(128)
  } else {
    PA_BWD_STAGES(64)
  }
#undef PA_BWD_STAGES
  return pa::launch_status();
}

int32_t check_tensor(const void* p) {
  if (!p) return PA_ERR_NULL;
  return pa::aligned16(p) ? PA_OK : PA_ERR_ALIGN;
}

size_t workspace_bytes(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads, int32_t head_dim) {
  if ((dtype != PA_F32 && dtype != PA_BF16) || nq < 1 || nkv < 1 || heads < 1 ||
      (head_dim != 64 && head_dim != 128))
    return 0;
  return pa::align_up(2 * (size_t)heads * nq * sizeof(float), 256);
}

int32_t check_workspace(const void* ws, size_t bytes, int32_t dtype, int32_t nq, int32_t heads,
                        int32_t head_dim) {
  if (!ws) return PA_ERR_NULL;
  if (bytes < workspace_bytes(dtype, nq, 1, heads, head_dim)) return PA_ERR_WORKSPACE;
  return pa::aligned256(ws) ? PA_OK : PA_ERR_ALIGN;
}

}  // namespace

extern "C" size_t attn_packed_bwd_workspace_bytes(int32_t dtype, int32_t nq, int32_t nkv,
                                                  int32_t heads, int32_t head_dim) {
  return workspace_bytes(dtype, nq, nkv, heads, head_dim);
}

extern "C" int32_t attn_packed_bwd_preprocess(int32_t dtype, int32_t nq, int32_t heads,
                                              int32_t head_dim, const void* o, const void* dout,
                                              const float* lse, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_HEADDIM;
  if (nq < 1 || heads < 1) return PA_ERR_SHAPE;
  if (!lse) return PA_ERR_NULL;
  int32_t st;
  for (const void* p : {o, dout})
    if ((st = check_tensor(p))) return st;
  if ((st = check_workspace(workspace, workspace_bytes, dtype, nq, heads, head_dim))) return st;
  return bwd_stage(0, dtype, nq, 1, heads, head_dim, 0.f, nullptr, nullptr, nullptr, o, dout,
                   lse, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, (float*)workspace,
                   (hipStream_t)stream);
}

extern "C" int32_t attn_packed_bwd_dq(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                                      int32_t head_dim, float scale, const void* q, const void* k,
                                      const void* v, const void* o, const void* dout,
                                      const float* lse, void* workspace, size_t workspace_bytes,
                                      const int32_t* q_seq_id, const int32_t* kv_seq_id,
                                      const pa_block_mask* mask, void* dq, void* stream) {
  int32_t st = pa::check_attn_args(dtype, nq, nkv, heads, head_dim, mask);
  if (st != PA_OK) return st;
  if (!lse || !q_seq_id || !kv_seq_id) return PA_ERR_NULL;
  for (const void* p : {q, k, v, o, dout, (const void*)dq})
    if ((st = check_tensor(p))) return st;
  if ((st = check_workspace(workspace, workspace_bytes, dtype, nq, heads, head_dim))) return st;
  return bwd_stage(1, dtype, nq, nkv, heads, head_dim, scale, q, k, v, o, dout, lse, q_seq_id,
                   kv_seq_id, mask, dq, nullptr, nullptr, (float*)workspace,
                   (hipStream_t)stream);
}

extern "C" int32_t attn_packed_bwd_dkdv(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                                        int32_t head_dim, float scale, const void* q,
                                        const void* k, const void* v, const void* dout,
                                        const float* lse, const void* workspace,
                                        size_t workspace_bytes, const int32_t* q_seq_id,
                                        const int32_t* kv_seq_id, const pa_block_mask* mask,
                                        void* dk, void* dv, void* stream) {
  int32_t st = pa::check_attn_args(dtype, nq, nkv, heads, head_dim, mask);
  if (st != PA_OK) return st;
  if (!lse || !q_seq_id || !kv_seq_id) return PA_ERR_NULL;
  for (const void* p : {q, k, v, dout, (const void*)dk, (const void*)dv})
    if ((st = check_tensor(p))) return st;
  if ((st = check_workspace(workspace, workspace_bytes, dtype, nq, heads, head_dim))) return st;
  return bwd_stage(2, dtype, nq, nkv, heads, head_dim, scale, q, k, v, nullptr, dout, lse,
                   q_seq_id, kv_seq_id, mask, nullptr, dk, dv, (float*)workspace,
                   (hipStream_t)stream);
}

extern "C" int32_t attn_packed_bwd(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                                   int32_t head_dim, float scale, const void* q, const void* k,
                                   const void* v, const void* o, const void* dout,
                                   const float* lse, const int32_t* q_seq_id,
                                   const int32_t* kv_seq_id, const pa_block_mask* mask, void* dq,
                                   void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  int32_t st = pa::check_attn_args(dtype, nq, nkv, heads, head_dim, mask);
  if (st != PA_OK) return st;
  if (!lse || !q_seq_id || !kv_seq_id) return PA_ERR_NULL;
  for (const void* p : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if ((st = check_tensor(p))) return st;
  if ((st = check_workspace(workspace, workspace_bytes, dtype, nq, heads, head_dim))) return st;
  const hipStream_t s = (hipStream_t)stream;
  for (int stage = 1; stage < 3; ++stage) {  // row terms + dQ, then dK/dV
    st = bwd_stage(stage, dtype, nq, nkv, heads, head_dim, scale, q, k, v, o, dout, lse,
                   q_seq_id, kv_seq_id, mask, dq, dk, dv, (float*)workspace, s);
    if (st != PA_OK) return st;
  }
  return PA_OK;
}

// ------------------------------------------------------- no-allocation backward
// Fixed device-resident workspace for attn_packed_bwd_noalloc: callers that may
// not allocate (graph capture, serving loops) still need the backward's row
// terms (Delta and LSE2, 8 bytes per head and query).  Each device the library
// runs on holds one copy of this array until the process ends.  Host code must
// never pass `scratch` itself to a kernel (that is a host-side stand-in): the
// device address comes from hipGetSymbolAddress, once per device.
namespace {
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;  // H * nq <= 8,388,608
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on the first
// call made with that device current), or nullptr on a HIP error.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" size_t attn_packed_bwd_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int32_t attn_packed_bwd_noalloc(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                                           int32_t head_dim, float scale, const void* q,
                                           const void* k, const void* v, const void* o,
                                           const void* dout, const float* lse,
                                           const int32_t* q_seq_id, const int32_t* kv_seq_id,
                                           const pa_block_mask* mask, void* dq, void* dk,
                                           void* dv, void* stream) {
  int32_t st = pa::check_attn_args(dtype, nq, nkv, heads, head_dim, mask);
  if (st != PA_OK) return st;
  if (!lse || !q_seq_id || !kv_seq_id) return PA_ERR_NULL;
  for (const void* p : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if ((st = check_tensor(p))) return st;
  const size_t need = workspace_bytes(dtype, nq, nkv, heads, head_dim);
  if (need == 0 || need > kNoAllocScratchBytes) return PA_ERR_WORKSPACE;
  float* ws = (float*)scratch_address();
  if (!ws) return PA_ERR_HIP;
  // Every entry of Delta and LSE2 that a later stage reads is written by the
  // preprocess first, so nothing in the array needs clearing between calls.
  const hipStream_t s = (hipStream_t)stream;
  for (int stage = 1; stage < 3; ++stage) {  // row terms + dQ, then dK/dV
    st = bwd_stage(stage, dtype, nq, nkv, heads, head_dim, scale, q, k, v, o, dout, lse,
                   q_seq_id, kv_seq_id, mask, dq, dk, dv, ws, s);
    if (st != PA_OK) return st;
  }
  return PA_OK;
}

extern "C" int32_t pa_handover_failures(int32_t reset) {
  int32_t n = 0;
  if (hipMemcpyFromSymbol(&n, HIP_SYMBOL(g_handover_failures), sizeof(n), 0,
                          hipMemcpyDeviceToHost) != hipSuccess)
    return PA_ERR_HIP;
  if (reset) {
    const int32_t zero = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_handover_failures), &zero, sizeof(zero), 0,
                          hipMemcpyHostToDevice) != hipSuccess)
      return PA_ERR_HIP;
  }
  return n;
}

extern "C" int32_t pa_test_set_handover_spin_limit(int32_t limit) {
  const int32_t prev = g_xch_spin_limit;
  g_xch_spin_limit = limit >= 0 ? limit : (1 << 20);
  return prev;
}
