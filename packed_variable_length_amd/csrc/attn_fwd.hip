// Forward pass of packed segment-id masked attention.
//
// Per head, O = softmax(scale * Q K^T over allowed pairs) V and LSE = log of the
// softmax denominator; rows without an allowed key get O = 0, LSE = -inf.  The
// pair predicate is "same seq id, id >= 0" ("Furniture packing, variable length"
// report, implementation part); the kernel visits only the non-empty key tiles
// of its query tile (block sparsity from the seq ids, "LingBot-VA packing"
// report, section 2.2) and applies the elementwise mask only on partial tiles.
//
// bf16 kernel (gfx950 MFMA): a workgroup of 4 waves owns one 128-row query tile
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

#include "pa_common.h"

namespace {

using namespace pa;

// ------------------------------------------------------------------ bf16 MFMA
template <int D>
struct FwdBf16 {
  static constexpr int kThreads = 256;
  static constexpr int kBQ = 128;              // query rows per workgroup (= mask tile)
  static constexpr int kBKV = 128;             // key rows per mask tile
  static constexpr int kSub = 64;              // key rows per inner step
  static constexpr int kKStride = D * 2 + 16;  // bytes per K row in LDS
  static constexpr int kVStride = kSub * 2 + 8;  // bytes per V^T row in LDS
  static constexpr int kKBytes = kSub * kKStride;
  static constexpr int kVBytes = D * kVStride;
  static constexpr int kIdBytes = kSub * 4;
  static constexpr int kBuf = kKBytes + kVBytes + kIdBytes;
  static constexpr int kKChunks = kSub * D / 8 / kThreads;  // 16-byte K chunks per thread
  static constexpr int kVThreads = (kSub / 4) * (D / 8);    // threads holding a 4x8 V block
  static constexpr int kDB = D / 32;                         // 32-wide d blocks
  static constexpr int kKK = D / 16;                         // 16-deep k steps over d
};

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, const int32_t* __restrict__ q_ids,
                const int32_t* __restrict__ kv_ids, int32_t nq, int32_t nkv, int32_t H,
                float s2, const uint8_t* __restrict__ tile_class,
                const int32_t* __restrict__ q_ptr, const int32_t* __restrict__ q_cols,
                const int32_t* __restrict__ q_order, int32_t nkt, uint16_t* __restrict__ o,
                float* __restrict__ lse) {
  using C = FwdBf16<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kBuf];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const int work = blockIdx.x / H, h = blockIdx.x - work * H;
  const int qt = q_order[work];
  const int beg = q_ptr[qt];
  const int nsub = 2 * (q_ptr[qt + 1] - beg);
  const size_t rs = (size_t)H * D;  // elements between consecutive tokens

  const int qrow = qt * C::kBQ + wv * 32 + col;
  const bool qin = qrow < nq;
  const int qtag = qin ? query_tag(q_ids[qrow]) : kPadQuery;

  bf16x8 qf[C::kKK];
  {
    const uint16_t* qp = q + (size_t)(qin ? qrow : nq - 1) * rs + h * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < C::kKK; ++kk) qf[kk] = *(const bf16x8*)(qp + 16 * kk);
  }

  f32x16 oacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  if (nsub > 0) {
    u32x4 kreg[C::kKChunks];
    u32x4 vreg[4];
    int32_t idreg = kPadKey;

    auto gload = [&](int s) {
      const int kt = q_cols[beg + (s >> 1)];
      const int k0 = kt * C::kBKV + (s & 1) * C::kSub;
#pragma unroll
      for (int i = 0; i < C::kKChunks; ++i) {
        const int c = tid + C::kThreads * i;
        const int row = c / (D / 8), c8 = c % (D / 8);
        const int kr = min(k0 + row, nkv - 1);
        kreg[i] = *(const u32x4*)(k + (size_t)kr * rs + h * D + c8 * 8);
      }
      if (tid < C::kVThreads) {
        const int kg = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int vr = min(k0 + 4 * kg + r, nkv - 1);
          vreg[r] = *(const u32x4*)(v + (size_t)vr * rs + h * D + dc * 8);
        }
      }
      if (tid < C::kSub) {
        const int kr = k0 + tid;
        idreg = kr < nkv ? key_tag(kv_ids[kr]) : kPadKey;
      }
    };
    auto lstore = [&](int buf) {
      char* kl = smem + buf * C::kBuf;
      char* vl = kl + C::kKBytes;
      int32_t* il = (int32_t*)(vl + C::kVBytes);
#pragma unroll
      for (int i = 0; i < C::kKChunks; ++i) {
        const int c = tid + C::kThreads * i;
        const int row = c / (D / 8), c8 = c % (D / 8);
        *(u32x4*)(kl + row * C::kKStride + c8 * 16) = kreg[i];
      }
      if (tid < C::kVThreads) {
        const int kg = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int w = c >> 1, sh = (c & 1) * 16;
          const uint32_t x0 = (vreg[0][w] >> sh) & 0xFFFFu, x1 = (vreg[1][w] >> sh) & 0xFFFFu;
          const uint32_t x2 = (vreg[2][w] >> sh) & 0xFFFFu, x3 = (vreg[3][w] >> sh) & 0xFFFFu;
          u32x2 pk = {x0 | (x1 << 16), x2 | (x3 << 16)};
          *(u32x2*)(vl + (8 * dc + c) * C::kVStride + 8 * kg) = pk;
        }
      }
      if (tid < C::kSub) il[tid] = idreg;
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int s = 0; s < nsub; ++s) {
      const int buf = s & 1;
      if (s + 1 < nsub) gload(s + 1);
      const int kt = q_cols[beg + (s >> 1)];
      const bool partial = tile_class[(size_t)qt * nkt + kt] == 1;
      const char* kl = smem + buf * C::kBuf;
      const char* vl = kl + C::kKBytes;
      const int32_t* il = (const int32_t*)(vl + C::kVBytes);

      // S^T = K Q^T for 64 keys (two 32-key blocks) x this wave's 32 queries
      f32x16 sacc[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[mb][j] = 0.f;
        const char* krow = kl + (mb * 32 + col) * C::kKStride + 16 * hi;
#pragma unroll
        for (int kk = 0; kk < C::kKK; ++kk) {
          const bf16x8 a = *(const bf16x8*)(krow + 32 * kk);
          sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[mb], 0, 0, 0);
        }
      }
      // lane holds keys mb*32 + 8*(j/4) + 4*hi + j%4 of query `col`
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[mb][j] *= s2;
      if (partial) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int4 t4 = *(const int4*)(il + mb * 32 + 8 * g + 4 * hi);
            if (t4.x != qtag) sacc[mb][4 * g + 0] = -INFINITY;
            if (t4.y != qtag) sacc[mb][4 * g + 1] = -INFINITY;
            if (t4.z != qtag) sacc[mb][4 * g + 2] = -INFINITY;
            if (t4.w != qtag) sacc[mb][4 * g + 3] = -INFINITY;
          }
      }
      float mx = sacc[0][0];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[mb][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(m, mx);
      const float muse = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m - muse);
      float ps = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = __builtin_amdgcn_exp2f(sacc[mb][j] - muse);
          sacc[mb][j] = p;
          ps += p;
        }
      lsum = lsum * alpha + ps;
      m = mnew;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;

      // P^T as bf16 B operands: slice kb covers keys 16kb..16kb+15
      bf16x8 pb[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int mb = kb >> 1, b0 = (kb & 1) * 8;
        u32x4 w;
        w[0] = pack_bf16x2(sacc[mb][b0 + 0], sacc[mb][b0 + 1]);
        w[1] = pack_bf16x2(sacc[mb][b0 + 2], sacc[mb][b0 + 3]);
        w[2] = pack_bf16x2(sacc[mb][b0 + 4], sacc[mb][b0 + 5]);
        w[3] = pack_bf16x2(sacc[mb][b0 + 6], sacc[mb][b0 + 7]);
        pb[kb] = __builtin_bit_cast(bf16x8, w);
      }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) {
        const char* vrow = vl + (db * 32 + col) * C::kVStride + 8 * hi;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const u32x2 lo = *(const u32x2*)(vrow + 32 * kb);
          const u32x2 up = *(const u32x2*)(vrow + 32 * kb + 16);
          const u32x4 w = {lo[0], lo[1], up[0], up[1]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                             pb[kb], oacc[db], 0, 0, 0);
        }
      }
      if (s + 1 < nsub) lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // epilogue: both half-waves hold partial sums of the same query
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  const bool any = ltot > 0.f;
  const float inv = any ? 1.f / ltot : 0.f;
  if (qin) {
    uint16_t* op = o + (size_t)qrow * rs + h * D;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pk = {0u, 0u};
        if (any) {
          pk[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
          pk[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        }
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
      hipLaunchKernelGGL(fwd_bf16_kernel<128>, grid, dim3(256), 0, s, (const uint16_t*)q,
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
