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
// Three launches, none with atomics:
//   delta    Delta = rowsum(dO * O)  (HBM-bound)
//   dq       query-major, one 128-row query tile per workgroup: S^T = K Q^T,
//            dP^T = V dO^T, dS^T, dQ^T += K^T dS^T (query index along the lanes)
//   dkdv     key-major, one 128-row key tile per workgroup: S = Q K^T,
//            dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS (key index along
//            the lanes, dK and dV accumulated in registers)
// Splitting dQ from dK/dV recomputes S and dP once more (14 instead of 10
// d*pairs flops per head) but needs no fp32 atomics, no zero-filled accumulator
// and no conversion pass, and is deterministic.
#include <math.h>

#include "pa_common.h"

namespace {

using namespace pa;

// ------------------------------------------------------------------ delta
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

// 8 threads per (token, head) row of D = 128 (16 elements each) or 4 threads
// for D = 64; the row sum is reduced with lane exchanges.
template <typename T, int D>
__global__ void __launch_bounds__(256)
delta_kernel(const T* __restrict__ o, const T* __restrict__ dout, int32_t nq, int32_t H,
             float* __restrict__ delta) {
  constexpr int kPer = D / 16;  // threads per row
  const int64_t rows = (int64_t)nq * H;
  const int64_t row = (int64_t)blockIdx.x * (256 / kPer) + threadIdx.x / kPer;
  const int part = threadIdx.x % kPer;
  float acc = 0.f;
  if (row < rows) {
    float a[16], b[16];
    load16<T>(o + row * D + part * 16, a);
    load16<T>(dout + row * D + part * 16, b);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = fmaf(a[i], b[i], acc);
  }
#pragma unroll
  for (int off = kPer / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) {
    const int i = (int)(row / H), h = (int)(row % H);
    delta[(size_t)h * nq + i] = acc;
  }
}

// ------------------------------------------------------------------ bf16 dq
template <int D>
struct DqBf16 {
  static constexpr int kSub = 32;                 // key rows per inner step
  static constexpr int kRow = D * 2 + 16;         // bytes per K / V row in LDS
  static constexpr int kTRow = kSub * 2 + 8;      // bytes per K^T row in LDS
  static constexpr int kK = 0;
  static constexpr int kV = kK + kSub * kRow;
  static constexpr int kKt = kV + kSub * kRow;
  static constexpr int kId = kKt + D * kTRow;
  static constexpr int kBuf = kId + kSub * 4;
  static constexpr int kBlocks = (kSub / 4) * (D / 8);  // 4x8 blocks per operand
  static constexpr int kDB = D / 32, kKK = D / 16;
};

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
dq_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
               const float* __restrict__ lse, const float* __restrict__ delta,
               const int32_t* __restrict__ q_ids, const int32_t* __restrict__ kv_ids,
               int32_t nq, int32_t nkv, int32_t H, float s2, float scale,
               const uint8_t* __restrict__ tile_class, const int32_t* __restrict__ q_ptr,
               const int32_t* __restrict__ q_cols, const int32_t* __restrict__ q_order,
               int32_t nkt, uint16_t* __restrict__ dq) {
  using C = DqBf16<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kBuf];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const int work = blockIdx.x / H, h = blockIdx.x - work * H;
  const int qt = q_order[work];
  const int beg = q_ptr[qt];
  const int nsub = 4 * (q_ptr[qt + 1] - beg);
  const size_t rs = (size_t)H * D;

  const int qrow = qt * 128 + wv * 32 + col;
  const bool qin = qrow < nq;
  const int qc = qin ? qrow : nq - 1;
  const int qtag = qin ? query_tag(q_ids[qrow]) : kPadQuery;
  const float l_raw = lse[(size_t)h * nq + qc];
  const float lse2 = l_raw == -INFINITY ? INFINITY : l_raw * kLog2e;  // P = 0 on empty rows
  const float dlt = delta[(size_t)h * nq + qc];

  bf16x8 qf[C::kKK], df[C::kKK];
  {
    const uint16_t* qp = q + (size_t)qc * rs + h * D + 8 * hi;
    const uint16_t* dp = dout + (size_t)qc * rs + h * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < C::kKK; ++kk) {
      qf[kk] = *(const bf16x8*)(qp + 16 * kk);
      df[kk] = *(const bf16x8*)(dp + 16 * kk);
    }
  }
  f32x16 acc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;

  if (nsub > 0) {
    // threads 0..127 stage K (row-major and transposed), 128..255 stage V
    const int b = tid & 127;
    const bool is_v = tid >= 128;
    const bool stager = b < C::kBlocks;
    const int kg = b / (D / 8), dc = b % (D / 8);
    u32x4 reg[4];
    int32_t idreg = kPadKey;
    auto gload = [&](int s) {
      const int kt = q_cols[beg + (s >> 2)];
      const int k0 = kt * 128 + (s & 3) * C::kSub;
      if (stager) {
        const uint16_t* src = is_v ? v : k;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kr = min(k0 + 4 * kg + r, nkv - 1);
          reg[r] = *(const u32x4*)(src + (size_t)kr * rs + h * D + dc * 8);
        }
      }
      if (tid < C::kSub) {
        const int kr = k0 + tid;
        idreg = kr < nkv ? key_tag(kv_ids[kr]) : kPadKey;
      }
    };
    auto lstore = [&](int buf) {
      char* base = smem + buf * C::kBuf;
      if (stager) {
        char* rm = base + (is_v ? C::kV : C::kK);
#pragma unroll
        for (int r = 0; r < 4; ++r) *(u32x4*)(rm + (4 * kg + r) * C::kRow + 16 * dc) = reg[r];
        if (!is_v) {
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const int w = c >> 1, sh = (c & 1) * 16;
            const uint32_t x0 = (reg[0][w] >> sh) & 0xFFFFu, x1 = (reg[1][w] >> sh) & 0xFFFFu;
            const uint32_t x2 = (reg[2][w] >> sh) & 0xFFFFu, x3 = (reg[3][w] >> sh) & 0xFFFFu;
            u32x2 pk = {x0 | (x1 << 16), x2 | (x3 << 16)};
            *(u32x2*)(base + C::kKt + (8 * dc + c) * C::kTRow + 8 * kg) = pk;
          }
        }
      }
      if (tid < C::kSub) ((int32_t*)(base + C::kId))[tid] = idreg;
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int s = 0; s < nsub; ++s) {
      const int buf = s & 1;
      if (s + 1 < nsub) gload(s + 1);
      const int kt = q_cols[beg + (s >> 2)];
      const bool partial = tile_class[(size_t)qt * nkt + kt] == 1;
      const char* base = smem + buf * C::kBuf;

      f32x16 st, dpt;  // S^T and dP^T: keys 8(j/4)+4hi+j%4 x query `col`
#pragma unroll
      for (int j = 0; j < 16; ++j) st[j] = dpt[j] = 0.f;
      const char* krow = base + C::kK + col * C::kRow + 16 * hi;
      const char* vrow = base + C::kV + col * C::kRow + 16 * hi;
#pragma unroll
      for (int kk = 0; kk < C::kKK; ++kk) {
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow + 32 * kk), qf[kk],
                                                      st, 0, 0, 0);
        dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vrow + 32 * kk), df[kk],
                                                       dpt, 0, 0, 0);
      }
      float p[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) p[j] = __builtin_amdgcn_exp2f(st[j] * s2 - lse2);
      if (partial) {
        const int32_t* il = (const int32_t*)(base + C::kId);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int4 t4 = *(const int4*)(il + 8 * g + 4 * hi);
          if (t4.x != qtag) p[4 * g + 0] = 0.f;
          if (t4.y != qtag) p[4 * g + 1] = 0.f;
          if (t4.z != qtag) p[4 * g + 2] = 0.f;
          if (t4.w != qtag) p[4 * g + 3] = 0.f;
        }
      }
      bf16x8 ds[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 8 * kb + 2 * e;
          w[e] = pack_bf16x2(p[j] * (dpt[j] - dlt), p[j + 1] * (dpt[j + 1] - dlt));
        }
        ds[kb] = __builtin_bit_cast(bf16x8, w);
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) {
        const char* kt_row = base + C::kKt + (db * 32 + col) * C::kTRow + 8 * hi;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x2 lo = *(const u32x2*)(kt_row + 32 * kb);
          const u32x2 up = *(const u32x2*)(kt_row + 32 * kb + 16);
          const u32x4 w = {lo[0], lo[1], up[0], up[1]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                            ds[kb], acc[db], 0, 0, 0);
        }
      }
      if (s + 1 < nsub) lstore(buf ^ 1);
      __syncthreads();
    }
  }
  if (qin) {
    uint16_t* op = dq + (size_t)qrow * rs + h * D;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
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
template <int D>
struct DkvBf16 {
  static constexpr int kSub = 32;             // query rows per inner step
  static constexpr int kRow = D * 2 + 16;     // bytes per Q / dO row in LDS
  static constexpr int kTRow = kSub * 2 + 8;  // bytes per Q^T / dO^T row in LDS
  static constexpr int kQ = 0;
  static constexpr int kDo = kQ + kSub * kRow;
  static constexpr int kQt = kDo + kSub * kRow;
  static constexpr int kDot = kQt + D * kTRow;
  static constexpr int kLse = kDot + D * kTRow;
  static constexpr int kDelta = kLse + kSub * 4;
  static constexpr int kTag = kDelta + kSub * 4;
  static constexpr int kBuf = kTag + kSub * 4;
  static constexpr int kBlocks = (kSub / 4) * (D / 8);
  static constexpr int kDB = D / 32, kKK = D / 16;
};

template <int D>
__global__ void __launch_bounds__(256)
dkdv_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                 const float* __restrict__ lse, const float* __restrict__ delta,
                 const int32_t* __restrict__ q_ids, const int32_t* __restrict__ kv_ids,
                 int32_t nq, int32_t nkv, int32_t H, float s2, float scale,
                 const uint8_t* __restrict__ tile_class, const int32_t* __restrict__ kv_ptr,
                 const int32_t* __restrict__ kv_rows, const int32_t* __restrict__ kv_order,
                 int32_t nkt, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  using C = DkvBf16<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kBuf];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const int work = blockIdx.x / H, h = blockIdx.x - work * H;
  const int kt = kv_order[work];
  const int beg = kv_ptr[kt];
  const int nsub = 4 * (kv_ptr[kt + 1] - beg);
  const size_t rs = (size_t)H * D;

  const int krow = kt * 128 + wv * 32 + col;
  const bool kin = krow < nkv;
  const int kc = kin ? krow : nkv - 1;
  const int ktag = kin ? key_tag(kv_ids[krow]) : kPadKey;

  bf16x8 kf[C::kKK], vf[C::kKK];
  {
    const uint16_t* kp = k + (size_t)kc * rs + h * D + 8 * hi;
    const uint16_t* vp = v + (size_t)kc * rs + h * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < C::kKK; ++kk) {
      kf[kk] = *(const bf16x8*)(kp + 16 * kk);
      vf[kk] = *(const bf16x8*)(vp + 16 * kk);
    }
  }
  f32x16 dka[C::kDB], dva[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) dka[db][j] = dva[db][j] = 0.f;

  if (nsub > 0) {
    // threads 0..127 stage Q, 128..255 stage dO (each row-major and transposed)
    const int b = tid & 127;
    const bool is_do = tid >= 128;
    const bool stager = b < C::kBlocks;
    const int qg = b / (D / 8), dc = b % (D / 8);
    u32x4 reg[4];
    float lreg = INFINITY, dreg = 0.f;
    int32_t treg = kPadQuery;
    auto gload = [&](int s) {
      const int qt = kv_rows[beg + (s >> 2)];
      const int q0 = qt * 128 + (s & 3) * C::kSub;
      if (stager) {
        const uint16_t* src = is_do ? dout : q;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qr = min(q0 + 4 * qg + r, nq - 1);
          reg[r] = *(const u32x4*)(src + (size_t)qr * rs + h * D + dc * 8);
        }
      }
      if (tid < C::kSub) {
        const int qr = q0 + tid;
        if (qr < nq) {
          const float l = lse[(size_t)h * nq + qr];
          lreg = l == -INFINITY ? INFINITY : l * kLog2e;
          dreg = delta[(size_t)h * nq + qr];
          treg = query_tag(q_ids[qr]);
        } else {
          lreg = INFINITY;
          dreg = 0.f;
          treg = kPadQuery;
        }
      }
    };
    auto lstore = [&](int buf) {
      char* base = smem + buf * C::kBuf;
      if (stager) {
        char* rm = base + (is_do ? C::kDo : C::kQ);
        char* tr = base + (is_do ? C::kDot : C::kQt);
#pragma unroll
        for (int r = 0; r < 4; ++r) *(u32x4*)(rm + (4 * qg + r) * C::kRow + 16 * dc) = reg[r];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int w = c >> 1, sh = (c & 1) * 16;
          const uint32_t x0 = (reg[0][w] >> sh) & 0xFFFFu, x1 = (reg[1][w] >> sh) & 0xFFFFu;
          const uint32_t x2 = (reg[2][w] >> sh) & 0xFFFFu, x3 = (reg[3][w] >> sh) & 0xFFFFu;
          u32x2 pk = {x0 | (x1 << 16), x2 | (x3 << 16)};
          *(u32x2*)(tr + (8 * dc + c) * C::kTRow + 8 * qg) = pk;
        }
      }
      if (tid < C::kSub) {
        ((float*)(base + C::kLse))[tid] = lreg;
        ((float*)(base + C::kDelta))[tid] = dreg;
        ((int32_t*)(base + C::kTag))[tid] = treg;
      }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int s = 0; s < nsub; ++s) {
      const int buf = s & 1;
      if (s + 1 < nsub) gload(s + 1);
      const int qt = kv_rows[beg + (s >> 2)];
      const bool partial = tile_class[(size_t)qt * nkt + kt] == 1;
      const char* base = smem + buf * C::kBuf;

      f32x16 sc, dpc;  // S and dP: queries 8(j/4)+4hi+j%4 x key `col`
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[j] = dpc[j] = 0.f;
      const char* qrow = base + C::kQ + col * C::kRow + 16 * hi;
      const char* drow = base + C::kDo + col * C::kRow + 16 * hi;
#pragma unroll
      for (int kk = 0; kk < C::kKK; ++kk) {
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(qrow + 32 * kk), kf[kk],
                                                      sc, 0, 0, 0);
        dpc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(drow + 32 * kk), vf[kk],
                                                       dpc, 0, 0, 0);
      }
      const float* lsel = (const float*)(base + C::kLse);
      const float* dlt = (const float*)(base + C::kDelta);
      const int32_t* tg = (const int32_t*)(base + C::kTag);
      float p[16], dl[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *(const f32x4*)(lsel + 8 * g + 4 * hi);
        const f32x4 d4 = *(const f32x4*)(dlt + 8 * g + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * g + e;
          p[j] = __builtin_amdgcn_exp2f(sc[j] * s2 - l4[e]);
          dl[j] = d4[e];
        }
        if (partial) {
          const int4 t4 = *(const int4*)(tg + 8 * g + 4 * hi);
          if (t4.x != ktag) p[4 * g + 0] = 0.f;
          if (t4.y != ktag) p[4 * g + 1] = 0.f;
          if (t4.z != ktag) p[4 * g + 2] = 0.f;
          if (t4.w != ktag) p[4 * g + 3] = 0.f;
        }
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 wp, wd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 8 * kb + 2 * e;
          wp[e] = pack_bf16x2(p[j], p[j + 1]);
          wd[e] = pack_bf16x2(p[j] * (dpc[j] - dl[j]), p[j + 1] * (dpc[j + 1] - dl[j + 1]));
        }
        pb[kb] = __builtin_bit_cast(bf16x8, wp);
        dsb[kb] = __builtin_bit_cast(bf16x8, wd);
      }
      // dV^T += dO^T P ; dK^T += Q^T dS
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) {
        const char* dot_row = base + C::kDot + (db * 32 + col) * C::kTRow + 8 * hi;
        const char* qt_row = base + C::kQt + (db * 32 + col) * C::kTRow + 8 * hi;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x2 a0 = *(const u32x2*)(dot_row + 32 * kb);
          const u32x2 a1 = *(const u32x2*)(dot_row + 32 * kb + 16);
          const u32x4 wa = {a0[0], a0[1], a1[0], a1[1]};
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wa),
                                                            pb[kb], dva[db], 0, 0, 0);
          const u32x2 b0 = *(const u32x2*)(qt_row + 32 * kb);
          const u32x2 b1 = *(const u32x2*)(qt_row + 32 * kb + 16);
          const u32x4 wb = {b0[0], b0[1], b1[0], b1[1]};
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wb),
                                                            dsb[kb], dka[db], 0, 0, 0);
        }
      }
      if (s + 1 < nsub) lstore(buf ^ 1);
      __syncthreads();
    }
  }
  if (kin) {
    uint16_t* kp = dk + (size_t)krow * rs + h * D;
    uint16_t* vp = dv + (size_t)krow * rs + h * D;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
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
void launch_delta(const void* o, const void* dout, int32_t nq, int32_t H, float* delta,
                  hipStream_t s) {
  constexpr int kPer = D / 16;
  const int64_t rows = (int64_t)nq * H;
  const int64_t blocks = (rows + (256 / kPer) - 1) / (256 / kPer);
  hipLaunchKernelGGL((delta_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, (const T*)o,
                     (const T*)dout, nq, H, delta);
}

}  // namespace

extern "C" size_t attn_packed_bwd_workspace_bytes(int32_t dtype, int32_t nq, int32_t nkv,
                                                  int32_t heads, int32_t head_dim) {
  if ((dtype != PA_F32 && dtype != PA_BF16) || nq < 1 || nkv < 1 || heads < 1 ||
      (head_dim != 64 && head_dim != 128))
    return 0;
  return pa::align_up((size_t)heads * nq * sizeof(float), 256);
}

namespace {

// Launches one stage of the backward; stage 0 = Delta, 1 = dQ, 2 = dK/dV.
int32_t bwd_stage(int stage, int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                  int32_t head_dim, float scale, const void* q, const void* k, const void* v,
                  const void* o, const void* dout, const float* lse, const int32_t* q_seq_id,
                  const int32_t* kv_seq_id, const pa_block_mask* mask, void* dq, void* dk,
                  void* dv, float* delta, hipStream_t s) {
  const dim3 gq(mask->nq_tiles * heads), gk(mask->nkv_tiles * heads);
  const float s2 = scale * pa::kLog2e;
  const bool bf = dtype == PA_BF16;
  const dim3 bqd(mask->block_q), bkd(mask->block_kv);
#define PA_BWD_STAGES(D)                                                                         \
  if (stage == 0) {                                                                              \
    if (bf) launch_delta<uint16_t, D>(o, dout, nq, heads, delta, s);                             \
    else launch_delta<float, D>(o, dout, nq, heads, delta, s);                                   \
  } else if (stage == 1) {                                                                       \
    if (bf)                                                                                      \
      hipLaunchKernelGGL(dq_bf16_kernel<D>, gq, dim3(256), 0, s, (const uint16_t*)q,             \
                         (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, lse,     \
                         delta, q_seq_id, kv_seq_id, nq, nkv, heads, s2, scale,                  \
                         mask->tile_class, mask->q_ptr, mask->q_cols, mask->q_order,             \
                         mask->nkv_tiles, (uint16_t*)dq);                                        \
    else                                                                                         \
      hipLaunchKernelGGL(dq_f32_kernel<D>, gq, bqd, 0, s, (const float*)q, (const float*)k,      \
                         (const float*)v, (const float*)dout, lse, delta, q_seq_id, kv_seq_id,   \
                         nq, nkv, heads, scale, mask->block_q, mask->block_kv,                   \
                         mask->tile_class, mask->q_ptr, mask->q_cols, mask->q_order,             \
                         mask->nkv_tiles, (float*)dq);                                           \
  } else {                                                                                       \
    if (bf)                                                                                      \
      hipLaunchKernelGGL(dkdv_bf16_kernel<D>, gk, dim3(256), 0, s, (const uint16_t*)q,           \
                         (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, lse,     \
                         delta, q_seq_id, kv_seq_id, nq, nkv, heads, s2, scale,                  \
                         mask->tile_class, mask->kv_ptr, mask->kv_rows, mask->kv_order,          \
                         mask->nkv_tiles, (uint16_t*)dk, (uint16_t*)dv);                         \
    else                                                                                         \
      hipLaunchKernelGGL(dkdv_f32_kernel<D>, gk, bkd, 0, s, (const float*)q, (const float*)k,    \
                         (const float*)v, (const float*)dout, lse, delta, q_seq_id, kv_seq_id,   \
                         nq, nkv, heads, scale, mask->block_q, mask->block_kv,                   \
                         mask->tile_class, mask->kv_ptr, mask->kv_rows, mask->kv_order,          \
                         mask->nkv_tiles, (float*)dk, (float*)dv);                               \
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

}  // namespace

extern "C" int32_t attn_packed_bwd_preprocess(int32_t dtype, int32_t nq, int32_t heads,
                                              int32_t head_dim, const void* o, const void* dout,
                                              float* delta, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_HEADDIM;
  if (nq < 1 || heads < 1) return PA_ERR_SHAPE;
  if (!delta) return PA_ERR_NULL;
  for (const void* p : {o, dout})
    if (int32_t st = check_tensor(p)) return st;
  const hipStream_t s = (hipStream_t)stream;
  if (head_dim == 128) {
    if (dtype == PA_BF16) launch_delta<uint16_t, 128>(o, dout, nq, heads, delta, s);
    else launch_delta<float, 128>(o, dout, nq, heads, delta, s);
  } else {
    if (dtype == PA_BF16) launch_delta<uint16_t, 64>(o, dout, nq, heads, delta, s);
    else launch_delta<float, 64>(o, dout, nq, heads, delta, s);
  }
  return pa::launch_status();
}

extern "C" int32_t attn_packed_bwd_dq(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                                      int32_t head_dim, float scale, const void* q, const void* k,
                                      const void* v, const void* dout, const float* lse,
                                      const float* delta, const int32_t* q_seq_id,
                                      const int32_t* kv_seq_id, const pa_block_mask* mask,
                                      void* dq, void* stream) {
  int32_t st = pa::check_attn_args(dtype, nq, nkv, heads, head_dim, mask);
  if (st != PA_OK) return st;
  if (!lse || !delta || !q_seq_id || !kv_seq_id) return PA_ERR_NULL;
  for (const void* p : {q, k, v, dout, (const void*)dq})
    if ((st = check_tensor(p))) return st;
  return bwd_stage(1, dtype, nq, nkv, heads, head_dim, scale, q, k, v, nullptr, dout, lse,
                   q_seq_id, kv_seq_id, mask, dq, nullptr, nullptr, (float*)delta,
                   (hipStream_t)stream);
}

extern "C" int32_t attn_packed_bwd_dkdv(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                                        int32_t head_dim, float scale, const void* q,
                                        const void* k, const void* v, const void* dout,
                                        const float* lse, const float* delta,
                                        const int32_t* q_seq_id, const int32_t* kv_seq_id,
                                        const pa_block_mask* mask, void* dk, void* dv,
                                        void* stream) {
  int32_t st = pa::check_attn_args(dtype, nq, nkv, heads, head_dim, mask);
  if (st != PA_OK) return st;
  if (!lse || !delta || !q_seq_id || !kv_seq_id) return PA_ERR_NULL;
  for (const void* p : {q, k, v, dout, (const void*)dk, (const void*)dv})
    if ((st = check_tensor(p))) return st;
  return bwd_stage(2, dtype, nq, nkv, heads, head_dim, scale, q, k, v, nullptr, dout, lse,
                   q_seq_id, kv_seq_id, mask, nullptr, dk, dv, (float*)delta,
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
  if (!lse || !q_seq_id || !kv_seq_id || !workspace) return PA_ERR_NULL;
  for (const void* p : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if ((st = check_tensor(p))) return st;
  if (workspace_bytes < attn_packed_bwd_workspace_bytes(dtype, nq, nkv, heads, head_dim))
    return PA_ERR_WORKSPACE;
  if (!pa::aligned256(workspace)) return PA_ERR_ALIGN;
  float* delta = (float*)workspace;
  const hipStream_t s = (hipStream_t)stream;
  for (int stage = 0; stage < 3; ++stage) {
    st = bwd_stage(stage, dtype, nq, nkv, heads, head_dim, scale, q, k, v, o, dout, lse,
                   q_seq_id, kv_seq_id, mask, dq, dk, dv, delta, s);
    if (st != PA_OK) return st;
  }
  return PA_OK;
}
