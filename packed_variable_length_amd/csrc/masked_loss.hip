// Frame-valid masked squared-error loss over a packed batch, and its gradient.
//
// "LingBot-VA packing" report, section 2.1 (compute_loss): the latent and action
// losses of a padded pack are averaged over valid frames only.  Here a token is
// valid iff its seq id is >= 0 (padding frames carry -1):
//   L = sum_{valid i} sum_c (pred - target)^2 / (n_valid * C),  L = 0 if n_valid = 0,
//   dL/dpred = 2 (pred - target) / (n_valid * C) on valid rows, 0 on padding rows.
//
// HBM-bound elementwise work plus a reduction.  A fixed grid of kLossBlocks
// workgroups owns contiguous row ranges; each sums its range in fp32 (16-byte
// vector loads, thread-sequential then wave and block trees) into a per-block
// partial, and one workgroup adds the partials in index order, so the result
// is bitwise reproducible.  Padding rows are never read.  The fused entry
// point first counts the valid rows (ids only), then reads pred and target
// once, writing the gradient and the squared-error partials in the same pass.
#include "pa_common.h"

namespace {

using namespace pa;

constexpr int kLossBlocks = 1024;  // fixed partial count
constexpr int kLossThreads = 256;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* f);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* f) {
  const u32x4 a = *(const u32x4*)p;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[2 * w] = bf16_bits_to_f32(a[w] & 0xFFFFu);
    f[2 * w + 1] = bf16_bits_to_f32(a[w] >> 16);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* f) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[w] = a[w];
    f[4 + w] = b[w];
  }
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* f);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float* f) {
  u32x4 a;
#pragma unroll
  for (int w = 0; w < 4; ++w) a[w] = pack_bf16x2(f[2 * w], f[2 * w + 1]);
  *(u32x4*)p = a;
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* f) {
  *(f32x4*)p = f32x4{f[0], f[1], f[2], f[3]};
  *(f32x4*)(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
}

template <typename V>
__device__ __forceinline__ V block_sum(V v, V* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  V t = 0;
#pragma unroll
  for (int w = 0; w < kLossThreads / 64; ++w) t += red[w];
  return t;
}

struct Range {
  int r0, r1;
};
__device__ __forceinline__ Range block_rows(int n, int rows_per) {
  const int r0 = min(n, (int)blockIdx.x * rows_per);
  return {r0, min(n, r0 + rows_per)};
}

// Valid-row count of this block's row range, into cnt_part[blockIdx.x].
__global__ void __launch_bounds__(kLossThreads)
loss_count_kernel(const int32_t* __restrict__ ids, int32_t n, int32_t rows_per,
             uint32_t* __restrict__ cnt_part) {
  __shared__ uint32_t red[kLossThreads / 64];
  const Range rg = block_rows(n, rows_per);
  uint32_t cnt = 0;
  for (int r = rg.r0 + threadIdx.x; r < rg.r1; r += kLossThreads) cnt += ids[r] >= 0 ? 1u : 0u;
  cnt = block_sum(cnt, red);
  if (threadIdx.x == 0) cnt_part[blockIdx.x] = cnt;
}

// Squared errors of the valid rows of this block's range, into sse_part[b];
// with COUNT also the valid-row count into cnt_part[b]; with GRAD also the
// gradient rows (scale from the finished counts in cnt_part).
template <typename T, bool COUNT, bool GRAD>
__global__ void __launch_bounds__(kLossThreads)
loss_sse_kernel(const T* __restrict__ pred, const T* __restrict__ target,
           const int32_t* __restrict__ ids, int32_t n, int32_t c, int32_t rows_per, int32_t nparts,
           float upstream, float* __restrict__ sse_part, uint32_t* __restrict__ cnt_part,
           T* __restrict__ dpred) {
  __shared__ float redf[kLossThreads / 64];
  __shared__ uint32_t redu[kLossThreads / 64];
  const Range rg = block_rows(n, rows_per);
  const uint32_t vec = (uint32_t)c / 8;  // 8-element vectors per row
  float k = 0.f;
  if (GRAD) {
    uint32_t total = 0;
    for (int i = threadIdx.x; i < nparts; i += kLossThreads) total += cnt_part[i];
    total = block_sum(total, redu);
    // same rounding as loss_finish_kernel's stats[3] times upstream (masked_mse_bwd)
    k = total > 0 ? (float)(2.0 / ((double)total * (double)c)) * upstream : 0.f;
  }
  float sse = 0.f;
  const uint32_t e1 = (uint32_t)(rg.r1 - rg.r0) * vec;
  for (uint32_t e = threadIdx.x; e < e1; e += kLossThreads) {
    const uint32_t rr = e / vec;
    const int r = rg.r0 + (int)rr;
    const size_t off = (size_t)r * c + (size_t)(e - rr * vec) * 8;
    if (ids[r] >= 0) {
      float a[8], b[8];
      load8<T>(pred + off, a);
      load8<T>(target + off, b);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = a[i] - b[i];
        sse = fmaf(d, d, sse);
        a[i] = k * d;
      }
      if (GRAD) store8<T>(dpred + off, a);
    } else if (GRAD) {
      const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      store8<T>(dpred + off, z);
    }
  }
  sse = block_sum(sse, redf);
  uint32_t cnt = 0;
  if (COUNT) {
    for (int r = rg.r0 + threadIdx.x; r < rg.r1; r += kLossThreads) cnt += ids[r] >= 0 ? 1u : 0u;
    cnt = block_sum(cnt, redu);
  }
  if (threadIdx.x == 0) {
    sse_part[blockIdx.x] = sse;
    if (COUNT) cnt_part[blockIdx.x] = cnt;
  }
}

// One workgroup: stats = {loss, sum of squared errors, n_valid, grad factor}.
__global__ void __launch_bounds__(kLossThreads)
loss_finish_kernel(const float* __restrict__ sse_part, const uint32_t* __restrict__ cnt_part,
              int32_t nparts, int32_t c, float* __restrict__ stats) {
  __shared__ float redf[kLossThreads / 64];
  __shared__ uint32_t redu[kLossThreads / 64];
  float sse = 0.f;
  uint32_t cnt = 0;
  for (int i = threadIdx.x; i < nparts; i += kLossThreads) {
    sse += sse_part[i];
    cnt += cnt_part[i];
  }
  sse = block_sum(sse, redf);
  cnt = block_sum(cnt, redu);
  if (threadIdx.x == 0) {
    const double denom = (double)cnt * (double)c;
    stats[0] = cnt > 0 ? (float)((double)sse / denom) : 0.f;
    stats[1] = sse;
    stats[2] = (float)cnt;
    stats[3] = cnt > 0 ? (float)(2.0 / denom) : 0.f;
  }
}

// Gradient only, from the factor stats[3] of a finished forward.
template <typename T>
__global__ void __launch_bounds__(kLossThreads)
loss_grad_kernel(const T* __restrict__ pred, const T* __restrict__ target,
            const int32_t* __restrict__ ids, int32_t n, int32_t c, int32_t rows_per,
            const float* __restrict__ stats, float upstream, T* __restrict__ dpred) {
  const Range rg = block_rows(n, rows_per);
  const uint32_t vec = (uint32_t)c / 8;
  const float k = stats[3] * upstream;
  const uint32_t e1 = (uint32_t)(rg.r1 - rg.r0) * vec;
  for (uint32_t e = threadIdx.x; e < e1; e += kLossThreads) {
    const uint32_t rr = e / vec;
    const int r = rg.r0 + (int)rr;
    const size_t off = (size_t)r * c + (size_t)(e - rr * vec) * 8;
    float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (ids[r] >= 0) {
      float a[8], b[8];
      load8<T>(pred + off, a);
      load8<T>(target + off, b);
#pragma unroll
      for (int i = 0; i < 8; ++i) g[i] = k * (a[i] - b[i]);
    }
    store8<T>(dpred + off, g);
  }
}

// Largest n * c accepted: keeps every per-block element count in 32 bits.
constexpr int64_t kMaxElems = (int64_t)1 << 36;

int32_t check_loss_args(int32_t dtype, int32_t n, int32_t c, const void* pred, const void* target,
                        const int32_t* ids) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (n < 0 || c < 8 || c % 8 != 0 || (int64_t)n * c > kMaxElems) return PA_ERR_SHAPE;
  if (n > 0 && (!pred || !target || !ids)) return PA_ERR_NULL;
  if (!aligned16(pred) || !aligned16(target)) return PA_ERR_ALIGN;
  return PA_OK;
}

int32_t check_workspace(const void* ws, size_t bytes, int32_t n) {
  if (!ws) return PA_ERR_NULL;
  if (bytes < masked_mse_workspace_bytes(n)) return PA_ERR_WORKSPACE;
  if (!aligned256(ws)) return PA_ERR_ALIGN;
  return PA_OK;
}

int rows_per_block(int32_t n) { return (n + kLossBlocks - 1) / kLossBlocks; }

template <typename T>
void launch_fwd(const void* pred, const void* target, const int32_t* ids, int32_t n, int32_t c,
                float* sse_part, uint32_t* cnt_part, float* stats, hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL((loss_sse_kernel<T, true, false>), dim3(kLossBlocks), dim3(kLossThreads), 0, s,
                       (const T*)pred, (const T*)target, ids, n, c, rows_per_block(n),
                       kLossBlocks, 0.f, sse_part, cnt_part, (T*)nullptr);
  hipLaunchKernelGGL(loss_finish_kernel, dim3(1), dim3(kLossThreads), 0, s, sse_part, cnt_part,
                     n > 0 ? kLossBlocks : 0, c, stats);
}

template <typename T>
void launch_fused(const void* pred, const void* target, const int32_t* ids, int32_t n, int32_t c,
                  float upstream, float* sse_part, uint32_t* cnt_part, float* stats, void* dpred,
                  hipStream_t s) {
  const int rp = rows_per_block(n);
  if (n > 0) {
    hipLaunchKernelGGL(loss_count_kernel, dim3(kLossBlocks), dim3(kLossThreads), 0, s, ids, n, rp,
                       cnt_part);
    hipLaunchKernelGGL((loss_sse_kernel<T, false, true>), dim3(kLossBlocks), dim3(kLossThreads), 0, s,
                       (const T*)pred, (const T*)target, ids, n, c, rp, kLossBlocks, upstream,
                       sse_part, cnt_part, (T*)dpred);
  }
  hipLaunchKernelGGL(loss_finish_kernel, dim3(1), dim3(kLossThreads), 0, s, sse_part, cnt_part,
                     n > 0 ? kLossBlocks : 0, c, stats);
}

}  // namespace

extern "C" size_t masked_mse_workspace_bytes(int32_t n) {
  return n < 0 ? 0 : align_up(kLossBlocks * (sizeof(float) + sizeof(uint32_t)), 256);
}

extern "C" int32_t masked_mse_fwd(int32_t dtype, int32_t n, int32_t c, const void* pred,
                                  const void* target, const int32_t* seq_id, float* stats,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  int32_t st = check_loss_args(dtype, n, c, pred, target, seq_id);
  if (st == PA_OK && !stats) st = PA_ERR_NULL;
  if (st == PA_OK) st = check_workspace(workspace, workspace_bytes, n);
  if (st != PA_OK) return st;
  float* sse_part = (float*)workspace;
  uint32_t* cnt_part = (uint32_t*)(sse_part + kLossBlocks);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == PA_BF16)
    launch_fwd<uint16_t>(pred, target, seq_id, n, c, sse_part, cnt_part, stats, s);
  else
    launch_fwd<float>(pred, target, seq_id, n, c, sse_part, cnt_part, stats, s);
  return launch_status();
}

extern "C" int32_t masked_mse_bwd(int32_t dtype, int32_t n, int32_t c, const void* pred,
                                  const void* target, const int32_t* seq_id, const float* stats,
                                  float upstream, void* dpred, void* stream) {
  int32_t st = check_loss_args(dtype, n, c, pred, target, seq_id);
  if (st == PA_OK && n > 0 && (!stats || !dpred)) st = PA_ERR_NULL;
  if (st == PA_OK && !aligned16(dpred)) st = PA_ERR_ALIGN;
  if (st != PA_OK || n == 0) return st;
  hipStream_t s = (hipStream_t)stream;
  const int rp = rows_per_block(n);
  if (dtype == PA_BF16)
    hipLaunchKernelGGL(loss_grad_kernel<uint16_t>, dim3(kLossBlocks), dim3(kLossThreads), 0, s,
                       (const uint16_t*)pred, (const uint16_t*)target, seq_id, n, c, rp, stats,
                       upstream, (uint16_t*)dpred);
  else
    hipLaunchKernelGGL(loss_grad_kernel<float>, dim3(kLossBlocks), dim3(kLossThreads), 0, s,
                       (const float*)pred, (const float*)target, seq_id, n, c, rp, stats,
                       upstream, (float*)dpred);
  return launch_status();
}

extern "C" int32_t masked_mse_fwd_bwd(int32_t dtype, int32_t n, int32_t c, const void* pred,
                                      const void* target, const int32_t* seq_id, float upstream,
                                      float* stats, void* dpred, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  int32_t st = check_loss_args(dtype, n, c, pred, target, seq_id);
  if (st == PA_OK && (!stats || (n > 0 && !dpred))) st = PA_ERR_NULL;
  if (st == PA_OK && !aligned16(dpred)) st = PA_ERR_ALIGN;
  if (st == PA_OK) st = check_workspace(workspace, workspace_bytes, n);
  if (st != PA_OK) return st;
  float* sse_part = (float*)workspace;
  uint32_t* cnt_part = (uint32_t*)(sse_part + kLossBlocks);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == PA_BF16)
    launch_fused<uint16_t>(pred, target, seq_id, n, c, upstream, sse_part, cnt_part, stats, dpred,
                           s);
  else
    launch_fused<float>(pred, target, seq_id, n, c, upstream, sse_part, cnt_part, stats, dpred, s);
  return launch_status();
}
