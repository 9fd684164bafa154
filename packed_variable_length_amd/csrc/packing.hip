// Unpadded packing: episodes concatenated back to back under a token budget.
//
// "LingBot-VA packing" report, section 1: a single episode per micro-step uses a
// small fraction of the roughly 68k-token budget of a GPU; "LingBot-VA attention
// profiling" report, conclusion and next steps: concatenate several episodes
// along the sequence axis and give each token its document id, so the attention
// mask keeps episodes apart with no frame padding at all.
//
// plan_token_packs (host) assigns episodes, in arrival order, to packs: next-fit,
// a pack is closed when the next episode would overflow the budget.
// seq_ids_from_lengths (device) writes the per-token ids of one pack.
#include "pa_common.h"

namespace {

constexpr int kIdThreads = 256;
constexpr int kMaxEpisodes = 8192;  // episode starts held in LDS (32 KB)

// Every block recomputes the episode starts (exclusive prefix sums of the
// lengths, clamped to n_tokens) in LDS: thread i scans a contiguous chunk,
// then the 256 chunk totals are scanned.  Token t then belongs to the last
// episode whose start is <= t (zero-length episodes share their successor's
// start and are never that last one), or to none once t reaches the total.
__global__ void __launch_bounds__(kIdThreads)
ids_from_lengths_kernel(const int32_t* __restrict__ lengths, int32_t B, int32_t n_tokens,
                        int32_t* __restrict__ seq_id, int32_t* __restrict__ offsets) {
  __shared__ int32_t start[kMaxEpisodes];
  __shared__ int64_t part[kIdThreads];
  const int tid = threadIdx.x;
  const int chunk = (B + kIdThreads - 1) / kIdThreads;
  const int e0 = min(B, tid * chunk), e1 = min(B, e0 + chunk);
  int64_t s = 0;
  for (int e = e0; e < e1; ++e) s += max(lengths[e], 0);
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int64_t run = 0;
    for (int i = 0; i < kIdThreads; ++i) {
      const int64_t v = part[i];
      part[i] = run;
      run += v;
    }
  }
  __syncthreads();
  int64_t run = part[tid];
  for (int e = e0; e < e1; ++e) {
    start[e] = (int32_t)min<int64_t>(run, n_tokens);
    run += max(lengths[e], 0);
  }
  __shared__ int32_t total_s;
  if (tid == kIdThreads - 1) total_s = (int32_t)min<int64_t>(run, n_tokens);
  // the last thread's chunk may be empty: its run is then the grand total too
  __syncthreads();
  const int32_t total = total_s;
  if (offsets != nullptr && blockIdx.x == 0) {
    for (int e = tid; e < B; e += kIdThreads) offsets[e] = start[e];
    if (tid == 0) offsets[B] = total;
  }
  for (int64_t t = (int64_t)blockIdx.x * kIdThreads + tid; t < n_tokens;
       t += (int64_t)gridDim.x * kIdThreads) {
    int id = -1;
    if (t < total) {
      int lo = 0, hi = B;  // first index with start > t is in [lo, hi]
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (start[mid] <= t) lo = mid + 1;
        else hi = mid;
      }
      id = lo - 1;
    }
    seq_id[t] = id;
  }
}

}  // namespace

extern "C" int32_t seq_ids_from_lengths(const int32_t* lengths, int32_t B, int32_t n_tokens,
                                        int32_t* seq_id, int32_t* offsets, void* stream) {
  if (B < 0 || B > kMaxEpisodes || n_tokens < 0) return PA_ERR_SHAPE;
  if ((B > 0 && !lengths) || (n_tokens > 0 && !seq_id)) return PA_ERR_NULL;
  if (n_tokens == 0 && offsets == nullptr) return PA_OK;
  const int64_t want = ((int64_t)n_tokens + 4 * kIdThreads - 1) / (4 * kIdThreads);
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(want, 1024));
  hipLaunchKernelGGL(ids_from_lengths_kernel, dim3(blocks), dim3(kIdThreads), 0,
                     (hipStream_t)stream, lengths, B, n_tokens, seq_id, offsets);
  return pa::launch_status();
}

extern "C" int32_t plan_token_packs(const int32_t* lengths, int32_t B, int64_t budget,
                                    int32_t* pack_of, int32_t* n_packs) {
  if (B < 0 || budget < 1) return PA_ERR_SHAPE;
  if (!n_packs || (B > 0 && (!lengths || !pack_of))) return PA_ERR_NULL;
  for (int32_t e = 0; e < B; ++e)
    if (lengths[e] < 0 || lengths[e] > budget) return PA_ERR_SHAPE;
  int32_t packs = 0;
  int64_t used = 0;
  for (int32_t e = 0; e < B; ++e) {
    if (packs == 0 || used + lengths[e] > budget) {
      ++packs;
      used = 0;
    }
    pack_of[e] = packs - 1;
    used += lengths[e];
  }
  *n_packs = packs;
  return PA_OK;
}
