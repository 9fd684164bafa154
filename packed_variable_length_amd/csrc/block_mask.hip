// Block-mask builder: classifies every query-tile x key-tile pair of the
// same-seq-id mask as empty, partial or full, and compacts the non-empty pairs
// into CSR lists in both directions.
//
// "LingBot-VA packing" report, sections 1 and 2.2: the packed sequence is
// masked by a block mask built from the seq ids so that blocks without an
// allowed pair are skipped; "Furniture packing, variable length" report,
// implementation part: a pair is allowed iff both ids are equal and not -1.
//
// Pipeline (all on the caller's stream, no host synchronisation):
//   1. tile_summary  one wave per tile of either axis: number of valid tokens and
//                    up to four distinct valid ids (or "more than four").
//   2. classify      one thread per tile pair, 32x32 pairs per block: decides the
//                    class from the two summaries whenever both list all their ids;
//                    otherwise queues the pair.  Writes the class matrix and its
//                    transpose (through LDS, so both writes are coalesced).
//   3. resolve       persistent waves settle queued pairs by an exact scan of the
//                    two tiles' ids (interleaved-id inputs only).
//   4. count         one block per row of the class matrix and of its transpose.
//   5. scan_sort     two blocks: exclusive scan of the counts into CSR row
//                    pointers, and a bitonic sort giving the longest-first order.
//   6. compact       one block per row: ascending column lists via wave ballots.
//   7. pair_compact  one block per pair of query tiles (positions 2w, 2w+1 of the
//                    longest-first order, the pairs the paired attention kernels
//                    run): the ascending union of the two key-tile lists, each
//                    entry the key tile with both tiles' classes packed beside it,
//                    so those kernels walk exactly the key tiles one of the two
//                    query tiles needs.
#include "pa_common.h"

namespace {

constexpr int kMaxTiles = 16384;      // per axis; bounds the sort in LDS
constexpr int kSortThreads = 1024;

struct TileSummary {
  int32_t n_valid;   // tokens with id >= 0
  int32_t n_ids;     // distinct valid ids, 5 = "more than four"
  int32_t ids[4];    // the distinct valid ids (ascending) when n_ids <= 4
  int32_t len;       // tokens in the tile (short for the last tile)
  int32_t pad;
};

__device__ __forceinline__ int wave_sum(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_min(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------- 1. summaries
__global__ void __launch_bounds__(256)
tile_summary_kernel(const int32_t* __restrict__ q_ids, int32_t nq, int32_t bq, int32_t nqt,
                    const int32_t* __restrict__ kv_ids, int32_t nkv, int32_t bkv, int32_t nkt,
                    TileSummary* __restrict__ q_sum, TileSummary* __restrict__ kv_sum,
                    int32_t* __restrict__ queue_count) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w == 0 && lane == 0) *queue_count = 0;
  if (w >= nqt + nkt) return;
  const bool qside = w < nqt;
  const int tile = qside ? w : w - nqt;
  const int32_t* ids = qside ? q_ids : kv_ids;
  const int n = qside ? nq : nkv;
  const int block = qside ? bq : bkv;
  const int start = tile * block;
  const int len = min(block, n - start);

  int cnt = 0;
  for (int i = lane; i < len; i += 64) cnt += ids[start + i] >= 0;
  cnt = wave_sum(cnt);

  TileSummary s;
  s.n_valid = cnt;
  s.n_ids = 0;
  s.ids[0] = s.ids[1] = s.ids[2] = s.ids[3] = -1;
  s.len = len;
  s.pad = 0;
  int lower = -1;  // next distinct id is the smallest id > lower
  for (int r = 0; r < 5; ++r) {
    int mn = INT32_MAX;
    bool any = false;
    for (int i = lane; i < len; i += 64) {
      const int id = ids[start + i];
      if (id > lower) {
        any = true;
        mn = min(mn, id);
      }
    }
    if (__ballot(any) == 0) break;
    mn = wave_min(mn);
    if (r == 4) {
      s.n_ids = 5;
      break;
    }
    s.ids[r] = mn;
    s.n_ids = r + 1;
    lower = mn;
  }
  if (lane == 0) (qside ? q_sum : kv_sum)[tile] = s;
}

// ---------------------------------------------------------------- 2. classify
__global__ void __launch_bounds__(256)
classify_kernel(const TileSummary* __restrict__ q_sum, const TileSummary* __restrict__ kv_sum,
                int32_t nqt, int32_t nkt, int32_t bq, int32_t bkv, uint8_t* __restrict__ cls,
                uint8_t* __restrict__ cls_t, int32_t* __restrict__ queue,
                int32_t* __restrict__ queue_count) {
  __shared__ uint8_t tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int I0 = blockIdx.y * 32, J0 = blockIdx.x * 32;
  const int J = J0 + tx;
  for (int r = 0; r < 4; ++r) {
    const int i = ty + 8 * r;
    const int I = I0 + i;
    uint8_t c = 0;
    if (I < nqt && J < nkt) {
      const TileSummary a = q_sum[I];
      const TileSummary b = kv_sum[J];
      if (a.n_valid == 0 || b.n_valid == 0) {
        c = 0;
      } else if (a.n_ids <= 4 && b.n_ids <= 4) {
        bool common = false;
        for (int x = 0; x < a.n_ids; ++x)
          for (int y = 0; y < b.n_ids; ++y) common |= a.ids[x] == b.ids[y];
        if (!common) {
          c = 0;
        } else if (a.n_ids == 1 && b.n_ids == 1 && a.n_valid == bq && b.n_valid == bkv) {
          c = 2;  // every token of both full-length tiles carries the same id
        } else {
          c = 1;
        }
      } else {
        c = 0;  // settled by resolve_kernel
        const int slot = atomicAdd(queue_count, 1);
        queue[slot] = I * nkt + J;
      }
      cls[(size_t)I * nkt + J] = c;
    }
    tile[i][tx] = c;
  }
  __syncthreads();
  // transposed write: thread tx now walks the query-tile axis
  for (int r = 0; r < 4; ++r) {
    const int j = ty + 8 * r;
    const int Jt = J0 + j, It = I0 + tx;
    if (Jt < nkt && It < nqt) cls_t[(size_t)Jt * nqt + It] = tile[tx][j];
  }
}

// ---------------------------------------------------------------- 3. resolve
// Persistent: each wave takes queued pairs w, w + total_waves, ... until the
// queue is exhausted, so every wave ends.  Key ids of the pair's key tile are
// staged in the wave's LDS slice (at most 1024 ids).
__global__ void __launch_bounds__(256)
resolve_kernel(const int32_t* __restrict__ q_ids, int32_t nq, int32_t bq,
               const int32_t* __restrict__ kv_ids, int32_t nkv, int32_t bkv, int32_t nqt,
               int32_t nkt, const int32_t* __restrict__ queue,
               const int32_t* __restrict__ queue_count, uint8_t* __restrict__ cls,
               uint8_t* __restrict__ cls_t) {
  __shared__ int32_t kbuf[4][1024];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int total_waves = gridDim.x * 4;
  const int count = *queue_count;
  for (int p = blockIdx.x * 4 + wv; p < count; p += total_waves) {
    const int pair = queue[p];
    const int I = pair / nkt, J = pair - I * nkt;
    const int q0 = I * bq, qlen = min(bq, nq - q0);
    const int k0 = J * bkv, klen = min(bkv, nkv - k0);
    for (int j = lane; j < klen; j += 64) kbuf[wv][j] = kv_ids[k0 + j];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    bool found = false;
    for (int i0 = 0; i0 < qlen && !found; i0 += 64) {
      const int i = i0 + lane;
      const int id = i < qlen ? q_ids[q0 + i] : -1;
      bool mine = false;
      if (id >= 0)
        for (int j = 0; j < klen && !mine; ++j) mine = kbuf[wv][j] == id;
      found = __ballot(mine) != 0;
    }
    if (lane == 0) {
      const uint8_t c = found ? 1 : 0;
      cls[(size_t)I * nkt + J] = c;
      cls_t[(size_t)J * nqt + I] = c;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
}

// ---------------------------------------------------------------- 4. count
__global__ void __launch_bounds__(256)
count_kernel(const uint8_t* __restrict__ cls, const uint8_t* __restrict__ cls_t, int32_t nqt,
             int32_t nkt, int32_t* __restrict__ cnt_q, int32_t* __restrict__ cnt_kv) {
  __shared__ int part[4];
  const int row = blockIdx.x;
  const bool qside = row < nqt;
  const uint8_t* src = qside ? cls + (size_t)row * nkt : cls_t + (size_t)(row - nqt) * nqt;
  const int len = qside ? nkt : nqt;
  int c = 0;
  for (int j = threadIdx.x; j < len; j += 256) c += src[j] != 0;
  c = wave_sum(c);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int t = part[0] + part[1] + part[2] + part[3];
    if (qside) cnt_q[row] = t; else cnt_kv[row - nqt] = t;
  }
}

// ---------------------------------------------------------------- 5. scan + sort
// Block 0 handles the query side, block 1 the key side.
__global__ void __launch_bounds__(kSortThreads)
scan_sort_kernel(const int32_t* __restrict__ cnt_q, const int32_t* __restrict__ cnt_kv,
                 int32_t nqt, int32_t nkt, int32_t* __restrict__ q_ptr,
                 int32_t* __restrict__ kv_ptr, int32_t* __restrict__ q_order,
                 int32_t* __restrict__ kv_order, int32_t* __restrict__ pair_off) {
  __shared__ uint32_t keys[kMaxTiles];
  __shared__ int32_t partial[kSortThreads];
  const bool qside = blockIdx.x == 0;
  const int32_t* cnt = qside ? cnt_q : cnt_kv;
  const int n = qside ? nqt : nkt;
  const int other = qside ? nkt : nqt;  // upper bound of a count
  int32_t* ptr = qside ? q_ptr : kv_ptr;
  int32_t* order = qside ? q_order : kv_order;
  const int t = threadIdx.x;

  // exclusive scan: each thread owns a contiguous chunk
  const int chunk = (n + kSortThreads - 1) / kSortThreads;
  const int b0 = t * chunk, b1 = min(n, b0 + chunk);
  int local = 0;
  for (int i = b0; i < b1; ++i) local += cnt[i];
  partial[t] = local;
  __syncthreads();
  for (int o = 1; o < kSortThreads; o <<= 1) {  // Hillis-Steele inclusive scan
    const int v = t >= o ? partial[t - o] : 0;
    __syncthreads();
    partial[t] += v;
    __syncthreads();
  }
  int run = partial[t] - local;
  for (int i = b0; i < b1; ++i) {
    ptr[i] = run;
    run += cnt[i];
  }
  if (t == kSortThreads - 1) ptr[n] = partial[t];

  // longest-first order: sort keys (other - cnt) * n + index ascending
  int P = 1;
  while (P < n) P <<= 1;
  for (int i = t; i < P; i += kSortThreads)
    keys[i] = i < n ? (uint32_t)(other - cnt[i]) * (uint32_t)n + (uint32_t)i : 0xFFFFFFFFu;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = t; i < P; i += kSortThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint32_t a = keys[i], b = keys[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            keys[i] = b;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = t; i < n; i += kSortThreads) order[i] = (int32_t)(keys[i] % (uint32_t)n);
  if (!qside) return;

  // query side: room for each pair's union list (the sum of its two list
  // lengths, an upper bound), as an exclusive scan over the pairs
  const int np = (n + 1) / 2;
  const int pchunk = (np + kSortThreads - 1) / kSortThreads;
  const int p0 = t * pchunk, p1 = min(np, p0 + pchunk);
  const auto cap = [&](int w) {
    const int a = (int)(keys[2 * w] % (uint32_t)n);
    return cnt[a] + (2 * w + 1 < n ? cnt[(int)(keys[2 * w + 1] % (uint32_t)n)] : 0);
  };
  int plocal = 0;
  for (int w = p0; w < p1; ++w) plocal += cap(w);
  __syncthreads();
  partial[t] = plocal;
  __syncthreads();
  for (int o = 1; o < kSortThreads; o <<= 1) {
    const int v = t >= o ? partial[t - o] : 0;
    __syncthreads();
    partial[t] += v;
    __syncthreads();
  }
  int prun = partial[t] - plocal;
  for (int w = p0; w < p1; ++w) {
    pair_off[w] = prun;
    prun += cap(w);
  }
  if (t == kSortThreads - 1) pair_off[np] = partial[t];
}

// ---------------------------------------------------------------- 6. compact
__global__ void __launch_bounds__(256)
compact_kernel(const uint8_t* __restrict__ cls, const uint8_t* __restrict__ cls_t, int32_t nqt,
               int32_t nkt, const int32_t* __restrict__ q_ptr,
               const int32_t* __restrict__ kv_ptr, int32_t* __restrict__ q_cols,
               int32_t* __restrict__ kv_rows) {
  __shared__ int wave_tot[4];
  const int row = blockIdx.x;
  const bool qside = row < nqt;
  const int r = qside ? row : row - nqt;
  const uint8_t* src = qside ? cls + (size_t)r * nkt : cls_t + (size_t)r * nqt;
  const int len = qside ? nkt : nqt;
  int32_t* dst = qside ? q_cols + q_ptr[r] : kv_rows + kv_ptr[r];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int base = 0;
  for (int j0 = 0; j0 < len; j0 += 256) {
    const int j = j0 + threadIdx.x;
    const bool nz = j < len && src[j] != 0;
    const uint64_t m = __ballot(nz);
    if (lane == 0) wave_tot[wv] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wv; ++w) off += wave_tot[w];
    if (nz) dst[off + __popcll(m & lt)] = j;
    base += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    __syncthreads();
  }
}

// ---------------------------------------------------------------- 7. pair lists
// Block w: query tiles a = q_order[2w] and b = q_order[2w + 1] (none past the
// end).  Entry = key tile | class(a, kt) << 16 | class(b, kt) << 24 for every
// key tile at least one of the two rows has an allowed pair with, ascending.
__global__ void __launch_bounds__(256)
pair_compact_kernel(const uint8_t* __restrict__ cls, int32_t nqt, int32_t nkt,
                    const int32_t* __restrict__ q_order, const int32_t* __restrict__ pair_off,
                    int32_t* __restrict__ pair_len, int32_t* __restrict__ pair_ent) {
  __shared__ int wave_tot[4];
  const int w = blockIdx.x;
  const int a = q_order[2 * w];
  const int b = 2 * w + 1 < nqt ? q_order[2 * w + 1] : -1;
  const uint8_t* ra = cls + (size_t)a * nkt;
  const uint8_t* rb = b >= 0 ? cls + (size_t)b * nkt : nullptr;
  int32_t* dst = pair_ent + pair_off[w];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int base = 0;
  for (int j0 = 0; j0 < nkt; j0 += 256) {
    const int j = j0 + threadIdx.x;
    const int ca = j < nkt ? ra[j] : 0;
    const int cb = (j < nkt && rb) ? rb[j] : 0;
    const bool nz = (ca | cb) != 0;
    const uint64_t m = __ballot(nz);
    if (lane == 0) wave_tot[wv] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int x = 0; x < wv; ++x) off += wave_tot[x];
    if (nz) dst[off + __popcll(m & lt)] = j | (ca << 16) | (cb << 24);
    base += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) pair_len[w] = base;
}

struct Layout {
  size_t cls, cls_t, q_ptr, kv_ptr, q_order, kv_order, q_cols, kv_rows, q_sum, kv_sum, cnt_q,
      cnt_kv, queue, queue_count, pair_off, pair_len, pair_ent, total;
};

bool make_layout(int32_t nq, int32_t nkv, int32_t bq, int32_t bkv, Layout* L, int32_t* nqt_out,
                 int32_t* nkt_out) {
  if (nq < 1 || nkv < 1 || bq < 16 || bq > 1024 || bkv < 16 || bkv > 1024) return false;
  const int64_t nqt = ((int64_t)nq + bq - 1) / bq, nkt = ((int64_t)nkv + bkv - 1) / bkv;
  if (nqt > kMaxTiles || nkt > kMaxTiles) return false;
  const size_t pairs = (size_t)nqt * (size_t)nkt;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = pa::align_up(off + bytes, 256);
    return at;
  };
  L->cls = take(pairs);
  L->cls_t = take(pairs);
  L->q_ptr = take((nqt + 1) * 4);
  L->kv_ptr = take((nkt + 1) * 4);
  L->q_order = take(nqt * 4);
  L->kv_order = take(nkt * 4);
  L->q_cols = take(pairs * 4);
  L->kv_rows = take(pairs * 4);
  L->q_sum = take(nqt * sizeof(TileSummary));
  L->kv_sum = take(nkt * sizeof(TileSummary));
  L->cnt_q = take(nqt * 4);
  L->cnt_kv = take(nkt * 4);
  L->queue = take(pairs * 4);
  L->queue_count = take(4);
  const size_t npairs = (size_t)(nqt + 1) / 2;
  L->pair_off = take((npairs + 1) * 4);
  L->pair_len = take(npairs * 4);
  L->pair_ent = take(pairs * 4);
  L->total = off;
  *nqt_out = (int32_t)nqt;
  *nkt_out = (int32_t)nkt;
  return true;
}

}  // namespace

extern "C" size_t build_block_mask_bytes(int32_t nq, int32_t nkv, int32_t block_q,
                                         int32_t block_kv) {
  Layout L;
  int32_t nqt, nkt;
  if (!make_layout(nq, nkv, block_q, block_kv, &L, &nqt, &nkt)) return 0;
  return L.total;
}

extern "C" int32_t build_block_mask(const int32_t* q_seq_id, int32_t nq, const int32_t* kv_seq_id,
                                    int32_t nkv, int32_t block_q, int32_t block_kv, void* storage,
                                    size_t bytes, pa_block_mask* out, void* stream) {
  if (!q_seq_id || !kv_seq_id || !storage || !out) return PA_ERR_NULL;
  Layout L;
  int32_t nqt, nkt;
  if (!make_layout(nq, nkv, block_q, block_kv, &L, &nqt, &nkt)) return PA_ERR_SHAPE;
  if (bytes < L.total) return PA_ERR_WORKSPACE;
  if (!pa::aligned256(storage)) return PA_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)storage;
  uint8_t* cls = (uint8_t*)(base + L.cls);
  uint8_t* cls_t = (uint8_t*)(base + L.cls_t);
  int32_t* q_ptr = (int32_t*)(base + L.q_ptr);
  int32_t* kv_ptr = (int32_t*)(base + L.kv_ptr);
  int32_t* q_order = (int32_t*)(base + L.q_order);
  int32_t* kv_order = (int32_t*)(base + L.kv_order);
  int32_t* q_cols = (int32_t*)(base + L.q_cols);
  int32_t* kv_rows = (int32_t*)(base + L.kv_rows);
  TileSummary* q_sum = (TileSummary*)(base + L.q_sum);
  TileSummary* kv_sum = (TileSummary*)(base + L.kv_sum);
  int32_t* cnt_q = (int32_t*)(base + L.cnt_q);
  int32_t* cnt_kv = (int32_t*)(base + L.cnt_kv);
  int32_t* queue = (int32_t*)(base + L.queue);
  int32_t* queue_count = (int32_t*)(base + L.queue_count);
  int32_t* pair_off = (int32_t*)(base + L.pair_off);
  int32_t* pair_len = (int32_t*)(base + L.pair_len);
  int32_t* pair_ent = (int32_t*)(base + L.pair_ent);

  const int waves = nqt + nkt;
  hipLaunchKernelGGL(tile_summary_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, q_seq_id, nq,
                     block_q, nqt, kv_seq_id, nkv, block_kv, nkt, q_sum, kv_sum, queue_count);
  hipLaunchKernelGGL(classify_kernel, dim3((nkt + 31) / 32, (nqt + 31) / 32), dim3(256), 0, s,
                     q_sum, kv_sum, nqt, nkt, block_q, block_kv, cls, cls_t, queue, queue_count);
  const size_t pairs = (size_t)nqt * nkt;
  const int rblocks = (int)std::min<size_t>((pairs + 3) / 4, 1024);
  hipLaunchKernelGGL(resolve_kernel, dim3(rblocks), dim3(256), 0, s, q_seq_id, nq, block_q,
                     kv_seq_id, nkv, block_kv, nqt, nkt, queue, queue_count, cls, cls_t);
  hipLaunchKernelGGL(count_kernel, dim3(nqt + nkt), dim3(256), 0, s, cls, cls_t, nqt, nkt, cnt_q,
                     cnt_kv);
  hipLaunchKernelGGL(scan_sort_kernel, dim3(2), dim3(kSortThreads), 0, s, cnt_q, cnt_kv, nqt, nkt,
                     q_ptr, kv_ptr, q_order, kv_order, pair_off);
  hipLaunchKernelGGL(compact_kernel, dim3(nqt + nkt), dim3(256), 0, s, cls, cls_t, nqt, nkt, q_ptr,
                     kv_ptr, q_cols, kv_rows);
  hipLaunchKernelGGL(pair_compact_kernel, dim3((nqt + 1) / 2), dim3(256), 0, s, cls, nqt, nkt,
                     q_order, pair_off, pair_len, pair_ent);
  const int32_t st = pa::launch_status();
  if (st != PA_OK) return st;
  out->nq = nq;
  out->nkv = nkv;
  out->block_q = block_q;
  out->block_kv = block_kv;
  out->nq_tiles = nqt;
  out->nkv_tiles = nkt;
  out->tile_class = cls;
  out->q_ptr = q_ptr;
  out->q_cols = q_cols;
  out->kv_ptr = kv_ptr;
  out->kv_rows = kv_rows;
  out->q_order = q_order;
  out->kv_order = kv_order;
  out->pair_off = pair_off;
  out->pair_len = pair_len;
  out->pair_ent = pair_ent;
  return PA_OK;
}
