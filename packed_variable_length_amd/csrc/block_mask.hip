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
//                    up to four distinct valid ids (or "more than four"); also
//                    clears the row counts.
//   2. classify      64 x 64 tile pairs per block, the 128 summaries staged in
//                    LDS: decides the class from the two summaries whenever both
//                    list all their ids, otherwise queues the pair.  Each thread
//                    classifies 16 pairs of one row of the class matrix and writes
//                    them as one 16-byte store, then 16 of its transpose the same
//                    way, and adds its rows' non-empty counts (one atomic each).
//   3. resolve       persistent waves settle queued pairs by an exact scan of the
//                    two tiles' ids (interleaved-id inputs only), and count them.
//   4. scan_sort     two blocks: exclusive scan of the counts into CSR row
//                    pointers (shuffle scans per wave), and a bitonic sort giving
//                    the longest-first order (partner distances below 128 in
//                    registers, the rest through LDS).
//   5. lists         one launch, two kinds of block.  One block per row:
//                    ascending column lists, 16 classes per thread per pass,
//                    positions from a block-wide prefix sum.  One block per
//                    pair of query tiles (positions 2w, 2w+1 of the
//                    longest-first order, the pairs the paired attention kernels
//                    run): the ascending union of the two key-tile lists, each
//                    entry the key tile with both tiles' classes packed beside it,
//                    so those kernels walk exactly the key tiles one of the two
//                    query tiles needs.
#include "pa_common.h"

namespace {

using pa::u32x4;

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
                    int32_t* __restrict__ queue_count, int32_t* __restrict__ cnt_q,
                    int32_t* __restrict__ cnt_kv) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w == 0 && lane == 0) *queue_count = 0;
  if (w >= nqt + nkt) return;
  const bool qside = w < nqt;
  const int tile = qside ? w : w - nqt;
  if (lane == 0) (qside ? cnt_q : cnt_kv)[tile] = 0;
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
constexpr int kAmbiguous = -1;

// Class of a tile pair from the two summaries, or kAmbiguous when a tile holds
// more than four distinct ids (the exact scan of resolve_kernel decides).
__device__ __forceinline__ int pair_class(const TileSummary& a, const TileSummary& b, int bq,
                                          int bkv) {
  if (a.n_valid == 0 || b.n_valid == 0) return 0;
  if (a.n_ids > 4 || b.n_ids > 4) return kAmbiguous;
  bool common = false;
  for (int x = 0; x < a.n_ids; ++x)
    for (int y = 0; y < b.n_ids; ++y) common |= a.ids[x] == b.ids[y];
  if (!common) return 0;
  // full: one id on both sides and every position of both full-length tiles valid
  return (a.n_ids == 1 && b.n_ids == 1 && a.n_valid == bq && b.n_valid == bkv) ? 2 : 1;
}

// 16 class bytes to dst[0 .. count) (count <= 16): one 16-byte store when the
// run is whole and aligned, word stores when word-aligned, else bytes.
__device__ __forceinline__ void store_classes(uint8_t* dst, const uint32_t (&w)[4], int count) {
  const uintptr_t a = (uintptr_t)dst;
  if (count == 16 && (a & 15) == 0) {
    *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
  } else if ((a & 3) == 0) {
    int k = 0;
    for (; k + 4 <= count; k += 4) *(uint32_t*)(dst + k) = w[k >> 2];
    for (; k < count; ++k) dst[k] = (uint8_t)(w[k >> 2] >> (8 * (k & 3)));
  } else {
    for (int k = 0; k < count; ++k) dst[k] = (uint8_t)(w[k >> 2] >> (8 * (k & 3)));
  }
}

// Block = 64 query tiles x 64 key tiles.  Thread t classifies row t / 4, columns
// 16 (t % 4) .. + 15 of the class matrix (queueing ambiguous pairs), then column
// t / 4, rows 16 (t % 4) .. + 15 for the transpose (ambiguous pairs written 0
// in both, settled by resolve_kernel).  The four threads of a row add their
// non-empty counts with one atomic.
// A tile's summary as one code: its id (>= 0) when it holds exactly one id
// below 2^30 (plus 1 << 30 when every position of a full-length tile carries
// it), -1 when it holds no valid token, -2 otherwise (pair_class on the full
// summaries).
__device__ __forceinline__ int tile_code(const TileSummary& a, int block) {
  if (a.n_valid == 0) return -1;
  if (a.n_ids != 1 || a.ids[0] >= (1 << 30)) return -2;
  return a.ids[0] | (a.n_valid == block ? (1 << 30) : 0);
}

__device__ __forceinline__ int code_class(int ca, int cb, const TileSummary& a,
                                          const TileSummary& b, int bq, int bkv) {
  if ((ca | cb) >= 0) {  // one id on each side
    if (((ca ^ cb) & ~(1 << 30)) != 0) return 0;
    return (ca & cb & (1 << 30)) ? 2 : 1;
  }
  if (ca == -1 || cb == -1) return 0;
  return pair_class(a, b, bq, bkv);
}

__global__ void __launch_bounds__(256)
classify_kernel(const TileSummary* __restrict__ q_sum, const TileSummary* __restrict__ kv_sum,
                int32_t nqt, int32_t nkt, int32_t bq, int32_t bkv, uint8_t* __restrict__ cls,
                uint8_t* __restrict__ cls_t, int32_t* __restrict__ queue,
                int32_t* __restrict__ queue_count, int32_t* __restrict__ cnt_q,
                int32_t* __restrict__ cnt_kv) {
  __shared__ TileSummary sq[64], sk[64];
  __shared__ int cq[64], ck[64];
  const int t = threadIdx.x;
  const int I0 = blockIdx.y * 64, J0 = blockIdx.x * 64;
  if (t < 64 && I0 + t < nqt) {
    sq[t] = q_sum[I0 + t];
    cq[t] = tile_code(sq[t], bq);
  }
  if (t >= 64 && t < 128 && J0 + t - 64 < nkt) {
    sk[t - 64] = kv_sum[J0 + t - 64];
    ck[t - 64] = tile_code(sk[t - 64], bkv);
  }
  __syncthreads();
  const int r = t >> 2, c0 = 16 * (t & 3);
  // rows of the class matrix
  {
    const int I = I0 + r;
    const int cnt = I < nqt ? min(16, nkt - (J0 + c0)) : 0;
    uint32_t w[4] = {0, 0, 0, 0};
    int nz = 0;
    const int ca = cnt > 0 ? cq[r] : 0;
    for (int k = 0; k < cnt; ++k) {
      int c = code_class(ca, ck[c0 + k], sq[r], sk[c0 + k], bq, bkv);
      if (c == kAmbiguous) {
        const int slot = atomicAdd(queue_count, 1);
        queue[slot] = I * nkt + J0 + c0 + k;
        c = 0;
      }
      nz += c != 0;
      w[k >> 2] |= (uint32_t)c << (8 * (k & 3));
    }
    if (cnt > 0) store_classes(cls + (size_t)I * nkt + J0 + c0, w, cnt);
    nz += __shfl_xor(nz, 1, 64);
    nz += __shfl_xor(nz, 2, 64);
    if ((t & 3) == 0 && I < nqt && nz) atomicAdd(&cnt_q[I], nz);
  }
  // rows of the transpose
  {
    const int J = J0 + r;
    const int cnt = J < nkt ? min(16, nqt - (I0 + c0)) : 0;
    uint32_t w[4] = {0, 0, 0, 0};
    int nz = 0;
    const int cb = cnt > 0 ? ck[r] : 0;
    for (int k = 0; k < cnt; ++k) {
      int c = code_class(cq[c0 + k], cb, sq[c0 + k], sk[r], bq, bkv);
      if (c == kAmbiguous) c = 0;
      nz += c != 0;
      w[k >> 2] |= (uint32_t)c << (8 * (k & 3));
    }
    if (cnt > 0) store_classes(cls_t + (size_t)J * nqt + I0 + c0, w, cnt);
    nz += __shfl_xor(nz, 1, 64);
    nz += __shfl_xor(nz, 2, 64);
    if ((t & 3) == 0 && J < nkt && nz) atomicAdd(&cnt_kv[J], nz);
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
               uint8_t* __restrict__ cls_t, int32_t* __restrict__ cnt_q,
               int32_t* __restrict__ cnt_kv) {
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
      if (found) {
        atomicAdd(&cnt_q[I], 1);
        atomicAdd(&cnt_kv[J], 1);
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
}

// ---------------------------------------------------------------- 4. scan + sort
// Exclusive prefix of v over the kSortThreads threads (total in *total): a
// shuffle scan inside each wave, then the wave totals (two barriers).
constexpr int kSortWaves = kSortThreads / 64;
__device__ __forceinline__ int sort_block_exclusive(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int off = incl - v, tot = 0;
  for (int x = 0; x < kSortWaves; ++x) {
    const int w = wsum[x];
    off += x < wv ? w : 0;
    tot += w;
  }
  *total = tot;
  __syncthreads();  // wsum is rewritten by the next scan
  return off;
}

// Compare-exchange of a bitonic stage (block size k, partner distance j) on the
// element at position pos holding a, whose partner holds b: the lower element
// of an ascending pair keeps the minimum.
__device__ __forceinline__ uint32_t bitonic_keep(uint32_t a, uint32_t b, int pos, int j, int k) {
  const bool lower = (pos & j) == 0, up = (pos & k) == 0;
  return lower == up ? min(a, b) : max(a, b);
}

// Ascending bitonic sort of keys[0 .. P) in LDS, P a power of two.  Stages
// whose partner distance j is >= 128 exchange through LDS (one barrier each);
// the rest run in registers: a wave holds a 128-key block, lane l the keys at
// l and l + 64 (so j = 64 pairs a lane's two keys and j < 64 is a shuffle).
__device__ void bitonic_sort(uint32_t* keys, int P) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int nblk = P >= 128 ? P / 128 : 0;
  // in-register stages for the block sizes kfirst .. klast (powers of two),
  // each with its distances min(k / 2, 64) .. 1
  const auto reg_stages = [&](int kfirst, int klast) {
    for (int b = wv; b < nblk; b += kSortWaves) {
      const int base = b * 128;
      uint32_t e0 = keys[base + lane], e1 = keys[base + 64 + lane];
      for (int kb = kfirst; kb <= klast; kb <<= 1) {
        for (int j = min(kb >> 1, 64); j > 0; j >>= 1) {
          if (j == 64) {
            const bool up = ((base + lane) & kb) == 0;
            const uint32_t lo = min(e0, e1), hi = max(e0, e1);
            e0 = up ? lo : hi;
            e1 = up ? hi : lo;
          } else {
            const uint32_t p0 = (uint32_t)__shfl_xor((int)e0, j, 64);
            const uint32_t p1 = (uint32_t)__shfl_xor((int)e1, j, 64);
            e0 = bitonic_keep(e0, p0, base + lane, j, kb);
            e1 = bitonic_keep(e1, p1, base + 64 + lane, j, kb);
          }
        }
      }
      keys[base + lane] = e0;
      keys[base + 64 + lane] = e1;
    }
    __syncthreads();
  };
  if (P < 128) {  // small: the plain network through LDS
    for (int k = 2; k <= P; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int p = t; p < (P >> 1); p += kSortThreads) {
          const int i = ((p & ~(j - 1)) << 1) | (p & (j - 1));
          const uint32_t a = keys[i], b = keys[i + j];
          if ((a > b) == ((i & k) == 0)) {
            keys[i] = b;
            keys[i + j] = a;
          }
        }
        __syncthreads();
      }
    return;
  }
  reg_stages(2, 128);  // block sizes 2 .. 128, all in registers
  for (int k = 256; k <= P; k <<= 1) {
    for (int j = k >> 1; j >= 128; j >>= 1) {
      for (int p = t; p < (P >> 1); p += kSortThreads) {
        const int i = ((p & ~(j - 1)) << 1) | (p & (j - 1));
        const uint32_t a = keys[i], b = keys[i + j];
        if ((a > b) == ((i & k) == 0)) {
          keys[i] = b;
          keys[i + j] = a;
        }
      }
      __syncthreads();
    }
    reg_stages(k, k);
  }
}

// Block 0 handles the query side, block 1 the key side.
__global__ void __launch_bounds__(kSortThreads)
scan_sort_kernel(const int32_t* __restrict__ cnt_q, const int32_t* __restrict__ cnt_kv,
                 int32_t nqt, int32_t nkt, int32_t* __restrict__ q_ptr,
                 int32_t* __restrict__ kv_ptr, int32_t* __restrict__ q_order,
                 int32_t* __restrict__ kv_order, int32_t* __restrict__ pair_off) {
  __shared__ uint32_t keys[kMaxTiles];
  __shared__ int wsum[kSortWaves];
  const bool qside = blockIdx.x == 0;
  const int32_t* cnt = qside ? cnt_q : cnt_kv;
  const int n = qside ? nqt : nkt;
  const int other = qside ? nkt : nqt;  // upper bound of a count
  int32_t* ptr = qside ? q_ptr : kv_ptr;
  int32_t* order = qside ? q_order : kv_order;
  const int t = threadIdx.x;

  // exclusive scan of the counts: each thread owns a contiguous chunk
  const int chunk = (n + kSortThreads - 1) / kSortThreads;
  const int b0 = t * chunk, b1 = min(n, b0 + chunk);
  int local = 0;
  for (int i = b0; i < b1; ++i) local += cnt[i];
  int total;
  int run = sort_block_exclusive(local, wsum, &total);
  for (int i = b0; i < b1; ++i) {
    ptr[i] = run;
    run += cnt[i];
  }
  if (t == 0) ptr[n] = total;

  // longest-first order: sort keys (other - cnt) << 14 | index ascending (index
  // < 16384 = kMaxTiles, count <= other <= 16384: 29 bits)
  int P = 1;
  while (P < n) P <<= 1;
  for (int i = t; i < P; i += kSortThreads)
    keys[i] = i < n ? ((uint32_t)(other - cnt[i]) << 14) | (uint32_t)i : 0xFFFFFFFFu;
  __syncthreads();
  bitonic_sort(keys, P);
  for (int i = t; i < n; i += kSortThreads) order[i] = (int32_t)(keys[i] & 0x3FFFu);
  if (!qside) return;

  // query side: room for each pair's union list (the sum of its two list
  // lengths, an upper bound), as an exclusive scan over the pairs
  const int np = (n + 1) / 2;
  const int pchunk = (np + kSortThreads - 1) / kSortThreads;
  const int p0 = t * pchunk, p1 = min(np, p0 + pchunk);
  const auto cap = [&](int w) {
    const int a = (int)(keys[2 * w] & 0x3FFFu);
    return cnt[a] + (2 * w + 1 < n ? cnt[(int)(keys[2 * w + 1] & 0x3FFFu)] : 0);
  };
  int plocal = 0;
  for (int w = p0; w < p1; ++w) plocal += cap(w);
  int ptotal;
  int prun = sort_block_exclusive(plocal, wsum, &ptotal);
  for (int w = p0; w < p1; ++w) {
    pair_off[w] = prun;
    prun += cap(w);
  }
  if (t == 0) pair_off[np] = ptotal;
}

// ---------------------------------------------------------------- 5. compact
// Bytes src[j .. j + 16) of a row of `len` bytes as four words (bytes past the
// row read as 0): one 16-byte load when whole and aligned.
__device__ __forceinline__ void load_classes(const uint8_t* __restrict__ src, int j, int len,
                                             uint32_t (&w)[4]) {
  const uint8_t* p = src + j;
  if (j + 16 <= len && ((uintptr_t)p & 15) == 0) {
    const u32x4 v = *(const u32x4*)p;
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    return;
  }
  w[0] = w[1] = w[2] = w[3] = 0;
  for (int k = 0; k < 16 && j + k < len; ++k) w[k >> 2] |= (uint32_t)p[k] << (8 * (k & 3));
}

__device__ __forceinline__ int class_byte(const uint32_t (&w)[4], int k) {
  return (int)((w[k >> 2] >> (8 * (k & 3))) & 0xFFu);
}

// Exclusive prefix over the block's 256 threads of v (pass total in *total).
__device__ __forceinline__ int block_exclusive(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int off = incl - v;
  for (int x = 0; x < wv; ++x) off += wsum[x];
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();  // wsum is rewritten by the next pass
  return off;
}

// One block per row of the class matrix (key-tile lists) or of its transpose
// (query-tile lists); thread t takes 16 consecutive tiles per pass.
__device__ __forceinline__ void compact_row(const uint8_t* __restrict__ cls,
                                            const uint8_t* __restrict__ cls_t, int32_t nqt,
                                            int32_t nkt, const int32_t* __restrict__ q_ptr,
                                            const int32_t* __restrict__ kv_ptr,
                                            int32_t* __restrict__ q_cols,
                                            int32_t* __restrict__ kv_rows, int row, int* wsum) {
  const bool qside = row < nqt;
  const int r = qside ? row : row - nqt;
  const uint8_t* src = qside ? cls + (size_t)r * nkt : cls_t + (size_t)r * nqt;
  const int len = qside ? nkt : nqt;
  int32_t* dst = qside ? q_cols + q_ptr[r] : kv_rows + kv_ptr[r];
  int base = 0;
  for (int j0 = 0; j0 < len; j0 += 4096) {
    const int j = j0 + 16 * threadIdx.x;
    uint32_t w[4];
    load_classes(src, j, len, w);
    int nz = 0;
    for (int k = 0; k < 16; ++k) nz += class_byte(w, k) != 0;
    int total;
    int off = base + block_exclusive(nz, wsum, &total);
    for (int k = 0; k < 16; ++k)
      if (class_byte(w, k) != 0) dst[off++] = j + k;
    base += total;
  }
}

// ---------------------------------------------------------------- 6. pair lists
// Block w: query tiles a = q_order[2w] and b = q_order[2w + 1] (none past the
// end).  Entry = key tile | class(a, kt) << 16 | class(b, kt) << 24 for every
// key tile at least one of the two rows has an allowed pair with, ascending.
__device__ __forceinline__ void pair_row(const uint8_t* __restrict__ cls, int32_t nqt, int32_t nkt,
                                         const int32_t* __restrict__ q_order,
                                         const int32_t* __restrict__ pair_off,
                                         int32_t* __restrict__ pair_len,
                                         int32_t* __restrict__ pair_ent, int w, int* wsum) {
  const int a = q_order[2 * w];
  const int b = 2 * w + 1 < nqt ? q_order[2 * w + 1] : -1;
  const uint8_t* ra = cls + (size_t)a * nkt;
  const uint8_t* rb = b >= 0 ? cls + (size_t)b * nkt : nullptr;
  int32_t* dst = pair_ent + pair_off[w];
  int base = 0;
  for (int j0 = 0; j0 < nkt; j0 += 4096) {
    const int j = j0 + 16 * threadIdx.x;
    uint32_t wa[4], wb[4] = {0, 0, 0, 0};
    load_classes(ra, j, nkt, wa);
    if (rb) load_classes(rb, j, nkt, wb);
    int nz = 0;
    for (int k = 0; k < 16; ++k) nz += (class_byte(wa, k) | class_byte(wb, k)) != 0;
    int total;
    int off = base + block_exclusive(nz, wsum, &total);
    for (int k = 0; k < 16; ++k) {
      const int ca = class_byte(wa, k), cb = class_byte(wb, k);
      if (ca | cb) dst[off++] = (j + k) | (ca << 16) | (cb << 24);
    }
    base += total;
  }
  if (threadIdx.x == 0) pair_len[w] = base;
}

// Both kinds of list in one launch: blocks 0 .. nqt + nkt - 1 compact a row of
// the class matrix or of its transpose, the next (nqt + 1) / 2 the pair lists.
__global__ void __launch_bounds__(256)
lists_kernel(const uint8_t* __restrict__ cls, const uint8_t* __restrict__ cls_t, int32_t nqt,
             int32_t nkt, const int32_t* __restrict__ q_ptr, const int32_t* __restrict__ kv_ptr,
             int32_t* __restrict__ q_cols, int32_t* __restrict__ kv_rows,
             const int32_t* __restrict__ q_order, const int32_t* __restrict__ pair_off,
             int32_t* __restrict__ pair_len, int32_t* __restrict__ pair_ent) {
  __shared__ int wsum[4];
  const int b = blockIdx.x;
  if (b < nqt + nkt)
    compact_row(cls, cls_t, nqt, nkt, q_ptr, kv_ptr, q_cols, kv_rows, b, wsum);
  else
    pair_row(cls, nqt, nkt, q_order, pair_off, pair_len, pair_ent, b - nqt - nkt, wsum);
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
                     block_q, nqt, kv_seq_id, nkv, block_kv, nkt, q_sum, kv_sum, queue_count,
                     cnt_q, cnt_kv);
  hipLaunchKernelGGL(classify_kernel, dim3((nkt + 63) / 64, (nqt + 63) / 64), dim3(256), 0, s,
                     q_sum, kv_sum, nqt, nkt, block_q, block_kv, cls, cls_t, queue, queue_count,
                     cnt_q, cnt_kv);
  const size_t pairs = (size_t)nqt * nkt;
  const int rblocks = (int)std::min<size_t>((pairs + 3) / 4, 1024);
  hipLaunchKernelGGL(resolve_kernel, dim3(rblocks), dim3(256), 0, s, q_seq_id, nq, block_q,
                     kv_seq_id, nkv, block_kv, nqt, nkt, queue, queue_count, cls, cls_t, cnt_q,
                     cnt_kv);
  hipLaunchKernelGGL(scan_sort_kernel, dim3(2), dim3(kSortThreads), 0, s, cnt_q, cnt_kv, nqt, nkt,
                     q_ptr, kv_ptr, q_order, kv_order, pair_off);
  hipLaunchKernelGGL(lists_kernel, dim3(nqt + nkt + (nqt + 1) / 2), dim3(256), 0, s, cls, cls_t,
                     nqt, nkt, q_ptr, kv_ptr, q_cols, kv_rows, q_order, pair_off, pair_len,
                     pair_ent);
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
