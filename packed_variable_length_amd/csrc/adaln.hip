// AdaLN on a packed sequence: LayerNorm over the feature dimension followed by a
// per-segment modulation, forward and backward, for gfx950.
//
// AdaptiveLoad summary, section 2B (fused LayerNorm-Modulate kernel): the row
// statistics stay on chip, the modulation is applied while the row is still in
// registers, and the backward's modulation-gradient reduction over the sequence
// is organised by feature tiles (a thread owns fixed feature columns and
// accumulates down a tile of rows) so every access is a contiguous row read.
//
//   xhat = (x - mean) * rstd,  rstd = 1 / sqrt(var + eps)   (biased variance)
//   y    = xhat * (1 + scale[s]) + shift[s]                  (s = segment of the row)
//   g    = dy * (1 + scale[s])
//   dx   = rstd * (g - mean_D(g) - xhat * mean_D(g * xhat))
//   d_scale[s] = sum over the valid rows of s of dy * xhat,  d_shift[s] = sum of dy
// Segment s covers rows offsets[s] .. offsets[s+1]-1; a row is valid iff it lies
// in a segment and its seq id is >= 0.  Invalid rows: y = dx = 0, mean = rstd = 0.
//
// Layout: NP = ceil(D / 512) passes of 512 features; lane l holds features
// 512*p + 8*l .. +7 of pass p, so a row slice is a fully coalesced 1 KB (bf16)
// wave load.  The forward gives a whole row to one wave; the backward gives
// pass p of every row to wave p of a workgroup (see below).
//
// Backward: rows are processed as in the forward; d_scale and d_shift
// accumulate in per-lane registers down each workgroup's rows (every lane owns
// fixed feature columns) and are written once per (workgroup, segment) pair; a
// second kernel adds each segment's pairs in workgroup order.  Every sum has a
// fixed order: results are bitwise reproducible.
#include "pa_common.h"

namespace {

using namespace pa;

constexpr int kMaxSeg = 2048;   // segments (offsets live in LDS)
constexpr int kMaxPasses = 8;   // D <= 4096
constexpr int kRedThreads = 1024;
constexpr int kRedCols = 64;    // columns per reduction workgroup (16 threads x 4)
constexpr int kRedLanes = kRedThreads / (kRedCols / 4);  // tiles summed in parallel

// ---------------------------------------------------------------- helpers
// Inclusive scan of v[0..m) in LDS (a running sum, or a running maximum with
// MAX), done by the first wave: lane l scans a contiguous chunk, a shuffle scan
// over the 64 chunk totals gives each lane its prefix, which it then applies.
// Every thread of the workgroup calls it (it ends with a barrier).
template <bool MAX>
__device__ void lds_scan(int32_t* v, int m) {
  if (threadIdx.x < 64) {
    const int l = threadIdx.x, ch = (m + 63) / 64;
    const int a = min(m, l * ch), b = min(m, a + ch);
    const int32_t id = MAX ? INT32_MIN : 0;
    int32_t run = id;
    for (int i = a; i < b; ++i) {
      run = MAX ? max(run, v[i]) : run + v[i];
      v[i] = run;
    }
    int32_t incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t t = __shfl_up(incl, o, 64);
      if (l >= o) incl = MAX ? max(incl, t) : incl + t;
    }
    int32_t pre = __shfl_up(incl, 1, 64);
    if (l == 0) pre = id;
    for (int i = a; i < b; ++i) v[i] = MAX ? max(pre, v[i]) : pre + v[i];
  }
  __syncthreads();
}

// off[0..S] <- offsets clamped into [0, n] and made non-decreasing (running max),
// so segments are disjoint row ranges inside the tensor whatever the input.
template <int NT>
__device__ void load_offsets(const int32_t* __restrict__ g, int S, int n, int32_t* off) {
  for (int i = threadIdx.x; i <= S; i += NT) off[i] = min(max(g[i], 0), n);
  __syncthreads();
  lds_scan<true>(off, S + 1);
}

// Last index j in [0, m) with v[j] <= x (v non-decreasing, v[0] <= x), else -1.
__device__ __forceinline__ int last_le(const int32_t* v, int m, int64_t x) {
  int lo = 0, hi = m;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (v[mid] <= x) lo = mid + 1;
    else hi = mid;
  }
  return lo - 1;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
struct Row8;
template <>
struct Row8<uint16_t> {  // 8 bf16 values = 4 dwords
  u32x4 r;
  // rows are read once: non-temporal (streaming) loads and stores
  // (forward 86 -> 82 us, backward 139 -> 133 us on 36,864 x 3072)
  __device__ __forceinline__ void load(const uint16_t* p) {
    r = __builtin_nontemporal_load((const u32x4*)p);
  }
  // opaque to the optimizer: values derived from r are recomputed after this
  __device__ __forceinline__ void launder() { asm volatile("" : "+v"(r)); }
  __device__ __forceinline__ float at(int j) const {
    const uint32_t w = r[j >> 1];
    return bf16_bits_to_f32((j & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
};
template <>
struct Row8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *(const f32x4*)p;
    b = *(const f32x4*)(p + 4);
  }
  __device__ __forceinline__ float at(int j) const { return j < 4 ? a[j] : b[j - 4]; }
  __device__ __forceinline__ void launder() { asm volatile("" : "+v"(a), "+v"(b)); }
};

__device__ __forceinline__ void store8(uint16_t* p, const float* f) {
  u32x4 a;
#pragma unroll
  for (int w = 0; w < 4; ++w) a[w] = pack_bf16x2(f[2 * w], f[2 * w + 1]);
  __builtin_nontemporal_store(a, (u32x4*)p);
}
__device__ __forceinline__ void store8(float* p, const float* f) {
  *(f32x4*)p = f32x4{f[0], f[1], f[2], f[3]};
  *(f32x4*)(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
}
__device__ __forceinline__ void load8f(const float* p, float* f) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = a[j];
    f[4 + j] = b[j];
  }
}

// ---------------------------------------------------------------- forward
// One wave per row, lane l holding the 8 features 512*p + 8*l .. of every pass
// p < NP, so a row is NP coalesced 1 KB (bf16) wave loads kept in registers
// for the two passes (mean, then variance).  No barrier in the row loop: the
// next row's loads are issued before the current row is reduced, so two rows
// per wave are in flight.  The workgroup takes a contiguous range of rows and
// cuts it into pieces that lie in one segment and span at most kPiece rows;
// for each piece it stages the segment's modulation slice (1 + scale, shift)
// and the rows' validity in LDS, then its 4 waves take every 4th row.
constexpr int kFwdWaves = 4;
constexpr int kPiece = 256;

template <typename T, int NP>
__global__ void __launch_bounds__(64 * kFwdWaves)
adaln_fwd_kernel(const T* __restrict__ x, const int32_t* __restrict__ ids,
                 const int32_t* __restrict__ offsets, int32_t S, int32_t n, int32_t D, float eps,
                 const float* __restrict__ shift, const float* __restrict__ scale,
                 T* __restrict__ y, float* __restrict__ mean_out, float* __restrict__ rstd_out) {
  constexpr int NT = 64 * kFwdWaves;
  extern __shared__ int32_t lds[];
  float* msc = (float*)lds;               // [D] 1 + scale of the piece's segment
  float* msh = msc + D;                   // [D] shift
  int32_t* okr = (int32_t*)(msh + D);     // [kPiece] row validity
  int32_t* off = okr + kPiece;            // [S + 1]
  load_offsets<NT>(offsets, S, n, off);
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const float inv_d = 1.0f / (float)D;
  const int i0 = (int)((int64_t)blockIdx.x * n / gridDim.x);
  const int i1 = (int)((int64_t)(blockIdx.x + 1) * n / gridDim.x);
  const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int seg = last_le(off, S + 1, i0);
  for (int p0 = i0; p0 < i1;) {
    // piece [p0, p1): one segment (or none), at most kPiece rows
    while (seg < S && p0 >= off[seg + 1]) ++seg;
    const bool in_seg = seg >= 0 && seg < S;
    const int seg_end = seg < 0 ? off[0] : (seg < S ? off[seg + 1] : n);
    const int p1 = min(min(i1, p0 + kPiece), seg_end);
    if (in_seg) {
      for (int j = 4 * threadIdx.x; j < D; j += 4 * NT) {
        const f32x4 a = *(const f32x4*)(scale + (size_t)seg * D + j);
        const f32x4 b = *(const f32x4*)(shift + (size_t)seg * D + j);
        *(f32x4*)(msc + j) = a + 1.0f;
        *(f32x4*)(msh + j) = b;
      }
      for (int r = threadIdx.x; r < p1 - p0; r += NT) okr[r] = ids[p0 + r] >= 0 ? 1 : 0;
    }
    __syncthreads();
    if (!in_seg) {  // rows in no segment: zeros
      for (int i = p0 + wv; i < p1; i += kFwdWaves) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int c = 512 * p + 8 * lane;
          if (c < D) store8(y + (size_t)i * D + c, z);
        }
        if (lane == 0) {
          mean_out[i] = 0.f;
          rstd_out[i] = 0.f;
        }
      }
    } else {
      Row8<T> xv[NP], xn[NP];
      int i = p0 + wv;
      bool ok_n = i < p1 && okr[i - p0] != 0;
      if (ok_n) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int c = 512 * p + 8 * lane;
          if (c < D) xn[p].load(x + (size_t)i * D + c);
        }
      }
      for (; i < p1; i += kFwdWaves) {
        const bool ok = ok_n;
#pragma unroll
        for (int p = 0; p < NP; ++p) xv[p] = xn[p];
        const int inx = i + kFwdWaves;
        ok_n = inx < p1 && okr[inx - p0] != 0;
        if (ok_n) {
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const int c = 512 * p + 8 * lane;
            if (c < D) xn[p].load(x + (size_t)inx * D + c);
          }
        }
        T* yr = y + (size_t)i * D;
        if (!ok) {
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const int c = 512 * p + 8 * lane;
            if (c < D) store8(yr + c, z);
          }
          if (lane == 0) {
            mean_out[i] = 0.f;
            rstd_out[i] = 0.f;
          }
          continue;
        }
        float sum = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if (512 * p + 8 * lane < D) {
#pragma unroll
            for (int j = 0; j < 8; ++j) sum += xv[p].at(j);
          }
        }
        const float mu = wave_sum(sum) * inv_d;
        float sq = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if (512 * p + 8 * lane < D) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float dlt = xv[p].at(j) - mu;
              sq = fmaf(dlt, dlt, sq);
            }
          }
        }
        const float rs = rsqrtf(wave_sum(sq) * inv_d + eps);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int c = 512 * p + 8 * lane;
          if (c < D) {
            float sc[8], sh[8], o[8];
            *(f32x4*)sc = *(const f32x4*)(msc + c);
            *(f32x4*)(sc + 4) = *(const f32x4*)(msc + c + 4);
            *(f32x4*)sh = *(const f32x4*)(msh + c);
            *(f32x4*)(sh + 4) = *(const f32x4*)(msh + c + 4);
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = fmaf((xv[p].at(j) - mu) * rs, sc[j], sh[j]);
            store8(yr + c, o);
          }
        }
        if (lane == 0) {
          mean_out[i] = mu;
          rstd_out[i] = rs;
        }
      }
    }
    __syncthreads();  // LDS is restaged for the next piece
    p0 = p1;
  }
}

// ---------------------------------------------------------------- backward
// Same row layout as the forward: one wave per row, the next row's x and dy
// loads issued before the current row is processed, workgroup b of G taking
// the contiguous rows [b*n/G, (b+1)*n/G) cut into pieces that lie in one
// segment (at most kPiece rows; the piece's 1 + scale slice, validity and row
// statistics staged in LDS).  dx needs two row sums (sum g, sum g*xhat), done
// in registers and by a wave reduction.  d_shift and d_scale accumulate in
// per-lane registers down the rows (every lane owns fixed feature columns:
// the feature-tile reduction, with each load a contiguous row slice); when
// the segment changes or the range ends, the 4 waves' sums are added in LDS
// in wave order and written to partial slot b + s.  The slot map is
// injective: the segments a workgroup's range meets are contiguous and
// non-decreasing in b.  A second kernel adds, for each segment, the slots of
// the workgroups whose range meets it, in workgroup order.
constexpr int kMaxGrid = 1024;  // backward workgroups (bounds the partial slots)

// Workgroup of G whose row range [b*n/G, (b+1)*n/G) holds row r (0 <= r < n).
__device__ __forceinline__ int block_of_row(int64_t r, int G, int n) {
  int b = (int)(r * G / n);
  while ((int64_t)(b + 1) * n / G <= r) ++b;
  return b;
}

template <typename T, int NP>
__global__ void __launch_bounds__(64 * kFwdWaves)
adaln_bwd_rows_kernel(const T* __restrict__ x, const T* __restrict__ dy,
                      const int32_t* __restrict__ ids, const int32_t* __restrict__ offsets,
                      int32_t S, int32_t n, int32_t D, const float* __restrict__ scale,
                      const float* __restrict__ mean, const float* __restrict__ rstd,
                      T* __restrict__ dx, float* __restrict__ partial) {
  constexpr int NT = 64 * kFwdWaves;
  extern __shared__ int32_t lds[];
  float* msc = (float*)lds;             // [D] 1 + scale of the current segment
  float* comb = msc + D;                // [2][D] the waves' partial sums, added in order
  float* rmu = comb + 2 * D;            // [kPiece] mean, 0 for invalid rows
  float* rrs = rmu + kPiece;            // [kPiece] rstd, 0 for invalid rows
  int32_t* okr = (int32_t*)(rrs + kPiece);  // [kPiece]
  int32_t* off = okr + kPiece;          // [S + 1]
  load_offsets<NT>(offsets, S, n, off);
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const float inv_d = 1.0f / (float)D;
  const int i0 = (int)((int64_t)blockIdx.x * n / gridDim.x);
  const int i1 = (int)((int64_t)(blockIdx.x + 1) * n / gridDim.x);
  const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float a_sh[NP][8], a_sc[NP][8];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int j = 0; j < 8; ++j) a_sh[p][j] = a_sc[p][j] = 0.f;
  int seg = last_le(off, S + 1, i0);
  int staged = -1;  // segment whose 1 + scale slice is in LDS
  for (int p0 = i0; p0 < i1;) {
    while (seg < S && p0 >= off[seg + 1]) ++seg;
    const bool in_seg = seg >= 0 && seg < S;
    const int seg_end = seg < 0 ? off[0] : (seg < S ? off[seg + 1] : n);
    const int p1 = min(min(i1, p0 + kPiece), seg_end);
    if (!in_seg) {  // rows in no segment: dx = 0
      for (int i = p0 + wv; i < p1; i += kFwdWaves) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int c = 512 * p + 8 * lane;
          if (c < D) store8(dx + (size_t)i * D + c, z);
        }
      }
      p0 = p1;
      continue;
    }
    if (staged != seg) {
      staged = seg;
      for (int j = 4 * threadIdx.x; j < D; j += 4 * NT)
        *(f32x4*)(msc + j) = *(const f32x4*)(scale + (size_t)seg * D + j) + 1.0f;
    }
    for (int r = threadIdx.x; r < p1 - p0; r += NT) {
      const bool ok = ids[p0 + r] >= 0;
      okr[r] = ok ? 1 : 0;
      rmu[r] = ok ? mean[p0 + r] : 0.f;
      rrs[r] = ok ? rstd[p0 + r] : 0.f;
    }
    __syncthreads();
    Row8<T> xv[NP], gv[NP], xn[NP], gn[NP];
    int i = p0 + wv;
    bool ok_n = i < p1 && okr[i - p0] != 0;
    if (ok_n) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int c = 512 * p + 8 * lane;
        if (c < D) {
          xn[p].load(x + (size_t)i * D + c);
          gn[p].load(dy + (size_t)i * D + c);
        }
      }
    }
    for (; i < p1; i += kFwdWaves) {
      const bool ok = ok_n;
      const float mu = rmu[i - p0], rs = rrs[i - p0];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        xv[p] = xn[p];
        gv[p] = gn[p];
      }
      const int inx = i + kFwdWaves;
      ok_n = inx < p1 && okr[inx - p0] != 0;
      if (ok_n) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int c = 512 * p + 8 * lane;
          if (c < D) {
            xn[p].load(x + (size_t)inx * D + c);
            gn[p].load(dy + (size_t)inx * D + c);
          }
        }
      }
      T* dxr = dx + (size_t)i * D;
      if (!ok) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int c = 512 * p + 8 * lane;
          if (c < D) store8(dxr + c, z);
        }
        continue;
      }
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int c = 512 * p + 8 * lane;
        if (c < D) {
          float sc[8];
          *(f32x4*)sc = *(const f32x4*)(msc + c);
          *(f32x4*)(sc + 4) = *(const f32x4*)(msc + c + 4);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float xh = (xv[p].at(j) - mu) * rs, d = gv[p].at(j);
            a_sc[p][j] = fmaf(d, xh, a_sc[p][j]);
            a_sh[p][j] += d;
            const float g = d * sc[j];
            s1 += g;
            s2 = fmaf(g, xh, s2);
          }
        }
      }
      const float c1 = wave_sum(s1) * inv_d, c2 = wave_sum(s2) * inv_d;
      // recompute xhat and g from the raw row below instead of keeping 16 floats
      // per pass live across the reduction (keeps the wave at two per SIMD)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        xv[p].launder();
        gv[p].launder();
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int c = 512 * p + 8 * lane;
        if (c < D) {
          float sc[8], o[8];
          *(f32x4*)sc = *(const f32x4*)(msc + c);
          *(f32x4*)(sc + 4) = *(const f32x4*)(msc + c + 4);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float xh = (xv[p].at(j) - mu) * rs, g = gv[p].at(j) * sc[j];
            o[j] = rs * (g - c1 - xh * c2);
          }
          store8(dxr + c, o);
        }
      }
    }
    __syncthreads();  // piece done: LDS may be restaged
    // flush the modulation-gradient sums when the segment ends here
    if (p1 == i1 || p1 == seg_end) {
      for (int w = 0; w < kFwdWaves; ++w) {
        if (wv == w) {
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const int c = 512 * p + 8 * lane;
            if (c < D) {
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                comb[c + j] = w == 0 ? a_sh[p][j] : comb[c + j] + a_sh[p][j];
                comb[D + c + j] = w == 0 ? a_sc[p][j] : comb[D + c + j] + a_sc[p][j];
              }
            }
          }
        }
        __syncthreads();
      }
      float* dst = partial + (size_t)(blockIdx.x + seg) * 2 * D;
      for (int j = 4 * threadIdx.x; j < 2 * D; j += 4 * NT) *(f32x4*)(dst + j) = *(const f32x4*)(comb + j);
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int j = 0; j < 8; ++j) a_sh[p][j] = a_sc[p][j] = 0.f;
      __syncthreads();  // comb is reused by the next flush
    }
    p0 = p1;
  }
}

// Workgroup (s, column chunk): d_shift[s] and d_scale[s] over kRedCols columns
// = the sum, in workgroup order, of the slots b + s of the row workgroups b
// whose range meets segment s.  Thread t owns 4 columns and the workgroups
// bA + lane, + kRedLanes, ...; the kRedLanes partial sums are then added in
// lane order.
__global__ void __launch_bounds__(kRedThreads)
adaln_bwd_reduce_kernel(const float* __restrict__ partial, const int32_t* __restrict__ offsets,
                        int32_t S, int32_t n, int32_t D, int32_t G, float* __restrict__ d_shift,
                        float* __restrict__ d_scale) {
  extern __shared__ int32_t lds[];
  int32_t* off = lds;
  float* red = (float*)(off + (S + 1));  // [kRedLanes][2][kRedCols]
  load_offsets<kRedThreads>(offsets, S, n, off);
  const int chunks = (D + kRedCols - 1) / kRedCols;
  const int s = blockIdx.x / chunks, c0 = (blockIdx.x - s * chunks) * kRedCols;
  const int ct = threadIdx.x % (kRedCols / 4), tl = threadIdx.x / (kRedCols / 4);
  const int c = c0 + 4 * ct;
  f32x4 ash = {0.f, 0.f, 0.f, 0.f}, asc = {0.f, 0.f, 0.f, 0.f};
  if (c < D && off[s] < off[s + 1]) {
    const int bA = block_of_row(off[s], G, n), bB = block_of_row(off[s + 1] - 1, G, n);
    for (int b = bA + tl; b <= bB; b += kRedLanes) {
      const float* src = partial + (size_t)(b + s) * 2 * D;
      ash += *(const f32x4*)(src + c);
      asc += *(const f32x4*)(src + D + c);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    red[(tl * 2 + 0) * kRedCols + 4 * ct + j] = ash[j];
    red[(tl * 2 + 1) * kRedCols + 4 * ct + j] = asc[j];
  }
  __syncthreads();
  if (threadIdx.x < 2 * kRedCols) {
    const int which = threadIdx.x / kRedCols, cc = threadIdx.x % kRedCols;
    float acc = 0.f;
    for (int l = 0; l < kRedLanes; ++l) acc += red[(l * 2 + which) * kRedCols + cc];
    if (c0 + cc < D) (which == 0 ? d_shift : d_scale)[(size_t)s * D + c0 + cc] = acc;
  }
}

// ---------------------------------------------------------------- host side
int32_t check_adaln(int32_t dtype, int32_t n, int32_t D, int32_t S, const void* x,
                    const int32_t* ids, const int32_t* offsets) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (n < 0 || S < 0 || S > kMaxSeg || D < 8 || D % 8 != 0 || D > 512 * kMaxPasses)
    return PA_ERR_SHAPE;
  if (!offsets || (n > 0 && (!x || !ids))) return PA_ERR_NULL;
  if (!aligned16(x)) return PA_ERR_ALIGN;
  return PA_OK;
}

// Workgroups of this kernel the device holds at once (at least one per CU).
int resident_workgroups(const void* kernel, int threads, size_t shm) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, shm) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return cus * per_cu;
}

template <typename T, int NP>
void launch_fwd(const void* x, const int32_t* ids, const int32_t* offsets, int32_t S, int32_t n,
                int32_t D, float eps, const float* shift, const float* scale, void* y,
                float* mean, float* rstd, hipStream_t st) {
  const size_t shm = (size_t)(2 * D + kPiece + S + 1) * sizeof(int32_t);
  const void* kern = (const void*)adaln_fwd_kernel<T, NP>;
  const int64_t want = ((int64_t)n + kFwdWaves - 1) / kFwdWaves;  // at least one row per wave
  const int blocks = (int)std::max<int64_t>(
      1, std::min<int64_t>(want, resident_workgroups(kern, 64 * kFwdWaves, shm)));
  hipLaunchKernelGGL((adaln_fwd_kernel<T, NP>), dim3(blocks), dim3(64 * kFwdWaves), shm, st,
                     (const T*)x, ids, offsets, S, n, D, eps, shift, scale, (T*)y, mean, rstd);
}

// Row workgroups of the backward for n rows (the partial slots it needs are
// this plus the segment count).
template <typename T, int NP>
int bwd_grid(int32_t n, int32_t D, int32_t S, size_t* shm) {
  *shm = (size_t)(3 * D + 3 * kPiece + S + 1) * sizeof(int32_t);
  const void* kern = (const void*)adaln_bwd_rows_kernel<T, NP>;
  const int64_t want = ((int64_t)n + kFwdWaves - 1) / kFwdWaves;
  return (int)std::max<int64_t>(
      1, std::min<int64_t>(std::min<int64_t>(want, kMaxGrid),
                           resident_workgroups(kern, 64 * kFwdWaves, *shm)));
}

template <typename T, int NP>
void launch_bwd(const void* x, const void* dy, const int32_t* ids, const int32_t* offsets,
                int32_t S, int32_t n, int32_t D, const float* scale, const float* mean,
                const float* rstd, void* dx, float* d_shift, float* d_scale, float* partial,
                hipStream_t st) {
  size_t shm1 = 0;
  const int G = bwd_grid<T, NP>(n, D, S, &shm1);
  hipLaunchKernelGGL((adaln_bwd_rows_kernel<T, NP>), dim3(G), dim3(64 * kFwdWaves), shm1, st,
                     (const T*)x, (const T*)dy, ids, offsets, S, n, D, scale, mean, rstd, (T*)dx,
                     partial);
  if (S == 0) return;
  const int chunks = (D + kRedCols - 1) / kRedCols;
  const size_t shm2 = (size_t)(S + 1) * sizeof(int32_t) +
                      (size_t)kRedLanes * 2 * kRedCols * sizeof(float);
  hipLaunchKernelGGL(adaln_bwd_reduce_kernel, dim3(S * chunks), dim3(kRedThreads), shm2, st,
                     partial, offsets, S, std::max(n, 1), D, G, d_shift, d_scale);
}

template <typename T>
void dispatch_fwd(int np, const void* x, const int32_t* ids, const int32_t* offsets, int32_t S,
                  int32_t n, int32_t D, float eps, const float* shift, const float* scale,
                  void* y, float* mean, float* rstd, hipStream_t st) {
  switch (np) {
#define PA_FWD_CASE(k) \
  case k: launch_fwd<T, k>(x, ids, offsets, S, n, D, eps, shift, scale, y, mean, rstd, st); break;
    PA_FWD_CASE(1) PA_FWD_CASE(2) PA_FWD_CASE(3) PA_FWD_CASE(4)
    PA_FWD_CASE(5) PA_FWD_CASE(6) PA_FWD_CASE(7) PA_FWD_CASE(8)
#undef PA_FWD_CASE
  }
}

template <typename T>
void dispatch_bwd(int np, const void* x, const void* dy, const int32_t* ids,
                  const int32_t* offsets, int32_t S, int32_t n, int32_t D, const float* scale,
                  const float* mean, const float* rstd, void* dx, float* d_shift, float* d_scale,
                  float* partial, hipStream_t st) {
  switch (np) {
#define PA_BWD_CASE(k)                                                                   \
  case k:                                                                                \
    launch_bwd<T, k>(x, dy, ids, offsets, S, n, D, scale, mean, rstd, dx, d_shift, d_scale, \
                     partial, st);                                                       \
    break;
    PA_BWD_CASE(1) PA_BWD_CASE(2) PA_BWD_CASE(3) PA_BWD_CASE(4)
    PA_BWD_CASE(5) PA_BWD_CASE(6) PA_BWD_CASE(7) PA_BWD_CASE(8)
#undef PA_BWD_CASE
  }
}

}  // namespace

extern "C" int32_t adaln_fwd(int32_t dtype, int32_t n, int32_t D, int32_t n_seg, float eps,
                             const void* x, const int32_t* seq_id, const int32_t* seg_offsets,
                             const float* shift, const float* scale, void* y, float* mean,
                             float* rstd, void* stream) {
  int32_t st = check_adaln(dtype, n, D, n_seg, x, seq_id, seg_offsets);
  if (st != PA_OK) return st;
  if (n == 0) return PA_OK;
  if (!y || !mean || !rstd || (n_seg > 0 && (!shift || !scale))) return PA_ERR_NULL;
  if (!aligned16(y) || !aligned16(shift) || !aligned16(scale)) return PA_ERR_ALIGN;
  if (!(eps >= 0.0f)) return PA_ERR_SHAPE;
  const int np = (D + 511) / 512;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == PA_BF16)
    dispatch_fwd<uint16_t>(np, x, seq_id, seg_offsets, n_seg, n, D, eps, shift, scale, y, mean,
                           rstd, s);
  else
    dispatch_fwd<float>(np, x, seq_id, seg_offsets, n_seg, n, D, eps, shift, scale, y, mean, rstd,
                        s);
  return launch_status();
}

extern "C" size_t adaln_bwd_workspace_bytes(int32_t n, int32_t D, int32_t n_seg) {
  if (n < 0 || n_seg < 0 || n_seg > kMaxSeg || D < 8 || D % 8 != 0 || D > 512 * kMaxPasses)
    return 0;
  // one partial slot per (row workgroup, segment) pair: at most kMaxGrid + n_seg
  return align_up(((size_t)kMaxGrid + (size_t)n_seg) * 2 * (size_t)D * sizeof(float), 256);
}

extern "C" int32_t adaln_bwd(int32_t dtype, int32_t n, int32_t D, int32_t n_seg, const void* x,
                             const void* dy, const int32_t* seq_id, const int32_t* seg_offsets,
                             const float* scale, const float* mean, const float* rstd, void* dx,
                             float* d_shift, float* d_scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int32_t st = check_adaln(dtype, n, D, n_seg, x, seq_id, seg_offsets);
  if (st != PA_OK) return st;
  if ((n > 0 && (!dy || !mean || !rstd || !dx)) ||
      (n_seg > 0 && (!scale || !d_shift || !d_scale)) || !workspace)
    return PA_ERR_NULL;
  if (!aligned16(dy) || !aligned16(dx) || !aligned16(scale) || !aligned16(d_shift) ||
      !aligned16(d_scale) || !aligned256(workspace))
    return PA_ERR_ALIGN;
  if (workspace_bytes < adaln_bwd_workspace_bytes(n, D, n_seg)) return PA_ERR_WORKSPACE;
  const int np = (D + 511) / 512;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == PA_BF16)
    dispatch_bwd<uint16_t>(np, x, dy, seq_id, seg_offsets, n_seg, n, D, scale, mean, rstd, dx,
                           d_shift, d_scale, (float*)workspace, s);
  else
    dispatch_bwd<float>(np, x, dy, seq_id, seg_offsets, n_seg, n, D, scale, mean, rstd, dx,
                        d_shift, d_scale, (float*)workspace, s);
  return launch_status();
}
