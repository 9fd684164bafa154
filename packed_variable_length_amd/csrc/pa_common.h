// Internal helpers shared by the HIP sources of libpackattn.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "packattn.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Key-side id used for out-of-range key positions and for padding keys, and the
// query-side id used for padding queries: chosen so that `qk == kk` holds
// exactly for allowed pairs (equal ids, both >= 0).
constexpr int32_t kPadKey = (int32_t)0x80000001;
constexpr int32_t kPadQuery = (int32_t)0x80000000;

__device__ __forceinline__ int32_t key_tag(int32_t id) { return id < 0 ? kPadKey : id; }
__device__ __forceinline__ int32_t query_tag(int32_t id) { return id < 0 ? kPadQuery : id; }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bf16 pair (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// A lane's value and that of lane l ^ 32 (the other half of the wave) from one
// v_permlane32_swap -- a VALU op, no LDS round trip.  Swapping a register with
// itself leaves (own, other) in the two results, in an order that depends on
// the half, so a symmetric reduction of the pair needs no select.
__device__ __forceinline__ f32x2 half_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float half_max(float v) {
  const f32x2 p = half_pair(v);
  return fmaxf(p[0], p[1]);
}
__device__ __forceinline__ float half_sum(float v) {
  const f32x2 p = half_pair(v);
  return p[0] + p[1];
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Argument checks shared by the forward and backward entry points (attn_fwd.hip).
int32_t check_attn_args(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads, int32_t head_dim,
                        const pa_block_mask* mask);

inline int32_t launch_status() {
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
