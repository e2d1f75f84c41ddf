// device_common.h -- small gfx950 helpers shared by the attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkb {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef int i32x4 __attribute__((__vector_size__(4 * sizeof(int))));
typedef int i32x8 __attribute__((__vector_size__(8 * sizeof(int))));
typedef int i32x16 __attribute__((__vector_size__(16 * sizeof(int))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int readlane_i32(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

__device__ __forceinline__ int64_t readlane_i64(int64_t x, int l) {
  uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Value of lane `src` (per-lane varying) of x, through the LDS crossbar.
__device__ __forceinline__ int shfl_i32(int x, int src) {
  return __builtin_amdgcn_ds_bpermute(src << 2, x);
}
__device__ __forceinline__ int64_t shfl_i64(int64_t x, int src) {
  uint32_t lo = (uint32_t)shfl_i32((int)(uint32_t)x, src);
  uint32_t hi = (uint32_t)shfl_i32((int)(uint32_t)((uint64_t)x >> 32), src);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float xor32_f32(float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ 32) << 2, __float_as_int(x)));
}

// v_permlane32_swap(v, v) yields (own, partner) or (partner, own): a max / sum
// of the two results combines the two half-waves (lanes l and l^32).
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Combine lanes l, l^16, l^32, l^48 (the four 16-lane groups).
__device__ __forceinline__ float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
  return half_max(x);
}
__device__ __forceinline__ float quad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(r[0]) + __int_as_float(r[1]);
  return half_sum(x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats -> packed bf16 pair (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld_global_16(const void* p) { return *(const u32x4*)p; }

// The same load marked non-temporal (the nt cache policy): for data read once
// and streamed through (decode's K/V pages), so it does not displace data that
// is reused in the caches.  Measured on the decode kernel, this lifts the
// sustained read rate by about 12%.
__device__ __forceinline__ u32x4 ld_stream_16(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// Load of kernel-read-only data through the constant address space: with a
// wave-uniform index this is a scalar load, whatever stores or direct-to-LDS
// copies the kernel issues around it.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

}  // namespace pkb
