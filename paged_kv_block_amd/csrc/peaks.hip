// peaks.hip -- on-device ceilings for the roofline denominators: HBM streaming
// read, HBM gather of 4 KiB slabs (paged decode's access shape), each with
// plain or non-temporal loads, L2-resident
// gather of 512-byte rows (the packed-query sparse kernel's), and dense MFMA
// loops in bf16, int8 and fp8.  Measurement code only.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/pkb_peaks.h"
#include "device_common.h"

namespace {

using pkb::i32x16;
using pkb::i32x4;
using pkb::i32x8;
using pkb::f32x16;
using pkb::u32x4;
using pkb::bf16x8;

constexpr uint32_t kMagic = 0x9e3779b9u;   // a checksum equal to this writes the sink

// Mixes three wave-uniform counters into a pseudo-random 32-bit value.
__device__ __forceinline__ uint32_t mix(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t x = a * 0x9E3779B1u ^ (b + 0x7F4A7C15u) * 0x85EBCA77u ^ (c + 1u) * 0xC2B2AE3Du;
  x ^= x >> 15;
  x *= 0x2C1B3C6Du;
  x ^= x >> 12;
  x *= 0x297A2D39u;
  x ^= x >> 15;
  return x;
}

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// 16 bytes per lane, plain or non-temporal (the nt cache policy).
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const unsigned char* p) {
  if (NT) return pkb::ld_stream_16(p);
  return *(const u32x4*)p;
}

// Streaming read: consecutive waves read consecutive 4 KiB chunks, each wave
// four chunks (16 KiB) in flight per iteration; every byte is read once.
template <bool NT>
__global__ void __launch_bounds__(256) hbm_read_kernel(const unsigned char* __restrict__ buf,
                                                      int64_t n_chunks, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t tw = (int64_t)gridDim.x * 4;
  const int64_t gw = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  uint32_t acc = 0;
  for (int64_t c0 = gw; c0 < n_chunks; c0 += 4 * tw) {
    u32x4 v[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t c = c0 + s * tw;
      const unsigned char* p = buf + (c < n_chunks ? c : c0) * 4096 + lane * 16;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[s][k] = ld16<NT>(p + k * 1024);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= fold(v[s][k]);
  }
  if (acc == kMagic) sink[0] = acc;
}

// Each wave reads 4 slabs of 4 KiB per iteration (4 KiB = 4 loads of 1 KiB).
template <bool NT>
__global__ void __launch_bounds__(256) hbm_gather_kernel(const unsigned char* __restrict__ buf,
                                                        uint32_t n_slabs, int iters, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t gw = (uint32_t)__builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    u32x4 v[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t slab = mix(gw, (uint32_t)it, (uint32_t)s) % n_slabs;
      const unsigned char* p = buf + (size_t)slab * 4096 + lane * 16;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[s][k] = ld16<NT>(p + k * 1024);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= fold(v[s][k]);
  }
  if (acc == kMagic) sink[0] = acc;
}

// Each wave reads 16 rows of 512 bytes per iteration: every 1 KiB load covers
// two rows (lanes 0-31 one row, lanes 32-63 another).
__global__ void __launch_bounds__(256) l2_gather_kernel(const unsigned char* __restrict__ buf,
                                                       uint32_t n_rows, int iters, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t gw = (uint32_t)__builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const uint32_t half = (uint32_t)(lane >> 5);
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t row = mix(gw, (uint32_t)it, (uint32_t)(2 * u) + half) % n_rows;
      v[u] = *(const u32x4*)(buf + (size_t)row * 512 + (lane & 31) * 16);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= fold(v[u]);
  }
  if (acc == kMagic) sink[0] = acc;
}

// 8 independent accumulator chains per wave (enough to cover the MFMA
// latency at two waves per SIMD).
template <int KIND>
__global__ void __launch_bounds__(256) mfma_kernel(int iters, uint32_t* sink) {
  const int t = threadIdx.x;
  float chk = 0.f;
  if constexpr (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.001f * (float)((t + i) & 7));
      b[i] = (__bf16)(0.002f * (float)((t * 3 + i) & 7));
    }
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 8; ++c) chk += acc[c][0] + acc[c][15];
  } else if constexpr (KIND == 1) {
    i32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = 0x01010101 * ((t + i) & 3);
      b[i] = 0x01010101 * ((t * 5 + i) & 3);
    }
    i32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] = 0;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 8; ++c) chk += (float)(acc[c][0] ^ acc[c][15]);
  } else {
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x38383838 + ((t + i) & 1);        // E4M3 codes near 1.0
      b[i] = 0x30303030 + ((t * 7 + i) & 1);
    }
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 8; ++c) chk += acc[c][0] + acc[c][15];
  }
  if (__float_as_uint(chk) == kMagic) sink[0] = kMagic;
}

// Vector-issue probe: every wave of the first `waves` of each 512-thread
// workgroup runs `iters` rounds of 8 independent instructions of one kind
// (0: v_fma_f32 with three VGPR sources, 1: v_exp_f32, 2: v_add_f32
// interleaved with an independent s_add_u32); the other waves exit at once.
// With one 512-thread workgroup per CU, waves w and w+4 share a SIMD, so
// waves = 4 puts one wave on each SIMD and waves = 8 two.
template <int KIND>
__global__ void __launch_bounds__(512) issue_kernel(int iters, int waves, uint32_t* sink) {
  const int t = threadIdx.x;
  if (__builtin_amdgcn_readfirstlane(t >> 6) >= waves) return;
  float x0 = t, x1 = t + 1, x2 = t + 2, x3 = t + 3, x4 = t + 4, x5 = t + 5, x6 = t + 6, x7 = t + 7;
  const float c1 = 0.999f + t * 1e-9f, c2 = 0.001f + t * 1e-9f;
  for (int it = 0; it < iters; ++it) {
    if constexpr (KIND == 0)
      asm volatile(
          "v_fma_f32 %0, %0, %8, %9\n\tv_fma_f32 %1, %1, %8, %9\n\tv_fma_f32 %2, %2, %8, %9\n\t"
          "v_fma_f32 %3, %3, %8, %9\n\tv_fma_f32 %4, %4, %8, %9\n\tv_fma_f32 %5, %5, %8, %9\n\t"
          "v_fma_f32 %6, %6, %8, %9\n\tv_fma_f32 %7, %7, %8, %9"
          : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3), "+v"(x4), "+v"(x5), "+v"(x6), "+v"(x7)
          : "v"(c1), "v"(c2));
    else if constexpr (KIND == 1)
      asm volatile(
          "v_exp_f32 %0, %0\n\tv_exp_f32 %1, %1\n\tv_exp_f32 %2, %2\n\tv_exp_f32 %3, %3\n\t"
          "v_exp_f32 %4, %4\n\tv_exp_f32 %5, %5\n\tv_exp_f32 %6, %6\n\tv_exp_f32 %7, %7"
          : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3), "+v"(x4), "+v"(x5), "+v"(x6), "+v"(x7));
    else
      // (the scalar adds work on four SGPRs reserved through the clobber list)
      asm volatile(
          "v_add_f32 %0, %0, %8\n\ts_add_u32 s40, s40, 3\n\tv_add_f32 %1, %1, %8\n\ts_add_u32 s41, s41, 5\n\t"
          "v_add_f32 %2, %2, %8\n\ts_add_u32 s42, s42, 7\n\tv_add_f32 %3, %3, %8\n\ts_add_u32 s43, s43, 9\n\t"
          "v_add_f32 %4, %4, %8\n\ts_add_u32 s40, s40, 3\n\tv_add_f32 %5, %5, %8\n\ts_add_u32 s41, s41, 5\n\t"
          "v_add_f32 %6, %6, %8\n\ts_add_u32 s42, s42, 7\n\tv_add_f32 %7, %7, %8\n\ts_add_u32 s43, s43, 9"
          : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3), "+v"(x4), "+v"(x5), "+v"(x6), "+v"(x7)
          : "v"(c1)
          : "s40", "s41", "s42", "s43", "scc");
  }
  const float chk = x0 + x1 + x2 + x3 + x4 + x5 + x6 + x7;
  if (__float_as_uint(chk) == kMagic) sink[0] = kMagic;
}

// Co-execution probe: waves 0-3 of each 512-thread workgroup run `iters_m`
// rounds of 4 independent bf16 MFMAs (mode 0 or 2), waves 4-7 `iters_v`
// rounds of 8 independent v_fma_f32 (mode 1 or 2).
template <int MODE>
__global__ void __launch_bounds__(512) coexec_kernel(int iters_m, int iters_v, uint32_t* sink) {
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  float chk = 0.f;
  if (wave < 4) {
    if (MODE == 1) return;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.001f * (float)((t + i) & 7));
      b[i] = (__bf16)(0.002f * (float)((t * 3 + i) & 7));
    }
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
    for (int it = 0; it < iters_m; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) chk += acc[c][0] + acc[c][15];
  } else {
    if (MODE == 0) return;
    float x0 = t, x1 = t + 1, x2 = t + 2, x3 = t + 3, x4 = t + 4, x5 = t + 5, x6 = t + 6, x7 = t + 7;
    const float c1 = 0.999f + t * 1e-9f, c2 = 0.001f + t * 1e-9f;
    for (int it = 0; it < iters_v; ++it)
      asm volatile(
          "v_fma_f32 %0, %0, %8, %9\n\tv_fma_f32 %1, %1, %8, %9\n\tv_fma_f32 %2, %2, %8, %9\n\t"
          "v_fma_f32 %3, %3, %8, %9\n\tv_fma_f32 %4, %4, %8, %9\n\tv_fma_f32 %5, %5, %8, %9\n\t"
          "v_fma_f32 %6, %6, %8, %9\n\tv_fma_f32 %7, %7, %8, %9"
          : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3), "+v"(x4), "+v"(x5), "+v"(x6), "+v"(x7)
          : "v"(c1), "v"(c2));
    chk = x0 + x1 + x2 + x3 + x4 + x5 + x6 + x7;
  }
  if (__float_as_uint(chk) == kMagic) sink[0] = kMagic;
}

inline int status(hipError_t e) { return e == hipSuccess ? 0 : -(int)e; }

// The issue and co-execution probes reserve 96 KB of LDS (unused) so that at
// most one of their 512-thread workgroups runs on a CU: waves w and w+4 then
// share a SIMD.
constexpr int kProbeLds = 96 * 1024;
template <auto KERN>
hipError_t allow_probe_lds() {
  // once per kernel and device
  static std::atomic<uint64_t> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute((const void*)KERN, hipFuncAttributeMaxDynamicSharedMemorySize, kProbeLds);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

}  // namespace

extern "C" {

int pkb_peak_hbm_read(const void* buf, int64_t bytes, void* sink, int32_t grid, int32_t nontemporal,
                      void* stream) {
  if (!buf || !sink || bytes < 4096 || bytes % 4096 || grid < 1 || (nontemporal & ~1))
    return -(int)hipErrorInvalidValue;
  if (nontemporal)
    hbm_read_kernel<true><<<grid, 256, 0, (hipStream_t)stream>>>((const unsigned char*)buf, bytes / 4096,
                                                                 (uint32_t*)sink);
  else
    hbm_read_kernel<false><<<grid, 256, 0, (hipStream_t)stream>>>((const unsigned char*)buf, bytes / 4096,
                                                                  (uint32_t*)sink);
  return status(hipGetLastError());
}

int pkb_peak_hbm_gather(const void* buf, int64_t bytes, int64_t n_reads, void* sink,
                        int32_t grid, int32_t nontemporal, int64_t* bytes_read, void* stream) {
  if (!buf || !sink || !bytes_read || bytes < 4096 || bytes % 4096 || grid < 1 || n_reads < 1 ||
      bytes / 4096 > 0xFFFFFFFFLL || (nontemporal & ~1))
    return -(int)hipErrorInvalidValue;
  const int64_t per_iter = (int64_t)grid * 4 * 4;   // slabs per iteration over the grid
  const int64_t iters = (n_reads + per_iter - 1) / per_iter;
  if (iters > 0x7fffffff) return -(int)hipErrorInvalidValue;
  *bytes_read = iters * per_iter * 4096;
  if (nontemporal)
    hbm_gather_kernel<true><<<grid, 256, 0, (hipStream_t)stream>>>((const unsigned char*)buf,
                                                                   (uint32_t)(bytes / 4096), (int)iters,
                                                                   (uint32_t*)sink);
  else
    hbm_gather_kernel<false><<<grid, 256, 0, (hipStream_t)stream>>>((const unsigned char*)buf,
                                                                    (uint32_t)(bytes / 4096), (int)iters,
                                                                    (uint32_t*)sink);
  return status(hipGetLastError());
}

int pkb_peak_l2_gather(const void* buf, int64_t bytes, int64_t n_reads, void* sink,
                       int32_t grid, int64_t* bytes_read, void* stream) {
  if (!buf || !sink || !bytes_read || bytes < 512 || bytes % 512 || bytes > (4 << 20) ||
      grid < 1 || n_reads < 1)
    return -(int)hipErrorInvalidValue;
  const int64_t per_iter = (int64_t)grid * 4 * 16;  // rows per iteration over the grid
  const int64_t iters = (n_reads + per_iter - 1) / per_iter;
  if (iters > 0x7fffffff) return -(int)hipErrorInvalidValue;
  *bytes_read = iters * per_iter * 512;
  l2_gather_kernel<<<grid, 256, 0, (hipStream_t)stream>>>((const unsigned char*)buf,
                                                          (uint32_t)(bytes / 512), (int)iters,
                                                          (uint32_t*)sink);
  return status(hipGetLastError());
}

int pkb_peak_mfma(int32_t kind, int32_t iters, void* sink, int32_t grid, void* stream) {
  if (!sink || iters < 1 || grid < 1) return -(int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0) mfma_kernel<0><<<grid, 256, 0, s>>>(iters, (uint32_t*)sink);
  else if (kind == 1) mfma_kernel<1><<<grid, 256, 0, s>>>(iters, (uint32_t*)sink);
  else if (kind == 2) mfma_kernel<2><<<grid, 256, 0, s>>>(iters, (uint32_t*)sink);
  else return -(int)hipErrorInvalidValue;
  return status(hipGetLastError());
}

int pkb_peak_issue(int32_t kind, int32_t iters, int32_t waves, void* sink, int32_t grid,
                   void* stream) {
  if (!sink || iters < 1 || waves < 1 || waves > 8 || grid < 1) return -(int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (kind == 0) {
    if ((e = allow_probe_lds<issue_kernel<0>>()) != hipSuccess) return status(e);
    issue_kernel<0><<<grid, 512, kProbeLds, s>>>(iters, waves, (uint32_t*)sink);
  } else if (kind == 1) {
    if ((e = allow_probe_lds<issue_kernel<1>>()) != hipSuccess) return status(e);
    issue_kernel<1><<<grid, 512, kProbeLds, s>>>(iters, waves, (uint32_t*)sink);
  } else if (kind == 2) {
    if ((e = allow_probe_lds<issue_kernel<2>>()) != hipSuccess) return status(e);
    issue_kernel<2><<<grid, 512, kProbeLds, s>>>(iters, waves, (uint32_t*)sink);
  } else {
    return -(int)hipErrorInvalidValue;
  }
  return status(hipGetLastError());
}

int pkb_peak_coexec(int32_t mode, int32_t iters_m, int32_t iters_v, void* sink, int32_t grid,
                    void* stream) {
  if (!sink || iters_m < 1 || iters_v < 1 || grid < 1) return -(int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (mode == 0) {
    if ((e = allow_probe_lds<coexec_kernel<0>>()) != hipSuccess) return status(e);
    coexec_kernel<0><<<grid, 512, kProbeLds, s>>>(iters_m, iters_v, (uint32_t*)sink);
  } else if (mode == 1) {
    if ((e = allow_probe_lds<coexec_kernel<1>>()) != hipSuccess) return status(e);
    coexec_kernel<1><<<grid, 512, kProbeLds, s>>>(iters_m, iters_v, (uint32_t*)sink);
  } else if (mode == 2) {
    if ((e = allow_probe_lds<coexec_kernel<2>>()) != hipSuccess) return status(e);
    coexec_kernel<2><<<grid, 512, kProbeLds, s>>>(iters_m, iters_v, (uint32_t*)sink);
  } else {
    return -(int)hipErrorInvalidValue;
  }
  return status(hipGetLastError());
}

}  // extern "C"
