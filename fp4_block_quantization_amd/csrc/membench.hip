// membench.hip -- K0: hand-written HBM probes that bound the quantizer's
// kernels on gfx950 (the copy ceiling its bandwidth fractions are read
// against, and the reference kernels the HBM byte counters are calibrated
// on).  Built as its own library, libfp4q_membench.so; the quantizer does
// not use it.
//
// Every probe has the quantizer's access pattern: a wavefront owns 64 * 4
// consecutive units (16 bytes each for the copy, the write and the 16-byte
// read), lane l taking units l, l + 64, l + 128 and l + 192, so each load
// or store instruction covers 1 KiB contiguously and a wavefront moves
// 4 KiB -- the chunk a wavefront of the NVFP4 kernel copies into LDS.  All
// four loads are issued before the first is used.  Indices are checked
// against the element count, so any size is safe.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_membench.h"

namespace {

// Build-time knob: units per lane (4: the quantizer's 4 KiB per wavefront).
#ifndef FP4Q_K0_UNITS
#define FP4Q_K0_UNITS 4
#endif
constexpr int kPerLane = FP4Q_K0_UNITS;  // units per lane
constexpr int kWgThreads = 256;
constexpr int64_t kPerWg = (int64_t)kWgThreads * kPerLane;  // units per workgroup

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T, bool NT>
__device__ __forceinline__ T load(const T* p) {
  if (NT) return __builtin_nontemporal_load(p);
  return *p;
}
template <typename T, bool NT>
__device__ __forceinline__ void store(T* p, T v) {
  if (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

__device__ __forceinline__ uint32_t fold(uint8_t v) { return v; }
__device__ __forceinline__ uint32_t fold(uint16_t v) { return v; }
__device__ __forceinline__ uint32_t fold(uint32_t v) { return v; }
__device__ __forceinline__ uint32_t fold(u32x2 v) { return v.x ^ v.y; }
__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// The first unit of this lane's wavefront.
__device__ __forceinline__ int64_t wave_base() {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  return ((int64_t)blockIdx.x * (kWgThreads / 64) + wave) * 64 * kPerLane;
}

// Read-only: n units of type T; the XOR of everything read is compared with
// a value the host never makes it equal (magic), so the loads are kept and
// nothing is written.
template <typename T, bool NT>
__global__ __launch_bounds__(kWgThreads) void k0_read(const T* __restrict__ src, int64_t n,
                                                      uint32_t magic,
                                                      uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
  T v[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int64_t u = base + 64 * i + lane;
    if (u < n) v[i] = load<T, NT>(src + u);
  }
  uint32_t acc = 0u;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i)
    if (base + 64 * i + lane < n) acc ^= fold(v[i]);
  if (acc == magic) sink[0] = acc;
}

// Copy of n 16-byte units.
template <bool NT>
__global__ __launch_bounds__(kWgThreads) void k0_copy(const u32x4* __restrict__ src,
                                                      u32x4* __restrict__ dst, int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
  u32x4 v[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int64_t u = base + 64 * i + lane;
    if (u < n) v[i] = load<u32x4, NT>(src + u);
  }
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int64_t u = base + 64 * i + lane;
    if (u < n) store<u32x4, NT>(dst + u, v[i]);
  }
}

// Streaming copy: a fixed grid whose wavefronts walk the chunks (64 x
// kPerLane units each) with a stride of the whole grid, loading the next
// chunk before storing the current one, so every wavefront always has loads
// in flight.
template <bool NT>
__global__ __launch_bounds__(kWgThreads) void k0_copy_stream(const u32x4* __restrict__ src,
                                                             u32x4* __restrict__ dst, int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t chunk_units = 64 * kPerLane;
  const int64_t stride = (int64_t)gridDim.x * (kWgThreads / 64) * chunk_units;
  int64_t base = wave_base();
  u32x4 v[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int64_t u = base + 64 * i + lane;
    if (u < n) v[i] = load<u32x4, NT>(src + u);
  }
  for (; base < n; base += stride) {
    u32x4 nv[kPerLane];
    const int64_t next = base + stride;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int64_t u = next + 64 * i + lane;
      if (u < n) nv[i] = load<u32x4, NT>(src + u);
    }
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int64_t u = base + 64 * i + lane;
      if (u < n) store<u32x4, NT>(dst + u, v[i]);
    }
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) v[i] = nv[i];
  }
}

// Write-only: n 16-byte units of a pattern derived from the index.
template <bool NT>
__global__ __launch_bounds__(kWgThreads) void k0_write(u32x4* __restrict__ dst, int64_t n,
                                                       uint32_t seed) {
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int64_t u = base + 64 * i + lane;
    const uint32_t w = seed ^ (uint32_t)u;
    if (u < n) store<u32x4, NT>(dst + u, (u32x4){w, w + 1u, w + 2u, w + 3u});
  }
}

// Launches of at most 2^31 work-items over consecutive units.
template <typename F>
hipError_t split(int64_t n, F&& launch) {
  const int64_t max_units = ((int64_t)1 << 31) / kWgThreads * kPerWg;
  for (int64_t u0 = 0; u0 < n; u0 += max_units) {
    const int64_t m = n - u0 < max_units ? n - u0 : max_units;
    launch(u0, m, dim3((unsigned)((m + kPerWg - 1) / kPerWg)));
  }
  return hipGetLastError();
}

template <typename T, bool NT>
hipError_t read_width(const void* src, int64_t bytes, uint32_t* sink, hipStream_t st) {
  const T* s = static_cast<const T*>(src);
  return split(bytes / (int64_t)sizeof(T), [&](int64_t u0, int64_t m, dim3 grid) {
    hipLaunchKernelGGL((k0_read<T, NT>), grid, dim3(kWgThreads), 0, st, s + u0, m,
                       0xFFFFFFFFu, sink);
  });
}

template <bool NT>
hipError_t read_any(const void* src, int64_t bytes, int width, uint32_t* sink, hipStream_t st) {
  switch (width) {
    case 1: return read_width<uint8_t, NT>(src, bytes, sink, st);
    case 2: return read_width<uint16_t, NT>(src, bytes, sink, st);
    case 4: return read_width<uint32_t, NT>(src, bytes, sink, st);
    case 8: return read_width<u32x2, NT>(src, bytes, sink, st);
    default: return read_width<u32x4, NT>(src, bytes, sink, st);
  }
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int64_t kMaxBytes = (int64_t)1 << 40;

}  // namespace

extern "C" {

fp4q_status fp4q_k0_read(const void* src, int64_t bytes, int width, int nontemporal,
                         uint32_t* sink, void* stream) {
  if (width != 1 && width != 2 && width != 4 && width != 8 && width != 16)
    return FP4Q_ERROR_INVALID_ARGUMENT;
  if (bytes < 0 || bytes % width != 0 || bytes > kMaxBytes) return FP4Q_ERROR_INVALID_SHAPE;
  if (bytes == 0) return FP4Q_SUCCESS;
  if (!src || !sink) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(src, (uintptr_t)width) || !aligned(sink, 4)) return FP4Q_ERROR_MISALIGNED;
  const hipError_t e = nontemporal ? read_any<true>(src, bytes, width, sink, (hipStream_t)stream)
                                   : read_any<false>(src, bytes, width, sink, (hipStream_t)stream);
  return e == hipSuccess ? FP4Q_SUCCESS : FP4Q_ERROR_LAUNCH;
}

fp4q_status fp4q_k0_copy(const void* src, void* dst, int64_t bytes, int nontemporal,
                         void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || bytes > kMaxBytes) return FP4Q_ERROR_INVALID_SHAPE;
  if (bytes == 0) return FP4Q_SUCCESS;
  if (!src || !dst) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(src, 16) || !aligned(dst, 16)) return FP4Q_ERROR_MISALIGNED;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = split(bytes / 16, [&](int64_t u0, int64_t m, dim3 grid) {
    if (nontemporal)
      hipLaunchKernelGGL(k0_copy<true>, grid, dim3(kWgThreads), 0, st, s + u0, d + u0, m);
    else
      hipLaunchKernelGGL(k0_copy<false>, grid, dim3(kWgThreads), 0, st, s + u0, d + u0, m);
  });
  return e == hipSuccess ? FP4Q_SUCCESS : FP4Q_ERROR_LAUNCH;
}

fp4q_status fp4q_k0_copy_stream(const void* src, void* dst, int64_t bytes, int nontemporal,
                                int workgroups, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || bytes > kMaxBytes) return FP4Q_ERROR_INVALID_SHAPE;
  if (workgroups < 1 || workgroups > (1 << 20)) return FP4Q_ERROR_INVALID_ARGUMENT;
  if (bytes == 0) return FP4Q_SUCCESS;
  if (!src || !dst) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(src, 16) || !aligned(dst, 16)) return FP4Q_ERROR_MISALIGNED;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  const hipStream_t st = (hipStream_t)stream;
  if (nontemporal)
    hipLaunchKernelGGL(k0_copy_stream<true>, dim3(workgroups), dim3(kWgThreads), 0, st, s, d,
                       bytes / 16);
  else
    hipLaunchKernelGGL(k0_copy_stream<false>, dim3(workgroups), dim3(kWgThreads), 0, st, s, d,
                       bytes / 16);
  return hipGetLastError() == hipSuccess ? FP4Q_SUCCESS : FP4Q_ERROR_LAUNCH;
}

fp4q_status fp4q_k0_write(void* dst, int64_t bytes, int nontemporal, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || bytes > kMaxBytes) return FP4Q_ERROR_INVALID_SHAPE;
  if (bytes == 0) return FP4Q_SUCCESS;
  if (!dst) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(dst, 16)) return FP4Q_ERROR_MISALIGNED;
  u32x4* d = static_cast<u32x4*>(dst);
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = split(bytes / 16, [&](int64_t u0, int64_t m, dim3 grid) {
    if (nontemporal)
      hipLaunchKernelGGL(k0_write<true>, grid, dim3(kWgThreads), 0, st, d + u0, m,
                         (uint32_t)u0);
    else
      hipLaunchKernelGGL(k0_write<false>, grid, dim3(kWgThreads), 0, st, d + u0, m,
                         (uint32_t)u0);
  });
  return e == hipSuccess ? FP4Q_SUCCESS : FP4Q_ERROR_LAUNCH;
}

}  // extern "C"
