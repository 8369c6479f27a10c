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
// against the element count in the last wavefront of a ragged size, so any
// size is safe.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_device.h"
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

// The wavefront's chunk, units [base, base + 64 kPerLane) of n.  When the
// whole chunk exists (wave-uniform) every load is issued before any is
// used; the last wavefront of a ragged size checks each index and reads
// zero past the end.
template <typename T, bool NT>
__device__ __forceinline__ void load_chunk(const T* __restrict__ src, int64_t base, int64_t n,
                                           int lane, T (&v)[kPerLane]) {
  if (base + 64 * kPerLane <= n) {
    const T* s = src + base;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) v[i] = load<T, NT>(s + 64 * i + lane);
  } else {
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int64_t u = base + 64 * i + lane;
      v[i] = T{};
      if (u < n) v[i] = load<T, NT>(src + u);
    }
  }
}
// Store modes: 0 ordinary, 1 non-temporal, 2 non-temporal with sc1 (the
// quantizer's dequant stream), the last as buffer stores from the
// wavefront's base.
template <int M>
__device__ __forceinline__ void store_unit(u32x4* __restrict__ d, uint32_t i, u32x4 v) {
  if constexpr (M == 2)
    fp4q::put<18>((uint4*)d, i, make_uint4(v.x, v.y, v.z, v.w));
  else
    store<u32x4, M == 1>(d + i, v);
}
template <int M>
__device__ __forceinline__ void store_chunk(u32x4* __restrict__ dst, int64_t base, int64_t n,
                                            int lane, const u32x4 (&v)[kPerLane]) {
  u32x4* d = dst + base;  // wave-uniform
  if (base + 64 * kPerLane <= n) {
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) store_unit<M>(d, 64 * i + lane, v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
      if (base + 64 * i + lane < n) store_unit<M>(d, 64 * i + lane, v[i]);
  }
}

// Read-only: n units of type T; the XOR of everything read is compared with
// a value the host never makes it equal (magic), so the loads are kept and
// nothing is written.
template <typename T, bool NT>
__global__ __launch_bounds__(kWgThreads) void k0_read(const T* __restrict__ src, int64_t n,
                                                      uint32_t magic,
                                                      uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  T v[kPerLane];
  load_chunk<T, NT>(src, wave_base(), n, lane, v);
  uint32_t acc = 0u;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) acc ^= fold(v[i]);
  if (acc == magic) sink[0] = acc;
}

// Copy of n 16-byte units (mode M: loads non-temporal for M >= 1).
template <int M>
__global__ __launch_bounds__(kWgThreads) void k0_copy(const u32x4* __restrict__ src,
                                                      u32x4* __restrict__ dst, int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
  u32x4 v[kPerLane];
  load_chunk<u32x4, (M >= 1)>(src, base, n, lane, v);
  store_chunk<M>(dst, base, n, lane, v);
}

// Streaming copy: a fixed grid whose wavefronts walk the chunks (64 x
// kPerLane units each) with a stride of the whole grid, loading the next
// chunk before storing the current one, so every wavefront always has loads
// in flight.
template <int M>
__global__ __launch_bounds__(kWgThreads) void k0_copy_stream(const u32x4* __restrict__ src,
                                                             u32x4* __restrict__ dst, int64_t n) {
  constexpr bool NT = M >= 1;
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * (kWgThreads / 64) * 64 * kPerLane;
  int64_t base = wave_base();
  u32x4 v[kPerLane];
  if (base < n) load_chunk<u32x4, NT>(src, base, n, lane, v);
  for (; base < n; base += stride) {
    u32x4 nv[kPerLane];
    const int64_t next = base + stride;
    if (next < n) load_chunk<u32x4, NT>(src, next, n, lane, nv);
    store_chunk<M>(dst, base, n, lane, v);
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) v[i] = nv[i];
  }
}

// Read/write mix: each wavefront reads its chunk of n 16-byte units and
// writes 1/D of it -- D = 4 is the routed-token quantizer's mix (4 KiB of
// input, 1 KiB of codes per wavefront) -- as the XOR of D of its units, to
// dst at the chunk's index times 64 kPerLane / D units.
template <int D, int M>
__global__ __launch_bounds__(kWgThreads) void k0_mix(const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst, int64_t n) {
  static_assert(D == 1 || D == 2 || D == 4, "1, 2 or 4 stores fit a lane's 4 units");
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
  u32x4 v[kPerLane];
  load_chunk<u32x4, (M >= 1)>(src, base, n, lane, v);
  u32x4 o[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) o[i] = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) o[i / D] ^= v[i];
  // the output chunk: kPerLane / D units per lane, in the same layout
  const int64_t obase = base / D, on = n / D;
  if (obase + 64 * (kPerLane / D) <= on) {
#pragma unroll
    for (int i = 0; i < kPerLane / D; ++i) store_unit<M>(dst + obase, 64 * i + lane, o[i]);
  } else {
#pragma unroll
    for (int i = 0; i < kPerLane / D; ++i)
      if (obase + 64 * i + lane < on) store_unit<M>(dst + obase, 64 * i + lane, o[i]);
  }
}

// Write-only: n 16-byte units of a pattern derived from the index.
template <int M>
__global__ __launch_bounds__(kWgThreads) void k0_write(u32x4* __restrict__ dst, int64_t n,
                                                       uint32_t seed) {
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
  u32x4 v[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const uint32_t w = seed ^ (uint32_t)(base + 64 * i + lane);
    v[i] = (u32x4){w, w + 1u, w + 2u, w + 3u};
  }
  store_chunk<M>(dst, base, n, lane, v);
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
  if (nontemporal < 0 || nontemporal > 2) return FP4Q_ERROR_INVALID_ARGUMENT;
  if (bytes < 0 || bytes % 16 != 0 || bytes > kMaxBytes) return FP4Q_ERROR_INVALID_SHAPE;
  if (bytes == 0) return FP4Q_SUCCESS;
  if (!src || !dst) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(src, 16) || !aligned(dst, 16)) return FP4Q_ERROR_MISALIGNED;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = split(bytes / 16, [&](int64_t u0, int64_t m, dim3 grid) {
    if (nontemporal == 2)
      hipLaunchKernelGGL(k0_copy<2>, grid, dim3(kWgThreads), 0, st, s + u0, d + u0, m);
    else if (nontemporal == 1)
      hipLaunchKernelGGL(k0_copy<1>, grid, dim3(kWgThreads), 0, st, s + u0, d + u0, m);
    else
      hipLaunchKernelGGL(k0_copy<0>, grid, dim3(kWgThreads), 0, st, s + u0, d + u0, m);
  });
  return e == hipSuccess ? FP4Q_SUCCESS : FP4Q_ERROR_LAUNCH;
}

fp4q_status fp4q_k0_copy_stream(const void* src, void* dst, int64_t bytes, int nontemporal,
                                int workgroups, void* stream) {
  if (nontemporal < 0 || nontemporal > 2) return FP4Q_ERROR_INVALID_ARGUMENT;
  if (bytes < 0 || bytes % 16 != 0 || bytes > kMaxBytes) return FP4Q_ERROR_INVALID_SHAPE;
  if (workgroups < 1 || workgroups > (1 << 20)) return FP4Q_ERROR_INVALID_ARGUMENT;
  if (bytes == 0) return FP4Q_SUCCESS;
  if (!src || !dst) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(src, 16) || !aligned(dst, 16)) return FP4Q_ERROR_MISALIGNED;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  const hipStream_t st = (hipStream_t)stream;
  if (nontemporal == 2)
    hipLaunchKernelGGL(k0_copy_stream<2>, dim3(workgroups), dim3(kWgThreads), 0, st, s, d,
                       bytes / 16);
  else if (nontemporal == 1)
    hipLaunchKernelGGL(k0_copy_stream<1>, dim3(workgroups), dim3(kWgThreads), 0, st, s, d,
                       bytes / 16);
  else
    hipLaunchKernelGGL(k0_copy_stream<0>, dim3(workgroups), dim3(kWgThreads), 0, st, s, d,
                       bytes / 16);
  return hipGetLastError() == hipSuccess ? FP4Q_SUCCESS : FP4Q_ERROR_LAUNCH;
}

fp4q_status fp4q_k0_write(void* dst, int64_t bytes, int nontemporal, void* stream) {
  if (nontemporal < 0 || nontemporal > 2) return FP4Q_ERROR_INVALID_ARGUMENT;
  if (bytes < 0 || bytes % 16 != 0 || bytes > kMaxBytes) return FP4Q_ERROR_INVALID_SHAPE;
  if (bytes == 0) return FP4Q_SUCCESS;
  if (!dst) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(dst, 16)) return FP4Q_ERROR_MISALIGNED;
  u32x4* d = static_cast<u32x4*>(dst);
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = split(bytes / 16, [&](int64_t u0, int64_t m, dim3 grid) {
    if (nontemporal == 2)
      hipLaunchKernelGGL(k0_write<2>, grid, dim3(kWgThreads), 0, st, d + u0, m, (uint32_t)u0);
    else if (nontemporal == 1)
      hipLaunchKernelGGL(k0_write<1>, grid, dim3(kWgThreads), 0, st, d + u0, m, (uint32_t)u0);
    else
      hipLaunchKernelGGL(k0_write<0>, grid, dim3(kWgThreads), 0, st, d + u0, m, (uint32_t)u0);
  });
  return e == hipSuccess ? FP4Q_SUCCESS : FP4Q_ERROR_LAUNCH;
}

fp4q_status fp4q_k0_mix(const void* src, void* dst, int64_t bytes, int divisor,
                        int nontemporal, void* stream) {
  if (divisor != 1 && divisor != 2 && divisor != 4) return FP4Q_ERROR_INVALID_ARGUMENT;
  if (nontemporal < 0 || nontemporal > 2) return FP4Q_ERROR_INVALID_ARGUMENT;
  if (bytes < 0 || bytes % (16 * 64 * kPerLane) != 0 || bytes > kMaxBytes)
    return FP4Q_ERROR_INVALID_SHAPE;
  if (bytes == 0) return FP4Q_SUCCESS;
  if (!src || !dst) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(src, 16) || !aligned(dst, 16)) return FP4Q_ERROR_MISALIGNED;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = split(bytes / 16, [&](int64_t u0, int64_t m, dim3 grid) {
    // u0 is a multiple of whole chunks, so each launch's output starts at u0 / divisor
#define K0_MIX(D, M) hipLaunchKernelGGL((k0_mix<D, M>), grid, dim3(kWgThreads), 0, st, s + u0, \
                                        d + u0 / D, m)
    switch (divisor * 4 + nontemporal) {
      case 4: K0_MIX(1, 0); break;
      case 5: K0_MIX(1, 1); break;
      case 6: K0_MIX(1, 2); break;
      case 8: K0_MIX(2, 0); break;
      case 9: K0_MIX(2, 1); break;
      case 10: K0_MIX(2, 2); break;
      case 16: K0_MIX(4, 0); break;
      case 17: K0_MIX(4, 1); break;
      default: K0_MIX(4, 2); break;
    }
#undef K0_MIX
  });
  return e == hipSuccess ? FP4Q_SUCCESS : FP4Q_ERROR_LAUNCH;
}

}  // extern "C"
