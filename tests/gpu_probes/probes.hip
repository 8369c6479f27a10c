// probes.hip -- exhaustive GPU evaluation of number-format conversions:
// the gfx950 hardware conversion instructions and the library's own device
// helpers (fp4q_device.h), over ranges of binary32 bit patterns.  The host
// compares every result with the CPU oracle's primitives.
//
// Every kernel handles element i < n only and writes out[i]; the launcher
// sizes the grid from n.  Input patterns are generated in-kernel from
// (lo + index), so no input buffer exists.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_device.h"

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

namespace {

__device__ __forceinline__ float pat(uint32_t lo, uint64_t k, uint32_t flip) {
  return __uint_as_float((uint32_t)(lo + k) ^ flip);
}

// out[i] = byte holding the FP4 codes of patterns lo+2i (first operand) and
// lo+2i+1 (second operand), hardware conversion with scale 1.0.
__global__ void k_hw_fp4(uint32_t lo, uint32_t flip, uint64_t n, uint8_t* out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float a = pat(lo, 2 * i, flip), b = pat(lo, 2 * i + 1, flip);
  out[i] = (uint8_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0);
}

// software E2M1 of |pattern| with the sign bit of the pattern, same layout
__global__ void k_sw_fp4(uint32_t lo, uint32_t flip, uint64_t n, uint8_t* out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t byte = 0;
  for (int h = 0; h < 2; ++h) {
    const float v = pat(lo, 2 * i + h, flip);
    float g;
    const uint32_t q = fp4q::e2m1_code_sw(fabsf(v), g);
    byte |= (q | ((__float_as_uint(v) >> 31) << 3)) << (4 * h);
  }
  out[i] = (uint8_t)byte;
}

// out[i] = the two BF16 patterns of lo+2i (low half) and lo+2i+1 (high)
__global__ void k_hw_bf16(uint32_t lo, uint64_t n, uint32_t* out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float2v v = {pat(lo, 2 * i, 0u), pat(lo, 2 * i + 1, 0u)};
  out[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

__global__ void k_sw_bf16(uint32_t lo, uint64_t n, uint32_t* out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = fp4q::pack_bf16x2(pat(lo, 2 * i, 0u), pat(lo, 2 * i + 1, 0u));
}

// out[i] = the two E4M3 bytes of lo+2i (low) and lo+2i+1 (high)
__global__ void k_hw_fp8(uint32_t lo, uint64_t n, uint16_t* out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = (uint16_t)__builtin_amdgcn_cvt_pk_fp8_f32(pat(lo, 2 * i, 0u), pat(lo, 2 * i + 1, 0u),
                                                     0, false);
}

__global__ void k_sw_fp8(uint32_t lo, uint64_t n, uint16_t* out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v;
  const uint32_t a = fp4q::e4m3_encode(pat(lo, 2 * i, 0u), v);
  const uint32_t b = fp4q::e4m3_encode(pat(lo, 2 * i + 1, 0u), v);
  out[i] = (uint16_t)(a | (b << 8));
}

// decode tables: out has 512 floats for FP4 (byte b -> low, high nibble)
// and 256 floats for FP8
__global__ void k_decode_tables(float* fp4_hw, float* fp4_sw, float* fp8_hw, float* fp8_sw) {
  const uint32_t b = threadIdx.x;  // 256 threads
  const float2v d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b, 1.0f, 0);
  fp4_hw[2 * b] = d.x;
  fp4_hw[2 * b + 1] = d.y;
  for (int h = 0; h < 2; ++h) {
    const uint32_t nib = (b >> (4 * h)) & 15u;
    const float g = fp4q::e2m1_value(nib & 7u);
    fp4_sw[2 * b + h] = (nib & 8u) ? -g : g;
  }
  fp8_hw[b] = __builtin_amdgcn_cvt_f32_fp8(b, 0);
  fp8_sw[b] = fp4q::e4m3_decode(b);
}

// Scaled conversions (MX scales).  sbits is the FP32 pattern of the scale
// operand.  bf16 variant: out[i] = codes of BF16 patterns 2i (low) and
// 2i+1 (high), i < 32768.
// out[2b], out[2b+1]: scaled decode of byte b (256 threads)
__global__ void k_hw_fp4_decode_scaled(uint32_t sbits, float* out) {
  const uint32_t b = threadIdx.x;
  const float2v d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b, __uint_as_float(sbits), 0);
  out[2 * b] = d.x;
  out[2 * b + 1] = d.y;
}

// out[i] = FP4 byte of the patterns (2i) << 13 (low nibble) and
// (2i + 1) << 13 -- every binary32 value whose low 13 bits are zero, so
// every BF16 value and every value of at most 10 significant bits -- from
// the encode with scale operand sbits
__global__ void k_hw_fp4_encode_scaled(uint32_t sbits, uint64_t n, uint8_t* out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float a = __uint_as_float((uint32_t)(2 * i) << 13);
  const float b = __uint_as_float((uint32_t)(2 * i + 1) << 13);
  out[i] = (uint8_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, __uint_as_float(sbits), 0);
}

// out[i] = FP4 byte of patterns lo+2i (low nibble) and lo+2i+1 from the
// stochastic-rounding conversion with seed 0 and scale 1.0 (the guided
// quantizer's lower neighbour)
__global__ void k_hw_fp4_sr0(uint32_t lo, uint64_t n, uint8_t* out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float a = pat(lo, 2 * i, 0u), b = pat(lo, 2 * i + 1, 0u);
  out[i] = (uint8_t)fp4q::cvt_e2m1x2_floor(a, b);
}

// out[i] = the refined hardware reciprocal of pattern lo + i
__global__ void k_recip_normal(uint32_t lo, uint64_t n, float* out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = fp4q::recip_normal(pat(lo, i, 0u));
}

// out[i] = the token scale of the BF16 amax pattern i % 0x7F80 (every
// non-negative finite BF16 value), four_over_six for i >= 0x7F80
__global__ void k_amax_over_c(float* out) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 2u * 0x7F80u) return;
  out[i] = fp4q::amax_over_c(__uint_as_float((i % 0x7F80u) << 16), i >= 0x7F80u);
}

dim3 grid_for(uint64_t n) { return dim3((unsigned)((n + 255) / 256)); }

}  // namespace

extern "C" {

// which: 0 hw fp4, 1 sw fp4, 2 hw bf16, 3 sw bf16, 4 hw fp8, 5 sw fp8,
// 6 hw fp4 lower neighbour (flip ignored), 7 refined reciprocal (one float
// per pattern, flip ignored)
int probe_launch(int which, uint32_t lo, uint32_t flip, uint64_t n, void* out, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (n == 0 || n > (1ull << 31)) return 2;
  switch (which) {
    case 0: hipLaunchKernelGGL(k_hw_fp4, grid_for(n), dim3(256), 0, st, lo, flip, n, (uint8_t*)out); break;
    case 1: hipLaunchKernelGGL(k_sw_fp4, grid_for(n), dim3(256), 0, st, lo, flip, n, (uint8_t*)out); break;
    case 2: hipLaunchKernelGGL(k_hw_bf16, grid_for(n), dim3(256), 0, st, lo, n, (uint32_t*)out); break;
    case 3: hipLaunchKernelGGL(k_sw_bf16, grid_for(n), dim3(256), 0, st, lo, n, (uint32_t*)out); break;
    case 4: hipLaunchKernelGGL(k_hw_fp8, grid_for(n), dim3(256), 0, st, lo, n, (uint16_t*)out); break;
    case 5: hipLaunchKernelGGL(k_sw_fp8, grid_for(n), dim3(256), 0, st, lo, n, (uint16_t*)out); break;
    case 6: hipLaunchKernelGGL(k_hw_fp4_sr0, grid_for(n), dim3(256), 0, st, lo, n, (uint8_t*)out); break;
    case 7: hipLaunchKernelGGL(k_recip_normal, grid_for(n), dim3(256), 0, st, lo, n, (float*)out); break;
    default: return 2;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// out[2b], out[2b+1]: the scaled decode of byte b (256 threads) under the
// scale operand bit pattern sbits
int probe_decode_scaled(uint32_t sbits, void* out, void* stream) {
  hipLaunchKernelGGL(k_hw_fp4_decode_scaled, dim3(1), dim3(256), 0, (hipStream_t)stream, sbits,
                     (float*)out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// out[i], i < n <= 2^18: the scaled encode of the patterns (2i) << 13 and
// (2i + 1) << 13 under the scale operand bit pattern sbits
int probe_encode_scaled(uint32_t sbits, uint64_t n, void* out, void* stream) {
  if (n == 0 || n > (1ull << 18)) return 2;
  hipLaunchKernelGGL(k_hw_fp4_encode_scaled, grid_for(n), dim3(256), 0, (hipStream_t)stream, sbits,
                     n, (uint8_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// out[i], i < 2 * 0x7F80: see k_amax_over_c
int probe_amax_over_c(void* out, void* stream) {
  hipLaunchKernelGGL(k_amax_over_c, grid_for(2 * 0x7F80), dim3(256), 0, (hipStream_t)stream,
                     (float*)out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int probe_decode_tables(void* fp4_hw, void* fp4_sw, void* fp8_hw, void* fp8_sw, void* stream) {
  hipLaunchKernelGGL(k_decode_tables, dim3(1), dim3(256), 0, (hipStream_t)stream,
                     (float*)fp4_hw, (float*)fp4_sw, (float*)fp8_hw, (float*)fp8_sw);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
