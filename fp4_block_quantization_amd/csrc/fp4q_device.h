// fp4q_device.h -- device-side number-format helpers for gfx950.
//
// Formats: E2M1 (TRACE page, Jargon: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6),
// OCP E4M3FN block scales (NVFP4-RL blog, section 2: "FP8 E4M3"), E8M0 MX
// scales and BF16 (HiFloat4 page, Rollout-ResQ section; NVFP4-RL blog,
// section 3).  All rounding is to nearest with ties to even.  Built with
// -ffp-contract=off, FP32 denormals preserved and correctly rounded FP32
// division, so every float operation below is one IEEE binary32 operation.
#pragma once

// The memory-pattern stand-in build (-DFP4Q_STANDIN=1) and the
// exact-error decision build (-DFP4Q_NV_CERTIFY=0) put everything in a
// namespace of their own, so that their kernels carry names of their own in
// profiles and cannot be mistaken for the quantizer's.
#if defined(FP4Q_STANDIN) && FP4Q_STANDIN && !defined(fp4q)
#define fp4q fp4q_standin
#elif defined(FP4Q_NV_CERTIFY) && !FP4Q_NV_CERTIFY && !defined(fp4q)
#define fp4q fp4q_exactdecision
#endif

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// ---- gfx950 conversion instructions -------------------------------------
// Each was compared exhaustively on the GPU with the CPU reference's
// definition over the inputs the kernels can feed it (see the GPU probe
// tests): E2M1 encode of signed FP32 with unit scale (round to nearest
// even, saturating, sign kept for zeros), E2M1 decode, E4M3FN encode on
// [0, 448], E4M3FN decode and FP32 -> BF16 (round to nearest even).  NaN
// must not reach the E2M1 encode (it yields 7, not 0).

// Codes of a (low nibble) and b (high nibble) into byte SEL of acc.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_e2m1x2(uint32_t acc, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, a, b, 1.0f, SEL);
}

// Codes of a / 2^k (low nibble) and b / 2^k into byte SEL of acc, where
// scale2k is the FP32 pattern (k + 127) << 23: the conversion divides by
// the power of two whose E8M0 byte is the scale's exponent field before
// rounding.  Pinned for every k in [-127, 125] over every input with at
// most 10 significant bits below 2^(k+3) -- each element and each residual
// of an MX block with shared exponent k.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_e2m1x2_scaled(uint32_t acc, float a, float b,
                                                      float scale2k) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, a, b, scale2k, SEL);
}

// The E2M1 codes of the grid points at or below a and b (a, b >= 0;
// saturating at code 7) in bits 0-7 (a in the low nibble): the
// stochastic-rounding conversion with a zero seed adds nothing before
// truncating, so it rounds toward zero (checked over every binary32 value in
// [0, 8], saturation windows and +inf by the conversion probes).  Only the
// selected byte of that instruction's result is defined -- the others do
// not keep the accumulator operand's bytes -- so the rest are cleared.
__device__ __forceinline__ uint32_t cvt_e2m1x2_floor(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, (float2v){a, b}, 0u, 1.0f, 0) & 0xFFu;
}

// Signed values of the two nibbles of byte SEL of src (low nibble in .x).
template <int SEL>
__device__ __forceinline__ float2v e2m1x2_values(uint32_t src) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(src, 1.0f, SEL);
}

// The two E2M1 values of byte SEL times 2^k, exact, where scale2k is the
// FP32 pattern (k + 127) << 23 (k = -127 gives the all-zero pattern: the
// conversion reads the scale's exponent field as an E8M0 byte).
template <int SEL>
__device__ __forceinline__ float2v e2m1x2_values_scaled(uint32_t src, float scale2k) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(src, scale2k, SEL);
}

// The same values as FP16 (exact: E2M1 values are FP16 numbers).
template <int SEL>
__device__ __forceinline__ half2v e2m1x2_values_f16(uint32_t src) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(src, 1.0f, SEL);
}

// A register whose every bit the caller overwrites before reading it (a
// code word filled byte by byte by the conversions below, or masked): the
// empty asm defines it, so no zero is materialized first.
__device__ __forceinline__ uint32_t any_word() {
  uint32_t w;
  asm volatile("" : "=v"(w));  // volatile: each call its own register
  return w;
}

// E4M3FN bytes of a (byte 0) and b (byte 1), both in [0, 448].
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)any_word(), false) & 0xFFFFu;
}

template <int SEL>
__device__ __forceinline__ float e4m3_value(uint32_t bytes) {
  return __builtin_amdgcn_cvt_f32_fp8((int)bytes, SEL);
}

// Two FP32 -> packed BF16 (a in the low half).
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  const float2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// fl(1/d), the IEEE quotient, for 2^-126 <= d <= 2^126: the hardware
// reciprocal approximation y, the residual e = 1 - d*y in one FMA, and the
// refined y + e*y in another.  Pinned against the CPU's IEEE division over
// every binary32 value of that range.
__device__ __forceinline__ float recip_normal(float d) {
  const float y = __builtin_amdgcn_rcpf(d);
  const float e = __builtin_fmaf(-d, y, 1.0f);
  return __builtin_fmaf(e, y, y);
}

// fl(a / C) for a non-negative finite BF16 value a (a row amax) and C = 1536
// (four_over_six) or 2688: the product with fl(1/C), corrected by one FMA
// residual step.  Equal to the IEEE quotient for every such a and both
// constants (pinned exhaustively on the GPU).
__device__ __forceinline__ float amax_over_c(float a, bool four_over_six) {
  const float c = four_over_six ? 1536.0f : 2688.0f;
  const float c_inv = four_over_six ? 0x1.555556p-11f : 0x1.861862p-12f;  // fl(1/c)
  const float q = a * c_inv;
  const float r = __builtin_fmaf(-q, c, a);
  return __builtin_fmaf(r, c_inv, q);
}

// ---- portable definitions -------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// FP32 -> BF16 bit pattern, round to nearest even.  Only finite values
// reach it (candidates are products of finite scales).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

// E2M1 magnitude code of a >= 0 and its value: the grid below 1 has step
// 0.5; from 1 up each binade holds two values (one fraction bit), so
// rounding the binary32 significand to one fraction bit by an integer add
// (ties to even; the carry steps the exponent) lands on the grid.  Codes
// past 6 saturate.  a = NaN (only 0 * inf, from an infinite reciprocal of a
// tiny decode step) gives code 0, like a zero input.
__device__ __forceinline__ uint32_t e2m1_code_sw(float a, float& g) {
  const uint32_t u = __float_as_uint(a);
  const uint32_t ur = u + 0x1FFFFFu + ((u >> 22) & 1u);
  uint32_t code = min(ur >> 22, 259u) - 252u;  // 1.0 -> 2, 1.5 -> 3, ..., 6.0 -> 7
  float val = (code == 7u) ? 6.0f : __uint_as_float(ur & 0xFFC00000u);
  if (a < 1.0f) {  // 0.25 -> 0 and 0.75 -> 1.0 (the even codes)
    code = (a > 0.25f ? 1u : 0u) + (a >= 0.75f ? 1u : 0u);
    val = 0.5f * (float)code;
  }
  if (u > 0x7F800000u) {  // NaN
    code = 0u;
    val = 0.0f;
  }
  g = val;
  return code;
}

// OCP E4M3FN byte of t >= 0 (or NaN, treated as 0) and its exact value.
// Bias 7, 3 fraction bits, smallest normal 2^-6 with step 2^-9 below it,
// largest finite 448 (0x7E); larger values saturate.
__device__ __forceinline__ uint32_t e4m3_encode(float t, float& val) {
  if (!(t > 0.0f)) {
    val = 0.0f;
    return 0u;
  }
  if (t > 448.0f) {
    val = 448.0f;
    return 0x7Eu;
  }
  if (t < 0.015625f) {  // multiples of 2^-9; 8 * 2^-9 is the first normal (byte 0x08)
    const float m = __builtin_rintf(t * 512.0f);
    val = m * (1.0f / 512.0f);
    return (uint32_t)m;
  }
  const uint32_t u = __float_as_uint(t);
  const uint32_t ur = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;
  val = __uint_as_float(ur);
  return (ur >> 20) - 960u;  // ((binary32 exponent - 127 + 7) << 3) | fraction
}

// Value of an E4M3FN byte (sign honoured).
__device__ __forceinline__ float e4m3_decode(uint32_t byte) {
  const uint32_t mag = byte & 0x7Fu;
  float v = (mag < 8u) ? (float)mag * (1.0f / 512.0f) : __uint_as_float((mag + 960u) << 20);
  if (mag == 0x7Fu) v = __builtin_nanf("");
  return (byte & 0x80u) ? -v : v;
}

// Value of E2M1 magnitude code q (0..7).
__device__ __forceinline__ float e2m1_value(uint32_t q) {
  return (q < 2u) ? 0.5f * (float)q
                  : __uint_as_float((((q >> 1) + 126u) << 23) | ((q & 1u) << 22));
}

// MX shared exponent of a block whose max magnitude has binary32 pattern
// bits (non-negative): floor(log2 b) - 2, clamped to [-127, 127]; zero and
// tiny maxima give -127.  For b >= 2^-126, floor(log2 b) is the unbiased
// exponent field; anything smaller clamps anyway.
__device__ __forceinline__ int mx_exponent(uint32_t bits) {
  return max((int)(bits >> 23) - 129, -127);
}

// ---- output stores with a cache policy ----------------------------------
// POL holds the cache-policy bits of the gfx950 memory instructions (1 sc0,
// 2 nt, 16 sc1; -1: none).  One lane stores element idx of an array whose
// base is uniform over the wavefront: no bits and nt alone as global stores
// (scalar base, lane offset), other bits as a buffer store through a
// descriptor at base, whose 32-bit byte offset idx * sizeof(T) every caller
// keeps far below 2^32 (one chunk or row of a wavefront).
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, -1, 0x20000);
}
template <int POL>
__device__ __forceinline__ void put(uint4* base, uint32_t idx, uint4 v) {
  const u32x4v w = {v.x, v.y, v.z, v.w};
  if constexpr (POL < 0)
    base[idx] = v;
  else if constexpr (POL == 2)
    __builtin_nontemporal_store(w, (u32x4v*)&base[idx]);
  else
    __builtin_amdgcn_raw_buffer_store_b128(w, rsrc_at(base), idx * 16u, 0, POL);
}
template <int POL>
__device__ __forceinline__ void put(uint2* base, uint32_t idx, uint2 v) {
  const u32x2v w = {v.x, v.y};
  if constexpr (POL < 0)
    base[idx] = v;
  else if constexpr (POL == 2)
    __builtin_nontemporal_store(w, (u32x2v*)&base[idx]);
  else
    __builtin_amdgcn_raw_buffer_store_b64(w, rsrc_at(base), idx * 8u, 0, POL);
}
template <int POL>
__device__ __forceinline__ void put(uint32_t* base, uint32_t idx, uint32_t v) {
  if constexpr (POL < 0)
    base[idx] = v;
  else if constexpr (POL == 2)
    __builtin_nontemporal_store(v, &base[idx]);
  else
    __builtin_amdgcn_raw_buffer_store_b32(v, rsrc_at(base), idx * 4u, 0, POL);
}
template <int POL>
__device__ __forceinline__ void put(uint16_t* base, uint32_t idx, uint16_t v) {
  if constexpr (POL < 0)
    base[idx] = v;
  else if constexpr (POL == 2)
    __builtin_nontemporal_store(v, &base[idx]);
  else
    __builtin_amdgcn_raw_buffer_store_b16(v, rsrc_at(base), idx * 2u, 0, POL);
}
template <int POL>
__device__ __forceinline__ void put(uint8_t* base, uint32_t idx, uint8_t v) {
  if constexpr (POL < 0)
    base[idx] = v;
  else if constexpr (POL == 2)
    __builtin_nontemporal_store(v, &base[idx]);
  else
    __builtin_amdgcn_raw_buffer_store_b8(v, rsrc_at(base), idx, 0, POL);
}

}  // namespace fp4q
