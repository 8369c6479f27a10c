// nvfp4.hip -- per-token NVFP4 quantization with Four-Over-Six (K1) and
// NVFP4 dequantization (K2) for gfx950.
//
// Method: "NVFP4-RL" (jianyuh.github.io), sections 2-4, and "humans&
// Open-Sources the First Stable 4-Bit RL Training Recipe at 1.73x Speedup"
// (alphasignal.ai), sections 1-3.  Each token row gets its own FP32 scale
// s from its amax over the hidden dimension; the E4M3 scale of every
// 16-element block is computed in the same kernel; per block the max is
// mapped to 6 or to 4, whichever gives the lower squared error (ties keep
// 6); the BF16 dequantized values of the chosen encoding are written in the
// same pass for the dequantized backward.
//
// Mapping (K1): one lane per 16-element block, two blocks per lane; a
// wavefront covers a chunk of 128 blocks (2048 elements) of one row, copied
// into its LDS tile with contiguous non-temporal loads, and a workgroup
// covers whole rows (up to 16 chunks), combining the row amax through LDS.
// The chunk stays in LDS and VGPRs between the amax and the block pass, so
// HBM sees every input byte once; rows longer than 16 chunks take a
// one-wave-per-row kernel with a second, L2-served read.  The file also
// holds the TRACE guided quantizer and the global-scale path.
//
// Arithmetic per block and candidate k (each an IEEE binary32 operation, no
// contraction), with the exact equivalences the kernel relies on:
//   t = fl(b / fl(k s)); e = E4M3(t).  With y the hardware reciprocal of
//     fl(k s) (within 2^-22 of it), the kernel forms b * fl(y (1 - 2^-18))
//     and b * fl(y (1 + 2^-18)) -- the factors folded into per-row
//     constants -- which lie strictly below and above t (2^-18 exceeds the
//     2^-22 and three roundings of 2^-24 together); when both give the same
//     E4M3 byte, so does t (rounding is monotone); otherwise it divides.
//   s = fl(amax / C) itself comes from the product with fl(1/C) and one FMA
//     residual correction, the IEEE quotient for every BF16 amax.
//   r = fl(1 / fl(e s)), looked up in each wavefront's LDS table of all
//     E4M3 bytes, filled once per row instead of per block: the hardware
//     reciprocal refined by one FMA residual step, which is the IEEE
//     quotient for every divisor in [2^-126, 2^126] (rows with other
//     divisors divide).  The same entry holds fl(fl(e s)^2) for the
//     certified 4/6 comparison.
//   v = fl(x r); q = E2M1(v) with the sign of x.
//   c = fl(fl(g e) s): g e is exact in FP16 (<= 6 significant bits, between
//     2^-10 and 2688), so the kernel multiplies in packed FP16 and rounds
//     ge * s once with v_fma_mix_f32 (addend -0, which leaves every product
//     unchanged, zeros included).
//   err = sum over the block, in element order, of fl(fl(x - c)^2).
// The E2M1, E4M3 and BF16 conversions are the gfx950 conversion
// instructions, checked exhaustively against the definitions by the tests.
#include "fp4q_device.h"
#include "fp4q_launch.h"

namespace fp4q {

namespace {

// Build-time knob: FP4Q_NV_NT_STORES = 1 writes the outputs with
// non-temporal stores (they are not re-read by this kernel).
#ifndef FP4Q_NV_NT_STORES
#define FP4Q_NV_NT_STORES 1
#endif
// Build-time knobs: FP4Q_NV_NT_BYTES and FP4Q_NV_NT_CODES select which
// block-scale stores (one byte per lane, 64 bytes per instruction) and code
// stores (8 bytes per lane) are non-temporal: 0 none, 1 all, 2 those of
// calls without dequant (measured: plain stores help beside the dequant
// stream, non-temporal ones help without it).
#ifndef FP4Q_NV_NT_BYTES
#define FP4Q_NV_NT_BYTES 2
#endif
#ifndef FP4Q_NV_NT_CODES
#define FP4Q_NV_NT_CODES 2
#endif
// Build-time knobs: the cache-policy bits of the output stores, as the
// gfx950 memory instructions encode them (1 sc0, 2 nt, 16 sc1; -1 none):
//   FP4Q_NV_DQ_POLICY     the BF16 dequant stream;
//   FP4Q_NV_NT_POLICY     the non-temporal code and block-scale stores;
//   FP4Q_NV_PLAIN_POLICY  the other code and block-scale stores (those
//                         beside the dequant stream).
// nt with sc1 on the dequant stream measured faster than nt alone on MI355X
// (the headline 42.6 against 43.6 us and 43.5 against 43.8 us on two boxes,
// the dequant call 23.6 against 23.8 us with distinct codes per call; K0
// writes of 256 MiB 42.1 against 43.5 us); on the code stores of the
// routed-token workload it gained nothing, and sc1 without nt was slower.
// Beside the dequant stream, sc1 on the code and scale stores measured
// 42.67 against 42.82 us (headline, ten rounds side by side; sc0 with sc1
// 42.71) and 310.9 against 311.3 us on expert weights.
#ifndef FP4Q_NV_DQ_POLICY
#define FP4Q_NV_DQ_POLICY (FP4Q_NV_NT_STORES ? 18 : -1)
#endif
#ifndef FP4Q_NV_NT_POLICY
#define FP4Q_NV_NT_POLICY (FP4Q_NV_NT_STORES ? 2 : -1)
#endif
#ifndef FP4Q_NV_PLAIN_POLICY
#define FP4Q_NV_PLAIN_POLICY (FP4Q_NV_NT_STORES ? 16 : -1)
#endif

// Build-time knob: FP4Q_NV_NT_LOADS = 1 makes the contiguous input copies
// into LDS (FP4Q_NV_LDS_LOAD) non-temporal: the input is read once, and each
// of those instructions covers whole cache lines.  Loads straight into
// registers stay ordinary: a lane's block is two 16-byte loads 32 bytes
// apart, so every line is read by two instructions.
#ifndef FP4Q_NV_NT_LOADS
#define FP4Q_NV_NT_LOADS 1
#endif
// Build-time knob: the cache-policy bits of those copies (1 sc0, 2 nt,
// 16 sc1).
#ifndef FP4Q_NV_LOAD_AUX
#define FP4Q_NV_LOAD_AUX (FP4Q_NV_NT_LOADS ? 2 : 0)
#endif

// Build-time knob: FP4Q_NV_LDS_DQ = 1 stages each wave's dequant chunk
// through LDS so that every dequant store instruction writes 1 KiB
// contiguously (16 bytes per lane); 0 stores each lane's 32 bytes directly.
#ifndef FP4Q_NV_LDS_DQ
#define FP4Q_NV_LDS_DQ 1
#endif
// Build-time knob: wavefronts per workgroup the split kernel aims for
// (whole rows per workgroup).  4: rows of one wavefront go four to a
// workgroup (the routed-token workload, 65536 x 2048 without dequant:
// 64.4 us against 65.1 us with two, median of three side by side); longer
// rows are unaffected.
#ifndef FP4Q_NV_WG_WAVES
#define FP4Q_NV_WG_WAVES 4
#endif
// Build-time knob: FP4Q_NV_LDS_LOAD = 1 copies each wave's input chunk
// into LDS with 16-byte-per-lane contiguous loads (global_load_lds) and
// reads the lane's blocks from there.
#ifndef FP4Q_NV_LDS_LOAD
#define FP4Q_NV_LDS_LOAD 1
#endif
// Build-time knob: blocks per lane in the split kernel (1 to 4; 2 measured
// fastest on 2048- and 7168-element rows).
#ifndef FP4Q_NV_NB
#define FP4Q_NV_NB 2
#endif
// Build-time knob: FP4Q_NV_CERTIFY = 0 decides every block of the exact
// 4/6 path from both candidates' errors computed by the definition (the
// straightforward FP32 decision), never from the certified margin below;
// the results are the same.  For measurement only (libfp4q_exactdecision.so).
#ifndef FP4Q_NV_CERTIFY
#define FP4Q_NV_CERTIFY 1
#endif
// Build-time knob: how the split kernel takes its block maxima.  1:
// three-input maxima of the magnitudes of the unpacked FP32 values, which
// the quantization then reuses (8 fewer VALU instructions per block, 16
// more live registers; 65536 x 2048 routed rows without dequant 60.4 ->
// 56.8 us, 65536 x 7168 with dequant 318.6 -> 316.2 us, 8192 x 7168 with
// dequant the same).  0: a packed 16-bit integer maximum of the
// sign-cleared BF16 words, before unpacking.
#ifndef FP4Q_NV_FLOAT_MAX
#define FP4Q_NV_FLOAT_MAX 1
#endif

// Build-time knob: FP4Q_STANDIN = 1 builds a memory-pattern stand-in of the
// split kernel for measurement only (libfp4q_standin.so, never the
// quantizer): the same loads, row amax, row constants, reciprocal tables
// and stores, with each block's quantization replaced by a few XORs of its
// input words, so its time is what this memory pattern costs without the
// per-block arithmetic.
#ifndef FP4Q_STANDIN
#define FP4Q_STANDIN 0
#endif

// Build-time knob: FP4Q_NV_STREAM = 1 quantizes rows of exactly one
// wavefront's chunk (2048 elements) without dequant, with per-token scales,
// with the persistent streaming kernel below.  Off: on the routed-token
// workload (65536 x 2048) it measured 66.3-66.8 us against 63.9-64.6 us for
// the split kernel's one-shot wavefronts, at every grid from 1024 to 4096
// workgroups, with its stores deferred (immediate stores: 68.2 us).
#ifndef FP4Q_NV_STREAM
#define FP4Q_NV_STREAM 0
#endif

// Build-time knob: FP4Q_GLOBAL_REVERSE = 1 quantizes the row groups of the
// global-scale call's second pass from last to first, starting with the
// rows the tensor-max pass read last (60.3 against 60.5 us on moe_act).
#ifndef FP4Q_GLOBAL_REVERSE
#define FP4Q_GLOBAL_REVERSE 1
#endif
// Build-time knob: the cache-policy bits of the global-scale call's second
// pass's input copies (the tensor the max pass has just read): ordinary or
// sc1 copies measured 62.4 us against 60.3 for non-temporal ones.
#ifndef FP4Q_GLOBAL_LOAD_AUX
#define FP4Q_GLOBAL_LOAD_AUX FP4Q_NV_LOAD_AUX
#endif

constexpr int kMaxWgWaves = 16;  // rows of up to 16 waves use the split kernel
constexpr int kLongWaves = 4;    // rows per workgroup of the long-row kernel

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The stores of each output stream, by the policies above.
__device__ __forceinline__ void store_dq(uint4* base, uint32_t idx, uint4 v) {
  put<FP4Q_NV_DQ_POLICY>(base, idx, v);
}
// A block-scale byte and a block's code word: non-temporal per
// FP4Q_NV_NT_BYTES and FP4Q_NV_NT_CODES (DQ: the call also writes the
// dequant).
// Build-time knobs: the block-scale stores' own policies (by default those
// of the code stores); sc1 measured slower on the routed-token call (58.3
// against 58.0 us) and the same on the headline.
#ifndef FP4Q_NV_SCALE_NT_POLICY
#define FP4Q_NV_SCALE_NT_POLICY FP4Q_NV_NT_POLICY
#endif
#ifndef FP4Q_NV_SCALE_PLAIN_POLICY
#define FP4Q_NV_SCALE_PLAIN_POLICY FP4Q_NV_PLAIN_POLICY
#endif
// Build-time knobs: the cache-policy bits of the guided call's code stores
// (4 bytes per lane) with a guide, and without one (round to nearest).
// Measured on moe_act (guided / to nearest, us): nt 28.1 / 25.2; sc1
// 32.3 / 24.2; none 33.5 / 25.2; sc0 33.5 / 25.2; nt with sc1 28.1 / 25.2.
#ifndef FP4Q_GUIDED_CODE_POLICY
#define FP4Q_GUIDED_CODE_POLICY 2
#endif
#ifndef FP4Q_RTN_CODE_POLICY
#define FP4Q_RTN_CODE_POLICY 16
#endif
template <bool DQ>
__device__ __forceinline__ void store_scale(uint8_t* base, uint32_t idx, uint8_t v) {
  if constexpr (FP4Q_NV_NT_BYTES == 1 || (FP4Q_NV_NT_BYTES == 2 && !DQ))
    put<FP4Q_NV_SCALE_NT_POLICY>(base, idx, v);
  else
    put<FP4Q_NV_SCALE_PLAIN_POLICY>(base, idx, v);
}
// NTC: non-temporal whatever the knob says -- the quantize pass of the
// global-scale call, whose plain code stores would leave dirty lines for the
// next call's tensor-max pass to write back (62 vs 68 us on moe_act).
template <bool DQ, bool NTC>
__device__ __forceinline__ void store_codes(uint2* base, uint32_t idx, uint2 v) {
  if constexpr (NTC || FP4Q_NV_NT_CODES == 1 || (FP4Q_NV_NT_CODES == 2 && !DQ))
    put<FP4Q_NV_NT_POLICY < 0 ? 2 : FP4Q_NV_NT_POLICY>(base, idx, v);
  else
    put<FP4Q_NV_PLAIN_POLICY>(base, idx, v);
}
// Code words of the guided call (one lane per 8 elements); RTN: without a
// guide.
template <bool RTN>
__device__ __forceinline__ void store_words(uint32_t* base, uint32_t idx, uint32_t v) {
  put<RTN ? FP4Q_RTN_CODE_POLICY : FP4Q_GUIDED_CODE_POLICY>(base, idx, v);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Wave-wide max of a non-negative value (DPP row shifts, then the row
// broadcasts; lane 63 ends with the max of all 64 lanes).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<0x111, 0xF>(v));  // row_shr:1
  v = max(v, dpp<0x112, 0xF>(v));  // row_shr:2
  v = max(v, dpp<0x114, 0xF>(v));  // row_shr:4
  v = max(v, dpp<0x118, 0xF>(v));  // row_shr:8
  v = max(v, dpp<0x142, 0xA>(v));  // row_bcast:15
  v = max(v, dpp<0x143, 0xC>(v));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The tensor-max pass's per-workgroup maxima, as 16-bit BF16 magnitude
// patterns, zero-padded to whole 16-byte units: at most 512 of them, so one
// 16-byte load per lane covers them all.  The load is issued before the
// chunk's own loads, so its latency hides under theirs.
__device__ __forceinline__ uint4 load_partials(const uint4* __restrict__ part, int n16,
                                               int lane) {
  return lane < n16 ? part[lane] : make_uint4(0u, 0u, 0u, 0u);
}
// The tensor amax as the bit pattern of a non-negative float.
__device__ __forceinline__ uint32_t tensor_amax(uint4 p) {
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 m = __builtin_elementwise_max(
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, p.x), __builtin_bit_cast(u16x2, p.y)),
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, p.z), __builtin_bit_cast(u16x2, p.w)));
  return wave_max_u32((uint32_t)max(m.x, m.y) << 16);
}

__device__ __forceinline__ void unpack16(const uint32_t (&w)[8], float (&x)[16]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[2 * k] = bf16_lo(w[k]);
    x[2 * k + 1] = bf16_hi(w[k]);
  }
}

// Max |x| of a block as the bit pattern of a non-negative float: a packed
// 16-bit max over the sign-cleared BF16 patterns (for non-negative values
// the integer order is the value order).
__device__ __forceinline__ uint32_t block_absmax_bits(const uint32_t (&w)[8]) {
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) m[k] = __builtin_bit_cast(u16x2, w[k] & 0x7FFF7FFFu);
#pragma unroll
  for (int n = 4; n >= 1; n >>= 1)
#pragma unroll
    for (int k = 0; k < n; ++k) m[k] = __builtin_elementwise_max(m[k], m[k + n]);
  return (uint32_t)max(m[0].x, m[0].y) << 16;
}

// The same from the block's FP32 values (BF16 widened exactly): max |x| by
// IEEE maximum, which returns one operand unchanged (denormals preserved),
// so its bits are the sign-cleared BF16 pattern shifted up, as above, for
// every finite or infinite input (NaN inputs are outside the domain).
__device__ __forceinline__ uint32_t block_absmax_f(const float (&x)[16]) {
  auto mx3 = [](float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
  };
  float a[5];
#pragma unroll
  for (int k = 0; k < 5; ++k)
    a[k] = mx3(__builtin_fabsf(x[3 * k]), __builtin_fabsf(x[3 * k + 1]),
               __builtin_fabsf(x[3 * k + 2]));
  const float m = __builtin_elementwise_maximum(mx3(a[0], a[1], a[2]),
                                                mx3(a[3], a[4], __builtin_fabsf(x[15])));
  return __float_as_uint(m);
}

// Per-row constants.
struct RowScale {
  float s;           // token scale, stored
  float ks6, ks4;    // fl(6 s), fl(4 s); 1 for a zero row (so b / ks = 0)
  // approximate reciprocals of ks6 and ks4 times 1 - 2^-18 and 1 + 2^-18:
  // b times them brackets the block scale (see quantize_block_fast)
  float rks6_lo, rks6_hi, rks4_lo, rks4_hi;
  bool fast;         // every decode step e s is 0 or >= 2^-127
  bool certify;      // 2^-50 <= s <= 2^40: the error enclosure applies
  bool rcp_normal;   // 2^-117 <= s <= 2^116: every nonzero e s in [2^-126, 2^126]
  float inv_s;       // fl(1 / s), for the FP16 decision (FOS == 2)
};

// Row constants from the token scale s itself (non-negative, uniform across
// the wavefront).  Its bit pattern orders like its value, so the range
// tests are integer compares on a scalar register.
template <int FOS>
__device__ __forceinline__ RowScale row_scale_s(float s_in) {
  RowScale r;
  const uint32_t sb = __builtin_amdgcn_readfirstlane(__float_as_uint(s_in));
  r.s = __uint_as_float(sb);
  const bool zero = sb == 0u;
  r.ks6 = zero ? 1.0f : 6.0f * r.s;
  r.ks4 = zero ? 1.0f : 4.0f * r.s;
  const float rks6 = __builtin_amdgcn_rcpf(r.ks6), rks4 = __builtin_amdgcn_rcpf(r.ks4);
  r.rks6_lo = rks6 * (1.0f - 0x1p-18f);
  r.rks6_hi = rks6 * (1.0f + 0x1p-18f);
  r.rks4_lo = rks4 * (1.0f - 0x1p-18f);
  r.rks4_hi = rks4 * (1.0f + 0x1p-18f);
  // s >= 2^-118: ks >= 2^-116 so 1/ks is normal, and the smallest decode
  // step 2^-9 s >= 2^-127 has a finite reciprocal.
  r.fast = (sb >= 0x04800000u && sb <= 0x7F800000u) || zero;  // 2^-118 .. inf
  r.certify = sb >= 0x26800000u && sb <= 0x53800000u;         // 2^-50 .. 2^40
  r.rcp_normal = sb >= 0x05000000u && sb <= 0x79800000u;      // 2^-117 .. 2^116
  r.inv_s = FOS == 2 ? 1.0f / r.s : 0.0f;
  return r;
}

// Row constants from the row amax (a non-negative float's bit pattern):
// s = fl(amax / C).
template <int FOS>
__device__ __forceinline__ RowScale row_scale(uint32_t amax_bits) {
  return row_scale_s<FOS>(amax_over_c(__uint_as_float(amax_bits), FOS != 0));
}

// tab[byte] = {1 / fl(e(byte) s), fl(e(byte) s)^2} for all 128 E4M3 bytes,
// lane l of the wavefront writing bytes l and l + 64.
__device__ __forceinline__ void fill_recip(float2v* tab, const RowScale& rs, int lane) {
  // For s in [2^-117, 2^116] every nonzero e*s (e from 2^-9 to 448) lies in
  // [2^-126, 2^126], where the refined hardware reciprocal is the IEEE
  // quotient; other rows divide.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int byte = lane + 64 * h;
    const float d = e4m3_value<0>((uint32_t)byte) * rs.s;
    const float r = rs.rcp_normal ? recip_normal(d) : 1.0f / d;
    tab[byte] = (float2v){(d != 0.0f) ? r : 0.0f, d * d};
  }
}

// Codes of one candidate, and (APPROX) A = sum over the block of
// (v - g)^2 in FP32 with fused multiply-adds: the candidate's error in units
// of its decode step, used by the certified comparison below.
template <bool APPROX>
__device__ __forceinline__ void encode_candidate(const float (&x)[16], float r,
                                                 uint32_t (&code)[2], float& A) {
  A = 0.0f;
  static_for<0, 2>([&](auto H) {
    constexpr int h = decltype(H)::value;
    float v[8];
    uint32_t word = any_word();  // bytes 0-3 all written below
    static_for<0, 4>([&](auto P) {
      constexpr int p = decltype(P)::value;
      v[2 * p] = x[8 * h + 2 * p] * r;
      v[2 * p + 1] = x[8 * h + 2 * p + 1] * r;
      word = cvt_e2m1x2<p>(word, v[2 * p], v[2 * p + 1]);
    });
    code[h] = word;
    if (APPROX) {
      // decoded from the finished word: each byte is final once written
      static_for<0, 4>([&](auto P) {
        constexpr int p = decltype(P)::value;
        const float2v g = e2m1x2_values<p>(word);
        const float a0 = v[2 * p] - g.x, a1 = v[2 * p + 1] - g.y;  // exact (Sterbenz; g = 0 gives v)
        A = __builtin_fmaf(a0, a0, A);
        A = __builtin_fmaf(a1, a1, A);
      });
    }
  });
  // computed here, while v is live, not sunk into the branch that reads it
  if (APPROX) asm volatile("" : "+v"(A));
}

// The candidate's squared error by the definition: c = fl(fl(g e) s),
// err = sum in element order of fl(fl(x - c)^2).  g e is exact in FP16
// (<= 6 significant bits, between 2^-10 and 2688); v_fma_mix_f32 with the
// addend -0 rounds ge * s once and leaves every product unchanged.
__device__ __forceinline__ float exact_error(const float (&x)[16], const uint32_t (&code)[2],
                                             float e, float s, float neg_zero) {
  const _Float16 eh = (_Float16)e;  // exact: E4M3 values are FP16 numbers
  const half2v e2 = {eh, eh};
  float err = 0.0f;
  static_for<0, 8>([&](auto P) {
    constexpr int p = decltype(P)::value;
    const half2v ge = e2m1x2_values_f16<p & 3>(code[p >> 2]) * e2;
    const float c0 = __builtin_fmaf((float)ge.x, s, neg_zero);
    const float c1 = __builtin_fmaf((float)ge.y, s, neg_zero);
    const float d0 = x[2 * p] - c0, d1 = x[2 * p + 1] - c1;
    const float q0 = d0 * d0, q1 = d1 * d1;
    err = err + q0;
    err = err + q1;
  });
  return err;
}

// The chosen candidate's values c = fl(fl(g e) s) rounded to BF16.
__device__ __forceinline__ void dequant_block(const uint32_t (&code)[2], float e, float s,
                                              float neg_zero, uint32_t (&deq)[8]) {
  const _Float16 eh = (_Float16)e;
  const half2v e2 = {eh, eh};
  static_for<0, 8>([&](auto P) {
    constexpr int p = decltype(P)::value;
    const half2v ge = e2m1x2_values_f16<p & 3>(code[p >> 2]) * e2;
    deq[p] = cvt_bf16x2(__builtin_fmaf((float)ge.x, s, neg_zero),
                        __builtin_fmaf((float)ge.y, s, neg_zero));
  });
}

// The FP16 fast path's error of one candidate (FOS == 2; NVFP4-RL blog,
// section 4, "The optimization"): targets y = FP16(x / s) (signed, from
// fl(x * inv_s)), candidate values g e exact in FP16, differences rounded
// to FP16, squares (exact in FP32) summed in FP32 in element order --
// v_fma_mix_f32 of an exact square and the running sum rounds once, as the
// separate multiply and add would.  Signed targets and signed candidate
// values give the same squares as magnitudes.
__device__ __forceinline__ float fp16_error(const half2v (&y)[8], const uint32_t (&code)[2],
                                            float e) {
  const _Float16 eh = (_Float16)e;
  const half2v e2 = {eh, eh};
  float err = 0.0f;
  static_for<0, 8>([&](auto P) {
    constexpr int p = decltype(P)::value;
    const half2v ge = e2m1x2_values_f16<p & 3>(code[p >> 2]) * e2;  // exact
    const half2v d = y[p] - ge;                                      // FP16 rounding
    err = __builtin_fmaf((float)d.x, (float)d.x, err);
    err = __builtin_fmaf((float)d.y, (float)d.y, err);
  });
  return err;
}

// Certified 4/6 decision from each candidate's A and D2 = fl(D^2), D =
// fl(e s) the decode step, for rows with 2^-50 <= s <= 2^40 and both e != 0.
// Each candidate's FP32 error err (as the definition computes it) is close
// to D^2 A.  With u = 2^-24: v = x r and the candidate value c carry relative
// rounding errors, so each x - c differs from D (v - g) by at most
// D 2.01u (|v| + |g|) <= D 32.2u (|v| < 10, |g| <= 6); summed over 16
// elements (Cauchy-Schwarz on the cross term),
// |sum (x-c)^2 - D^2 S| <= D^2 (258u sqrt(S) + 0.001u) with S the exact sum
// of (v - g)^2, and sqrt(S) <= (S + 1) / 2 makes that at most
// D^2 (129u S + 129.001u).  A = S (1 +- 16.1u); the FP32 error is
// sum (x-c)^2 (1 +- 18.1u), plus at most 2^-145 from underflow, which is
// below D^2 u / 8 because D >= 2^-9 s >= 2^-59 here.  Together:
//   |err - D^2 A| <= D^2 (163.4u A + 129.3u).
// So with P = D4^2 A4 and Q = D6^2 A6, the 4 candidate's error is certainly
// lower when Q - P > 163.4u (P + Q) + 129.3u (D4^2 + D6^2), and certainly
// not lower (6 kept, ties included) when P - Q exceeds the same margin.
// Below, P, Q, their difference and sum, D4^2 + D6^2 and the margin M are
// each one FP32 rounding (relative u each, D2 = fl(D^2) one more), so the
// computed Q - P is within 2.01u (P + Q) of the exact one and the computed
// M is at least 329.9u (P + Q) + 259.9u (D4^2 + D6^2): a computed
// |Q - P| > M implies the exact difference exceeds 327u (P + Q) +
// 259u (D4^2 + D6^2), twice the margin needed.  The range of s keeps every
// D^2 normal and every product finite.  Returns whether the decision is
// certified; four says which.
__device__ __forceinline__ bool certified_four(float A6, float D2_6, float A4, float D2_4,
                                               bool& four) {
  constexpr float u = 0x1p-24f;
  const float P = D2_4 * A4, Q = D2_6 * A6;
  const float diff = Q - P;
  const float M = __builtin_fmaf(P + Q, 330.0f * u, (D2_4 + D2_6) * (260.0f * u));
  four = diff > M;
  return fabsf(diff) > M;
}

// One element of a candidate by the portable definition: |x| r may be
// +inf (code 7) or NaN (0 * inf, code 0).  Returns the nibble and the FP32
// candidate value.
__device__ __forceinline__ uint32_t element_portable(float x, float e, float r, float s,
                                                     float& c) {
  const uint32_t neg = __float_as_uint(x) >> 31;
  float g;
  const uint32_t q = e2m1_code_sw(fabsf(x) * r, g);
  const float ge = g * e;
  c = ge * s;
  c = neg ? -c : c;
  return q | (neg << 3);
}

// Rows with s < 2^-118 (row amax below about 2^-107): decode steps may be
// subnormal and their reciprocals infinite, so the block follows the
// definition step by step -- exact division for the block scale, portable
// rounding -- in loops that re-read the block from memory.  Nothing here
// stays live across the hot path, so it costs the common case no registers.
template <int FOS, bool DQ>
__device__ __attribute__((noinline)) void tiny_row_block(const uint16_t* __restrict__ xb,
                                                         float b, const float2v* tab, float s,
                                                         float inv_s,
                                                         uint8_t* __restrict__ code_bytes,
                                                         uint8_t* __restrict__ scale,
                                                         uint16_t* __restrict__ dqb) {
  float best_err = 0.0f, best_e = 0.0f, best_r = 0.0f;
  uint32_t best_byte = 0u;
#pragma unroll 1
  for (int k = 0; k < (FOS ? 2 : 1); ++k) {
    float e = 0.0f;
    uint32_t byte = 0u;
    if (b != 0.0f) byte = e4m3_encode(b / ((k == 0 ? 6.0f : 4.0f) * s), e);
    const float r = tab[byte].x;
    float err = 0.0f;
#pragma unroll 1
    for (int i = 0; i < 16; ++i) {
      const float xi = __uint_as_float((uint32_t)xb[i] << 16);
      float c;
      const uint32_t q = element_portable(xi, e, r, s, c);
      if (FOS == 2) {  // the FP16 fast path's error (see fp16_error)
        const half2v y = {(_Float16)(fabsf(xi) * inv_s), (_Float16)0.0f};
        const half2v ge = {(_Float16)(e2m1_value(q & 7u) * e), (_Float16)0.0f};  // exact
        const half2v d = y - ge;
        err = __builtin_fmaf((float)d.x, (float)d.x, err);
      } else {
        const float d = xi - c;
        const float sq = d * d;
        err = err + sq;
      }
    }
    if (k == 0 || err < best_err) {  // strictly lower error: 4 wins
      best_err = err;
      best_e = e;
      best_r = r;
      best_byte = byte;
    }
  }
  *scale = (uint8_t)best_byte;
#pragma unroll 1
  for (int i = 0; i < 16; i += 2) {
    float c0, c1;
    const uint32_t n0 =
        element_portable(__uint_as_float((uint32_t)xb[i] << 16), best_e, best_r, s, c0);
    const uint32_t n1 =
        element_portable(__uint_as_float((uint32_t)xb[i + 1] << 16), best_e, best_r, s, c1);
    code_bytes[i / 2] = (uint8_t)(n0 | (n1 << 4));
    if (DQ) {
      const uint32_t pair = cvt_bf16x2(c0, c1);
      dqb[i] = (uint16_t)pair;
      dqb[i + 1] = (uint16_t)(pair >> 16);
    }
  }
}

// Outputs of one block on the fast path.
struct BlockOut {
  uint32_t code0, code1, ebyte;
  uint32_t deq[8];
};

template <int FOS, bool DQ>
__device__ __forceinline__ void quantize_block_fast(const float (&x)[16], uint32_t bbits,
                                                    const RowScale& rs, const float2v* tab,
                                                    float neg_zero, BlockOut& out) {
  const float b = __uint_as_float(bbits);
  // bracketed block scales for both candidates (byte 0: map to 6, byte 1:
  // map to 4)
  const uint32_t lo = cvt_e4m3x2(b * rs.rks6_lo, FOS ? b * rs.rks4_lo : 0.0f);
  uint32_t eb = cvt_e4m3x2(b * rs.rks6_hi, FOS ? b * rs.rks4_hi : 0.0f);
  if (__builtin_expect(lo != eb, 0))
    eb = cvt_e4m3x2(fminf(b / rs.ks6, 448.0f), FOS ? fminf(b / rs.ks4, 448.0f) : 0.0f);
  const float2v t6 = tab[eb & 0xFFu];  // {r, D^2} of the 6 candidate
  uint32_t code[2];
  float A6;
  encode_candidate<FOS == 1 && FP4Q_NV_CERTIFY>(x, t6.x, code, A6);
  uint32_t ebyte = eb & 0xFFu;
  if (FOS) {
    const float2v t4 = tab[eb >> 8];
    uint32_t code4[2];
    float A4;
    encode_candidate<FOS == 1 && FP4Q_NV_CERTIFY>(x, t4.x, code4, A4);
    bool four;
    if (FOS == 2) {
      half2v y[8];
      static_for<0, 8>([&](auto P) {
        constexpr int p = decltype(P)::value;
        y[p] = __builtin_convertvector((float2v){x[2 * p] * rs.inv_s, x[2 * p + 1] * rs.inv_s},
                                       half2v);
      });
      four = fp16_error(y, code4, e4m3_value<1>(eb)) <
             fp16_error(y, code, e4m3_value<0>(eb));  // ties keep 6
    } else {
      // 4 wins only with a strictly lower error; both scales zero: the same
      // error, keep 6
      four = false;
      bool decided = eb == 0u;
      // both e nonzero: the 4 candidate's byte is never below the 6
      // candidate's (both round b / (k s) to nearest, monotonically, and
      // b / (6 s) < b / (4 s)), so a nonzero 6 byte is enough
      if (FP4Q_NV_CERTIFY && rs.certify && (eb & 0xFFu) != 0u)
        decided = certified_four(A6, t6.y, A4, t4.y, four);
      if (__builtin_expect(!decided, 0))
        four = exact_error(x, code4, e4m3_value<1>(eb), rs.s, neg_zero) <
               exact_error(x, code, e4m3_value<0>(eb), rs.s, neg_zero);
    }
    code[0] = four ? code4[0] : code[0];
    code[1] = four ? code4[1] : code[1];
    ebyte = four ? (eb >> 8) : ebyte;
  }
  out.code0 = code[0];
  out.code1 = code[1];
  out.ebyte = ebyte;
  if (DQ) dequant_block(code, e4m3_value<0>(ebyte), rs.s, neg_zero, out.deq);
}

// One block, written directly (one lane, 32 contiguous dequant bytes).
// xin, codes, scales and dq point at block 0 of the wavefront's chunk
// (wave-uniform, so the stores take a scalar base and a 32-bit lane
// offset); blk is the block within it.
template <int FOS, bool DQ, bool NTC>
__device__ __forceinline__ void quantize_block(const float (&x)[16], uint32_t bbits,
                                               const RowScale& rs, const float2v* tab,
                                               float neg_zero, const uint4* __restrict__ xin,
                                               int blk, uint2* __restrict__ codes,
                                               uint8_t* __restrict__ scales,
                                               uint4* __restrict__ dq,
                                               uint4* stage = nullptr) {
  if (__builtin_expect(!rs.fast, 0)) {
    tiny_row_block<FOS, DQ>((const uint16_t*)(xin + 2 * blk), __uint_as_float(bbits), tab, rs.s,
                            rs.inv_s,
                            (uint8_t*)(codes + blk), scales + blk,
                            DQ ? (uint16_t*)(dq + 2 * blk) : nullptr);
    return;
  }
  BlockOut o;
  quantize_block_fast<FOS, DQ>(x, bbits, rs, tab, neg_zero, o);
  store_codes<DQ, NTC>(codes, blk, make_uint2(o.code0, o.code1));
  store_scale<DQ>(scales, blk, (uint8_t)o.ebyte);
  if (DQ) {
    if (stage != nullptr) {  // the caller writes the chunk out contiguously
      stage[0] = make_uint4(o.deq[0], o.deq[1], o.deq[2], o.deq[3]);
      stage[1] = make_uint4(o.deq[4], o.deq[5], o.deq[6], o.deq[7]);
    } else {
      store_dq(dq, 2 * blk, make_uint4(o.deq[0], o.deq[1], o.deq[2], o.deq[3]));
      store_dq(dq, 2 * blk + 1, make_uint4(o.deq[4], o.deq[5], o.deq[6], o.deq[7]));
    }
  }
}

// The stand-in's block (FP4Q_STANDIN): the stores of quantize_block, with
// codes, scale byte and dequant values taken from the input words.
template <bool DQ, bool NTC>
__device__ __forceinline__ void standin_block(const uint32_t (&w)[8], uint32_t bbits,
                                              int blk, uint2* __restrict__ codes,
                                              uint8_t* __restrict__ scales,
                                              uint4* __restrict__ dq, uint4* stage) {
  store_codes<DQ, NTC>(codes, blk, make_uint2(w[0] ^ w[2] ^ w[4] ^ w[6], w[1] ^ w[3] ^ w[5] ^ w[7]));
  store_scale<DQ>(scales, blk, (uint8_t)(bbits >> 24));
  if (DQ) {
    if (stage != nullptr) {
      stage[0] = make_uint4(w[0], w[1], w[2], w[3]);
      stage[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      store_dq(dq, 2 * blk, make_uint4(w[0], w[1], w[2], w[3]));
      store_dq(dq, 2 * blk + 1, make_uint4(w[4], w[5], w[6], w[7]));
    }
  }
}

// a < b for int64 values, from the signed high and unsigned low words, so
// that wave-uniform operands are compared by the scalar unit
__device__ __forceinline__ bool lt_i64(int64_t a, int64_t b) {
  const int ah = (int)(a >> 32), bh = (int)(b >> 32);
  const uint32_t al = (uint32_t)a, bl = (uint32_t)b;
  return ah < bh || (ah == bh && al < bl);
}

__device__ __forceinline__ bool row_range(int64_t row, int64_t rows, const int64_t* offs,
                                          int64_t ngroups) {
  int64_t lo = 0, hi = rows;
  if (offs != nullptr) {
    lo = max(offs[0], (int64_t)0);
    hi = min(offs[ngroups], rows);
  }
  return row >= lo && row < hi;
}

__device__ __forceinline__ uint4 load_in(const uint4* p) { return *p; }

__device__ __forceinline__ void load_block(const uint4* __restrict__ x, int64_t blk,
                                           uint32_t (&w)[8]) {
  const uint4 a = load_in(&x[2 * blk]), b = load_in(&x[2 * blk + 1]);
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// Split rows: a workgroup holds R rows x W wavefronts; wave c of a row owns
// chunk c of it -- 64 * NB consecutive blocks, lane l taking blocks l and
// l + 64 (NB = 2) -- so each lane quantizes NB blocks per pass.  The row
// amax is combined across the W waves through LDS; then every wave derives
// the row constants and fills its own reciprocal table.  Row and chunk are
// wave-uniform, so all addressing is scalar base + 32-bit lane offset.
// Rows of group g this wave works on: row, the blocks of its chunk that
// exist (0 for a row outside the range or past the end), their first index.
struct ChunkRef {
  int64_t row, cbase;
  int valid;
  bool active;
};
template <int NB>
__device__ __forceinline__ ChunkRef chunk_ref(int64_t g, int rw, int chunk, int R, int nblk,
                                              int64_t row0, int64_t row_end, int64_t rows,
                                              const int64_t* offs, int64_t ngroups) {
  ChunkRef c;
  c.row = row0 + g * R + rw;
  // row < row_end <= rows, and row >= 0, so only the group range is left
  // to check; the comparisons stay in scalar registers
  c.active = lt_i64(c.row, row_end) &&
             (offs == nullptr || (!lt_i64(c.row, offs[0]) && lt_i64(c.row, offs[ngroups])));
  c.valid = c.active ? min(64 * NB, nblk - chunk * 64 * NB) : 0;
  c.cbase = c.row * nblk + (int64_t)chunk * 64 * NB;
  return c;
}

template <int NB>
__device__ __forceinline__ void load_chunk(const uint4* __restrict__ x, const ChunkRef& c,
                                           int lane, uint32_t (&w)[NB][8]) {
  const uint4* xc = x + 2 * c.cbase;
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    if (64 * n < c.valid) {  // wave-uniform: the block slot exists for some lane
      load_block(xc, min(lane + 64 * n, c.valid - 1), w[n]);  // in bounds for every lane
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) w[n][k] = 0u;
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// The same chunk through LDS: every lane copies 16 consecutive bytes per
// instruction straight into the wave's LDS tile (1 KiB contiguous per
// instruction), then reads its own blocks back.  Lanes whose half-block
// lies past the chunk's end copy nothing.
template <int NB, int kAux = FP4Q_NV_LOAD_AUX>
__device__ __forceinline__ void issue_chunk_lds(const uint4* __restrict__ x, int64_t cbase,
                                                int valid, int lane, uint4* tile) {
  const uint4* xc = x + 2 * cbase;
  if (valid == 64 * NB) {
    // a whole chunk: one base pair, the KiB steps in the instruction's
    // offset, which moves the global and the LDS address alike
    static_for<0, 2 * NB>([&](auto I) {
      constexpr int i = decltype(I)::value;
      __builtin_amdgcn_global_load_lds(xc + lane, (lds_void*)tile, 16, 1024 * i, kAux);
    });
  } else {
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int q = 128 * n + 64 * k + lane;  // 16-byte unit of the chunk
        if (64 * n < valid && (q >> 1) < valid)
          __builtin_amdgcn_global_load_lds(xc + q, (lds_void*)(tile + 128 * n + 64 * k), 16, 0,
                                           kAux);
      }
  }
}

// The lane's NB blocks from the wave's tile.  Slots past the chunk's end
// read whatever the tile holds; the caller uses only blocks below valid.
template <int NB>
__device__ __forceinline__ void read_tile(const uint4* tile, int lane, uint32_t (&w)[NB][8]) {
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const uint4 a = tile[128 * n + 2 * lane], b = tile[128 * n + 2 * lane + 1];
    w[n][0] = a.x; w[n][1] = a.y; w[n][2] = a.z; w[n][3] = a.w;
    w[n][4] = b.x; w[n][5] = b.y; w[n][6] = b.z; w[n][7] = b.w;
  }
}

template <int NB, int kAux = FP4Q_NV_LOAD_AUX>
__device__ __forceinline__ void load_chunk_lds(const uint4* __restrict__ x, const ChunkRef& c,
                                               int lane, uint4* tile, uint32_t (&w)[NB][8]) {
  issue_chunk_lds<NB, kAux>(x, c.cbase, c.valid, lane, tile);
  __builtin_amdgcn_s_waitcnt(0);  // the copies have landed in LDS
  read_tile<NB>(tile, lane, w);
}

template <int FOS, bool DQ, int NB, bool NTC>
__global__ __launch_bounds__(64 * kMaxWgWaves) void nvfp4_quantize_split(
    const uint4* __restrict__ x, int64_t rows, int64_t row0, int64_t row_end, int nblk, int W,
    int wdiv, int R, const int64_t* __restrict__ offs, int64_t ngroups,
    uint2* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tscale, uint4* __restrict__ dq,
    float neg_zero, const uint4* __restrict__ gpart, int npart16,
    float* __restrict__ gscale_out) {
  __shared__ uint32_t wave_max[kMaxWgWaves];
  // dynamic LDS: the reciprocal table of each wave (W R x 128 entries of
  // two floats), then the waves' tiles
  extern __shared__ uint4 dyn_lds[];
  float2v(*recip)[128] = (float2v(*)[128])dyn_lds;
  constexpr bool kLdsLoad = FP4Q_NV_LDS_LOAD;
  // per wave: the input tile (NB x 2 KiB) when loading through LDS, whose
  // half n, once read, stages the dequant values of block group n; else
  // 2 KiB of staging
  constexpr int kWaveLds = kLdsLoad ? 128 * NB : 128;
  // NTC marks the global-scale call's quantize pass, the one instantiation
  // that gets the tensor-max pass's partials (gpart) and no token scales
  constexpr bool kGlobal = NTC;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint4* wave_lds = dyn_lds + 64 * W * R + kWaveLds * wave;
  // wave / W as a scalar multiply and shift: wdiv = ceil(2^16 / W) is exact
  // for every wave < 16 and W <= 16
  const int rw = (wave * wdiv) >> 16, chunk = wave - rw * W;  // wave-uniform

  // with one scale for the whole tensor (FP4Q_GLOBAL_REVERSE) the row
  // groups go last to first, so that the rows the tensor-max pass read last
  // -- the likeliest still in the last-level cache -- are read first
  const int64_t g = (FP4Q_GLOBAL_REVERSE && kGlobal) ? gridDim.x - 1 - blockIdx.x
                                                               : blockIdx.x;
  uint4 gp = make_uint4(0u, 0u, 0u, 0u);
  uint32_t w[NB][8];
  ChunkRef c;
  if (kLdsLoad) {
    // the copies start as soon as the row is known to be in this launch
    // (every such row is in the tensor); whether the row lies in the group
    // range (two values read from memory) is settled while they are in
    // flight.  The tensor-max pass's partials go first (60.2 against 60.4 us
    // for the global-scale call with them after the copies).
    if (kGlobal) gp = load_partials(gpart, npart16, lane);
    const int64_t row = row0 + g * R + rw;
    const int lvalid = lt_i64(row, row_end) ? min(64 * NB, nblk - chunk * 64 * NB) : 0;
    issue_chunk_lds<NB, NTC ? FP4Q_GLOBAL_LOAD_AUX : FP4Q_NV_LOAD_AUX>(
        x, row * nblk + (int64_t)chunk * 64 * NB, lvalid, lane, wave_lds);
    c = chunk_ref<NB>(g, rw, chunk, R, nblk, row0, row_end, rows, offs, ngroups);
    __builtin_amdgcn_s_waitcnt(0);  // the copies have landed in LDS
    read_tile<NB>(wave_lds, lane, w);
  } else {
    if (kGlobal) gp = load_partials(gpart, npart16, lane);
    c = chunk_ref<NB>(g, rw, chunk, R, nblk, row0, row_end, rows, offs, ngroups);
    load_chunk<NB>(x, c, lane, w);
  }
  // the blocks' values (FP32), unpacked once for the block maxima and the
  // quantization (FP4Q_NV_FLOAT_MAX)
  constexpr bool kFloatMax = FP4Q_NV_FLOAT_MAX && !FP4Q_STANDIN;
  float xv[NB][16];
  uint32_t bmax[NB];
  uint32_t lmax = 0;
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    if (kFloatMax) {
      unpack16(w[n], xv[n]);
      bmax[n] = lane + 64 * n < c.valid ? block_absmax_f(xv[n]) : 0u;
    } else {
      bmax[n] = lane + 64 * n < c.valid ? block_absmax_bits(w[n]) : 0u;
    }
    lmax = max(lmax, bmax[n]);
  }

  // the row amax: a one-wave row has it already; otherwise the row's waves
  // combine theirs through LDS.  Every wave then derives the row constants
  // and fills its own reciprocal table, so the row needs no second
  // workgroup barrier.  With gpart (one scale for the whole tensor) every
  // wave reduces the tensor-max pass's partial maxima itself and the row
  // needs no barrier at all.
  uint32_t amax_bits;
  if (kGlobal) {
    amax_bits = tensor_amax(gp);
  } else {
    amax_bits = wave_max_u32(lmax);
    if (W > 1) {  // uniform over the workgroup
      if (lane == 0) wave_max[wave] = amax_bits;
      __syncthreads();
      amax_bits = 0;
      for (int k = 0; k < W; ++k) amax_bits = max(amax_bits, wave_max[rw * W + k]);
    }
  }
  const RowScale rs = row_scale<FOS>(amax_bits);
  if (chunk == 0 && lane == 0 && c.active && tscale != nullptr) tscale[c.row] = rs.s;
  if (gscale_out != nullptr && row0 == 0 && blockIdx.x == 0 && wave == 0 && lane == 0)
    *gscale_out = rs.s;
  float2v* tab = recip[wave];
  fill_recip(tab, rs, lane);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr bool kStage = FP4Q_NV_LDS_DQ && DQ;
  const bool stage = kStage && rs.fast;  // wave-uniform
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int j = lane + 64 * n;
    uint4* dq_stage_n = wave_lds + (kLdsLoad ? 128 * n : 0);
    if (64 * n < c.valid && j < c.valid) {
      if (FP4Q_STANDIN) {
        standin_block<DQ, NTC>(w[n], bmax[n], j, codes + c.cbase, scales + c.cbase,
                               DQ ? dq + 2 * c.cbase : nullptr,
                               stage ? &dq_stage_n[2 * lane] : nullptr);
      } else {
        if (!kFloatMax) unpack16(w[n], xv[n]);
        quantize_block<FOS, DQ, NTC>(xv[n], bmax[n], rs, tab, neg_zero, x + 2 * c.cbase, j,
                                     codes + c.cbase, scales + c.cbase,
                                     DQ ? dq + 2 * c.cbase : nullptr,
                                     stage ? &dq_stage_n[2 * lane] : nullptr);
      }
    }
    if (stage && 64 * n < c.valid) {
      // the group's dequant values leave as two contiguous KiB
      const int nv = min(64, c.valid - 64 * n);  // blocks of this group
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      uint4* dqc = dq + 2 * (c.cbase + 64 * n);
      if (lane < 2 * nv) store_dq(dqc, lane, dq_stage_n[lane]);
      if (64 + lane < 2 * nv) store_dq(dqc, 64 + lane, dq_stage_n[64 + lane]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// Rows of exactly one wavefront's chunk (64 NB blocks: 2048 elements)
// without dequant, persistent (FP4Q_NV_STREAM): wavefront g of a grid of G
// quantizes rows lo + g, lo + g + G, ...  The
// next row's chunk is copied into the wavefront's LDS tile as soon as the
// current row's words are in registers, so a load is in flight while the
// wavefront computes.  A row's codes, scales and token scale are stored
// after the wait for the next row's chunk: that wait (which covers stores
// too) then only ever finds the load and stores issued a whole row earlier.
// The arithmetic is the split kernel's.
constexpr int kStreamWaves = 4;    // wavefronts per workgroup
#ifndef FP4Q_NV_STREAM_GRID
#define FP4Q_NV_STREAM_GRID 2048
#endif
constexpr int kStreamGrid = FP4Q_NV_STREAM_GRID;  // workgroups: 8 per compute unit of 256

// Build-time knob: FP4Q_NV_STREAM_DEFER = 1 stores a row's outputs after the
// wait for the next row's chunk (0: right after its arithmetic, so that the
// wait also covers those stores).
#ifndef FP4Q_NV_STREAM_DEFER
#define FP4Q_NV_STREAM_DEFER 1
#endif

// One row's outputs, held from the end of its arithmetic until its stores:
// the lane's code words and its block-scale bytes (block n in byte n).
template <int NB>
struct RowOut {
  uint32_t c[NB][2], e;
  float s;
  bool pending;  // wave-uniform: false when the row stored its own outputs
};

template <int NB>
__device__ __forceinline__ void store_row(const RowOut<NB>& o, int64_t row, int nblk, int lane,
                                          uint2* __restrict__ codes,
                                          uint8_t* __restrict__ scales,
                                          float* __restrict__ tscale) {
  if (!o.pending) return;
  const int64_t base = row * nblk;  // nblk = 64 NB: every lane's blocks exist
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int j = lane + 64 * n;
    store_codes<false, false>(codes + base, j, make_uint2(o.c[n][0], o.c[n][1]));
    store_scale<false>(scales + base, j, (uint8_t)(o.e >> (8 * n)));
  }
  if (lane == 0) tscale[row] = o.s;
}

template <int FOS, int NB>
__global__ __launch_bounds__(64 * kStreamWaves) void nvfp4_quantize_stream(
    const uint4* __restrict__ x, int64_t row0, int64_t row_end, int nblk,
    const int64_t* __restrict__ offs, int64_t ngroups, uint2* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tscale, float neg_zero) {
  __shared__ uint4 tiles[kStreamWaves][128 * NB];
  __shared__ float2v recip[kStreamWaves][128];
  int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t lo = row0, hi = row_end;  // this launch's rows, within the group range
  if (offs != nullptr) {
    lo = max(lo, offs[0]);
    hi = min(hi, offs[ngroups]);
  }
  const int64_t stride = (int64_t)gridDim.x * kStreamWaves;
  int64_t row = lo + (int64_t)blockIdx.x * kStreamWaves + wave;  // wave-uniform
  if (!lt_i64(row, hi)) return;
  uint4* tile = tiles[wave];
  float2v* tab = recip[wave];
  constexpr int valid = 64 * NB;  // blocks of a row (nblk): whole chunks only

  uint32_t w[NB][8], bmax[NB], lmax;
  // the tile holds row `row`; its block maxima are taken, then the next
  // row's copy is started into the same tile
  const auto take_tile = [&](int64_t next) {
    read_tile<NB>(tile, lane, w);
    lmax = 0;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      bmax[n] = block_absmax_bits(w[n]);
      lmax = max(lmax, bmax[n]);
    }
    // lmax depends on every word read, so the reads have completed before
    // the copy below overwrites the tile
    asm volatile("" ::"v"(lmax) : "memory");
    if (lt_i64(next, hi)) issue_chunk_lds<NB>(x, next * nblk, valid, lane, tile);
  };
  issue_chunk_lds<NB>(x, row * nblk, valid, lane, tile);
  __builtin_amdgcn_s_waitcnt(0);
  int64_t next = row + stride;
  take_tile(next);
  for (;;) {
    // lane, redefined opaquely each row, so that addresses derived from it
    // are formed where they are used instead of held across the loop (which
    // would cost the occupancy of 8 wavefronts per SIMD)
    asm volatile("" : "+v"(lane));
    RowOut<NB> o;
    const RowScale rs = row_scale<FOS>(wave_max_u32(lmax));
    fill_recip(tab, rs, lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t cbase = row * nblk;
    o.s = rs.s;
    o.pending = rs.fast;
    o.e = 0u;
    if (__builtin_expect(rs.fast, 1)) {
#pragma unroll
      for (int n = 0; n < NB; ++n) {  // every lane's blocks exist (whole chunks)
        float xv[16];
        unpack16(w[n], xv);
        BlockOut bo;
        quantize_block_fast<FOS, false>(xv, bmax[n], rs, tab, neg_zero, bo);
        o.c[n][0] = bo.code0;
        o.c[n][1] = bo.code1;
        o.e |= bo.ebyte << (8 * n);
      }
    } else {
      // tiny rows take the out-of-line definition and store at once
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const int j = lane + 64 * n;
        tiny_row_block<FOS, false>((const uint16_t*)(x + 2 * (cbase + j)),
                                   __uint_as_float(bmax[n]), tab, rs.s, rs.inv_s,
                                   (uint8_t*)(codes + cbase + j), scales + cbase + j, nullptr);
      }
      if (lane == 0) tscale[row] = rs.s;
    }
    if (!FP4Q_NV_STREAM_DEFER || !lt_i64(next, hi))
      store_row<NB>(o, row, nblk, lane, codes, scales, tscale);
    if (!lt_i64(next, hi)) break;
    __builtin_amdgcn_s_waitcnt(0);  // the next row's chunk has landed
    if (FP4Q_NV_STREAM_DEFER) store_row<NB>(o, row, nblk, lane, codes, scales, tscale);
    row = next;
    next = row + stride;
    take_tile(next);
  }
}

// Any row length: one wavefront per row; a first pass for the amax, a
// second pass (served mostly by L2) for the blocks.
template <int FOS, bool DQ, bool NTC>
__global__ __launch_bounds__(64 * kLongWaves) void nvfp4_quantize_long_rows(
    const uint4* __restrict__ x, int64_t rows, int64_t row0, int64_t row_end, int nblk,
    const int64_t* __restrict__ offs, int64_t ngroups, uint2* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tscale, uint4* __restrict__ dq,
    float neg_zero, const uint4* __restrict__ gpart, int npart16,
    float* __restrict__ gscale_out) {
  __shared__ float2v recip[kLongWaves][128];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = row0 + (int64_t)blockIdx.x * kLongWaves + wave;
  if (row >= row_end || !row_range(row, rows, offs, ngroups)) return;
  const int64_t base = row * nblk;

  uint32_t row_amax;
  if (gpart != nullptr) {  // one scale for the whole tensor
    row_amax = tensor_amax(load_partials(gpart, npart16, lane));
  } else {
    uint32_t lmax = 0;
    for (int j = lane; j < nblk; j += 64) {
      uint32_t w[8];
      load_block(x, base + j, w);
      lmax = max(lmax, block_absmax_bits(w));
    }
    row_amax = wave_max_u32(lmax);
  }
  const RowScale rs = row_scale<FOS>(row_amax);
  if (lane == 0 && tscale != nullptr) tscale[row] = rs.s;
  if (gscale_out != nullptr && row0 == 0 && blockIdx.x == 0 && wave == 0 && lane == 0)
    *gscale_out = rs.s;
  fill_recip(recip[wave], rs, lane);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int j = lane; j < nblk; j += 64) {
    uint32_t w[8];
    float xv[16];
    load_block(x, base + j, w);
    unpack16(w, xv);
    quantize_block<FOS, DQ, NTC>(xv, block_absmax_f(xv), rs, recip[wave], neg_zero,
                                 x + 2 * base, j, codes + base, scales + base,
                                 DQ ? dq + 2 * base : nullptr);
  }
}

// K2: one lane per 8-element unit (half a block): 4 code bytes in and 16
// BF16 bytes out.  Wavefront gw covers part gw % wpr of row gw / wpr: up to
// 64 * FP4Q_DQ_UNITS consecutive units, lane l taking units l, l + 64, ...,
// so every load and store instruction is contiguous across the wave and the
// token scale is one uniform load.
// Units per lane: 4 measured fastest (moe_act 8192 x 7168, distinct codes
// per call: 24.1 us against 24.5 with 2, 25.1 with 8, 25.6 with 1).  Every
// unit's loads are issued before the first unit's arithmetic: loading each
// unit after the previous unit's store measured slower (25.3 against
// 23.4 us).
#ifndef FP4Q_DQ_UNITS
#define FP4Q_DQ_UNITS 4
#endif
// Units per lane of the guided kernel, mapped the same way: 4 measured
// fastest (moe_act, guided / to nearest: 28.3 / 25.4 us against 28.7 / 26.2
// with 2, 29.5 / 27.0 with 8, 34.0 / 29.6 with 1).
#ifndef FP4Q_GUIDED_UNITS
#define FP4Q_GUIDED_UNITS 4
#endif
#ifndef FP4Q_DQ_NT_STORES
#define FP4Q_DQ_NT_STORES 1
#endif
// Build-time knob: the cache-policy bits of K2's BF16 stores (see put).
#ifndef FP4Q_DQ_POLICY
#define FP4Q_DQ_POLICY FP4Q_NV_DQ_POLICY
#endif
// Build-time knob: FP4Q_DQ_NT_LOADS reads the codes (bit 0) and the block
// scales (bit 1) of the dequantizer with non-temporal loads.
#ifndef FP4Q_DQ_NT_LOADS
#define FP4Q_DQ_NT_LOADS 0
#endif
// Build-time knob: FP4Q_GUIDED_NT_LOADS = 1 reads the input (bit 0) and the
// guide codes (bit 1) of the guided quantizer with non-temporal loads.
#ifndef FP4Q_GUIDED_NT_LOADS
#define FP4Q_GUIDED_NT_LOADS 1
#endif
__global__ __launch_bounds__(256) void nvfp4_dequantize_rows(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tscale, int64_t row0, int64_t row_end, int h8, uint32_t wpr,
    uint4* __restrict__ out) {
  constexpr int NU = FP4Q_DQ_UNITS;
  const int lane = threadIdx.x & 63;
  const uint32_t gw = blockIdx.x * 4u + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t rr = gw / wpr;  // uniform
  const int64_t row = row0 + rr;
  if (row >= row_end) return;
  const int first = (int)(gw - rr * wpr) * 64 * NU;
  const int nv = h8 - first < 64 * NU ? h8 - first : 64 * NU;  // units of this wave
  const int64_t base = row * h8 + first;
  const uint32_t* cw_in = codes + base;
  const uint8_t* sc_in = scales + (base >> 1);
  uint4* o = out + base;
  const float s = tscale[row];
  uint32_t cw[NU];
  uint32_t eb[NU];
#pragma unroll
  for (int n = 0; n < NU; ++n) {
    const int j = min(lane + 64 * n, nv - 1);  // in bounds for every lane
    cw[n] = (FP4Q_DQ_NT_LOADS & 1) ? __builtin_nontemporal_load(&cw_in[j]) : cw_in[j];
    eb[n] = (FP4Q_DQ_NT_LOADS & 2) ? __builtin_nontemporal_load(&sc_in[j >> 1]) : sc_in[j >> 1];
  }
#pragma unroll
  for (int n = 0; n < NU; ++n) {
    const float e = e4m3_value<0>(eb[n]);
    uint32_t q[4];
    static_for<0, 4>([&](auto P) {
      constexpr int k = decltype(P)::value;
      const float2v g = e2m1x2_values<k>(cw[n]);
      const float ge0 = g.x * e, ge1 = g.y * e;  // exact
      q[k] = cvt_bf16x2(ge0 * s, ge1 * s);
    });
    if (lane + 64 * n < nv) {
      if (FP4Q_DQ_NT_STORES)
        put<FP4Q_DQ_POLICY < 0 ? 2 : FP4Q_DQ_POLICY>(o, lane + 64 * n,
                                                     make_uint4(q[0], q[1], q[2], q[3]));
      else
        o[lane + 64 * n] = make_uint4(q[0], q[1], q[2], q[3]);
    }
  }
}

// TRACE rollout-guided rounding ("TRACE FP4 RL -- Rollout-guided FP4
// rounding", learnaivisually.com): under the rollout's block and token
// scales, each element takes, of the two E2M1 codewords around
// v = |x| * fl(1 / fl(e s)), the one nearer the rollout's codeword.  With
// the same sign, or a zero guide, that is the upper neighbour exactly when
// the guide's magnitude code is at least the upper one; a guide of the
// other sign is nearer the lower neighbour.  One lane per 8-element unit,
// mapped like the dequant kernel.  RTN (no guide): each element takes its
// nearest codeword under the same scales instead -- the training side's own
// rounding that the page compares guided rounding with.
template <bool RTN, bool DQ>
__global__ __launch_bounds__(256) void nvfp4_guided_units(
    const uint4* __restrict__ x, const uint32_t* __restrict__ guide,
    const uint8_t* __restrict__ scales, const float* __restrict__ tscale, int64_t row0,
    int64_t row_end, int h8, uint32_t wpr, uint32_t* __restrict__ codes,
    uint4* __restrict__ dq) {
  constexpr int NU = FP4Q_GUIDED_UNITS;
  const int lane = threadIdx.x & 63;
  const uint32_t gw = blockIdx.x * 4u + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t rr = gw / wpr;  // uniform
  const int64_t row = row0 + rr;
  if (row >= row_end) return;
  const int first = (int)(gw - rr * wpr) * 64 * NU;
  const int nv = h8 - first < 64 * NU ? h8 - first : 64 * NU;
  const int64_t base = row * h8 + first;
  const float s = tscale[row];
  const uint4* xin = x + base;
  const uint32_t* gin = RTN ? nullptr : guide + base;
  const uint8_t* sin = scales + (base >> 1);
  // Unit by unit: each unit's loads are issued after the previous unit's
  // stores.  Requesting every unit's inputs before using the first (so that
  // the wave has them all in flight) measured slower: 31.3 against 28.7 us
  // guided, 27.6 against 26.3 us to nearest, on moe_act; so did copying the
  // wave's 4 KiB of input into LDS with global_load_lds and its guide words
  // and scale bytes into registers before one wait (35.1 against 28.0 us
  // guided, 28.0 against 25.4 us to nearest), and so did issuing unit
  // n + 1's loads before unit n's arithmetic, with one wait ahead of unit
  // n's stores (28.9 against 28.0 us guided; to nearest 25.1 either way).
  // The dequant output is a template argument, so that an instance issues
  // the same memory operations for every unit (28.3 -> 28.0 us guided, 25.4
  // -> 25.2 us to nearest, without the dequant).
#pragma unroll
  for (int n = 0; n < NU; ++n) {
    const int j = lane + 64 * n;
    if (j >= nv) continue;
    uint4 a;
    if (FP4Q_GUIDED_NT_LOADS & 1) {
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)&xin[j]);
      a = make_uint4(v.x, v.y, v.z, v.w);
    } else {
      a = xin[j];
    }
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    uint32_t gwd = 0u;
    if (!RTN)
      gwd = (FP4Q_GUIDED_NT_LOADS & 2) ? __builtin_nontemporal_load(&gin[j]) : gin[j];
    const float e = e4m3_value<0>(sin[j >> 1]);
    const float d = e * s;
    float r;  // fl(1 / fl(e s)), the IEEE quotient
    if (d >= 0x1p-126f && d <= 0x1p126f)
      r = recip_normal(d);
    else
      r = d != 0.0f ? 1.0f / d : 0.0f;
    // With lo <= hi adjacent (or equal) codes, the guide rule is a clamp:
    // the guide's magnitude code when the signs agree (else 0), clamped to
    // [lo, hi].
    uint32_t out = 0u;
    if (RTN && __builtin_expect(r < __builtin_inff(), 1)) {
      // nearest codes of v = |x| r (+inf, from an overflowing product,
      // saturates to code 7) with x's signs
      uint32_t word = any_word();  // bytes 0-3 all written below
      uint32_t sx = 0u;
      static_for<0, 4>([&](auto P) {
        constexpr int p = decltype(P)::value;
        word = cvt_e2m1x2<p>(word, fabsf(bf16_lo(w[p])) * r, fabsf(bf16_hi(w[p])) * r);
        sx |= (((w[p] >> 12) & 0x08u) | ((w[p] >> 24) & 0x80u)) << (8 * p);
      });
      out = word | sx;
    } else if (!RTN && __builtin_expect(r < __builtin_inff(), 1)) {
      // r finite (v may still overflow to +inf, whose lower neighbour is
      // code 7): the lower neighbours of all eight elements from the
      // truncating conversion, the upper ones one code up where v is off the
      // grid (not above 7), and the clamp on whole code words, nibble by
      // nibble: every nibble difference below stays in its nibble because
      // the minuend nibbles are 8 + (0..7) and the subtrahends 0..7.
      float v[8];
      uint32_t lw = 0u;
      static_for<0, 4>([&](auto P) {
        constexpr int p = decltype(P)::value;
        v[2 * p] = fabsf(bf16_lo(w[p])) * r;
        v[2 * p + 1] = fabsf(bf16_hi(w[p])) * r;
        lw |= cvt_e2m1x2_floor(v[2 * p], v[2 * p + 1]) << (8 * p);
      });
      uint32_t up = 0u, sx = 0u;
      static_for<0, 4>([&](auto P) {
        constexpr int p = decltype(P)::value;
        const float2v g = e2m1x2_values<p>(lw);
        up |= ((g.x != v[2 * p]) ? 0x01u : 0u) << (8 * p);
        up |= ((g.y != v[2 * p + 1]) ? 0x10u : 0u) << (8 * p);
        sx |= (((w[p] >> 12) & 0x08u) | ((w[p] >> 24) & 0x80u)) << (8 * p);  // x's signs
      });
      up &= ~(lw & (lw >> 1) & (lw >> 2));  // no step up from code 7
      const uint32_t hw = lw + up;
      // the guide's magnitude where its sign is x's, else 0
      const uint32_t agree = ~(gwd ^ sx) & 0x88888888u;
      const uint32_t m = gwd & (agree - (agree >> 3));
      const uint32_t ge = ((((m | 0x88888888u) - lw) >> 3) & 0x11111111u) * 15u;  // m >= lo
      const uint32_t mx = (m & ge) | (lw & ~ge);
      const uint32_t le = ((((hw | 0x88888888u) - mx) >> 3) & 0x11111111u) * 15u;  // mx <= hi
      out = ((mx & le) | (hw & ~le)) | sx;
    } else {
      // r = +inf (a subnormal decode step): v may be +inf or NaN, which the
      // threshold counts follow as the definition does
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xi = (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
        const float vi = fabsf(xi) * r;
        const uint32_t sx = __float_as_uint(xi) >> 31;
        uint32_t q;
        if (RTN) {
          float g;
          q = e2m1_code_sw(vi, g);  // NaN (0 * inf) gives 0, +inf 7
        } else {
          const uint32_t lo = (vi >= 0.5f) + (vi >= 1.0f) + (vi >= 1.5f) + (vi >= 2.0f) +
                              (vi >= 3.0f) + (vi >= 4.0f) + (vi >= 6.0f);
          const uint32_t hi = (lo < 7u && e2m1_value(lo) < vi) ? lo + 1u : lo;
          const uint32_t gn = (gwd >> (4 * i)) & 15u;
          const uint32_t m = (gn >> 3) == sx ? (gn & 7u) : 0u;
          q = min(max(m, lo), hi);
        }
        out |= ((sx << 3) | q) << (4 * i);
      }
    }
    store_words<RTN>(codes + base, j, out);
    if (DQ) {
      uint32_t o[4];
      static_for<0, 4>([&](auto P) {
        constexpr int k = decltype(P)::value;
        const float2v g = e2m1x2_values<k>(out);
        const float ge0 = g.x * e, ge1 = g.y * e;  // exact
        o[k] = cvt_bf16x2(ge0 * s, ge1 * s);
      });
      store_dq(dq + base, j, make_uint4(o[0], o[1], o[2], o[3]));
    }
  }
}

// One FP32 scale for the whole tensor: every workgroup of the max pass
// writes the max of its share -- the 16-bit pattern of a BF16 magnitude,
// which orders like its value -- to its own slot of a partial array in the
// caller's workspace; every wave of the quantize pass then reduces those
// partials itself (one 16-byte load a lane, tensor_amax), derives
// s = fl(amax / C) and quantizes its blocks under it, and the first wave
// writes s to the caller's tensor scale.  (One atomic max per workgroup on a
// single word instead serializes the atomics; a separate one-workgroup
// reduction between the passes costs a dependent launch of about 4.6 us.)

// Build-time knobs of the tensor max pass: workgroups (FP4Q_GAMAX_GRID),
// 16-byte loads in flight per lane (FP4Q_GAMAX_DEPTH), non-temporal loads
// (FP4Q_GAMAX_NT).
#ifndef FP4Q_GAMAX_GRID
#define FP4Q_GAMAX_GRID 512
#endif
static_assert(FP4Q_GAMAX_GRID >= 1 && 2 * ((FP4Q_GAMAX_GRID + 7) / 8 * 8) <=
                                          FP4Q_GLOBAL_WORKSPACE_BYTES &&
                  (FP4Q_GAMAX_GRID + 7) / 8 <= 64,
              "the padded partial maxima must fit the workspace and one 16-byte load a lane");
#ifndef FP4Q_GAMAX_DEPTH
#define FP4Q_GAMAX_DEPTH 4
#endif
#ifndef FP4Q_GAMAX_NT
#define FP4Q_GAMAX_NT 0
#endif
// Build-time knob: FP4Q_GAMAX_CHUNKED = 1 gives each wavefront of the max
// pass whole chunks of D contiguous KiB (the grid striding over chunks, as
// K0 reads); 0 strides every lane over single 16-byte units, so that a
// wavefront's D loads in flight lie a whole grid apart.  Chunks: max pass
// 18.8 against 19.7 us on moe_act (2 KiB chunks 21.6 us, 8 KiB 19.1 us;
// 512 or 1024 threads per workgroup 19.5 and 20.7 us).
#ifndef FP4Q_GAMAX_CHUNKED
#define FP4Q_GAMAX_CHUNKED 1
#endif
// Build-time knob: threads per workgroup of the tensor max pass (256, 512
// or 1024; one partial maximum per workgroup either way).  More waves in
// flight made the whole call slower on moe_act: 61.5 us with 1024 threads,
// 62.3 with 512, against 60.5 with 256.  (Loads with the sc0 or sc1 bits,
// through buffer instructions, made no difference: 60.4-60.5 us.)
#ifndef FP4Q_GAMAX_THREADS
#define FP4Q_GAMAX_THREADS 256
#endif
static_assert(FP4Q_GAMAX_THREADS == 256 || FP4Q_GAMAX_THREADS == 512 ||
                  FP4Q_GAMAX_THREADS == 1024, "whole wavefronts, at most 1024 threads");

__global__ __launch_bounds__(FP4Q_GAMAX_THREADS) void global_amax_pass(
    const uint4* __restrict__ x, int64_t n16, uint16_t* __restrict__ partial) {
  constexpr int T = FP4Q_GAMAX_THREADS;
  __shared__ uint32_t wmax[T / 64];
  uint32_t m = 0u;
  constexpr int D = FP4Q_GAMAX_DEPTH;
  if (FP4Q_GAMAX_CHUNKED) {
    // each wavefront reads whole chunks of 64 D consecutive units (D
    // contiguous KiB), chunk k going to wavefront k mod (all wavefronts), so
    // a step of the grid covers one contiguous stretch of the tensor
    const int lane = threadIdx.x & 63;
    constexpr int64_t CH = 64 * D;
    const int64_t nwaves = (int64_t)gridDim.x * (T / 64);
    int64_t base =
        ((int64_t)blockIdx.x * (T / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * CH;
    for (; base + CH <= n16; base += nwaves * CH) {  // whole chunks
      uint4 a[D];
#pragma unroll
      for (int u = 0; u < D; ++u) a[u] = x[base + 64 * u + lane];
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const uint32_t w[4] = {a[u].x & 0x7FFF7FFFu, a[u].y & 0x7FFF7FFFu, a[u].z & 0x7FFF7FFFu,
                               a[u].w & 0x7FFF7FFFu};
#pragma unroll
        for (int k = 0; k < 4; ++k) m = max(m, max(w[k] << 16, w[k] & 0xFFFF0000u));
      }
    }
    if (base < n16) {  // the one partial chunk at the end of the tensor
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int64_t idx = base + 64 * u + lane;
        if (idx < n16) {
          const uint4 a = x[idx];
          const uint32_t w[4] = {a.x & 0x7FFF7FFFu, a.y & 0x7FFF7FFFu, a.z & 0x7FFF7FFFu,
                                 a.w & 0x7FFF7FFFu};
#pragma unroll
          for (int k = 0; k < 4; ++k) m = max(m, max(w[k] << 16, w[k] & 0xFFFF0000u));
        }
      }
    }
  }
  const int64_t stride = (int64_t)gridDim.x * T;
  int64_t i = FP4Q_GAMAX_CHUNKED ? n16 : (int64_t)blockIdx.x * T + threadIdx.x;
  for (; i + (D - 1) * stride < n16; i += D * stride) {  // D loads in flight per lane
    uint4 a[D];
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (FP4Q_GAMAX_NT) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)&x[i + u * stride]);
        a[u] = make_uint4(v.x, v.y, v.z, v.w);
      } else {
        a[u] = x[i + u * stride];
      }
    }
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const uint32_t w[4] = {a[u].x & 0x7FFF7FFFu, a[u].y & 0x7FFF7FFFu, a[u].z & 0x7FFF7FFFu,
                             a[u].w & 0x7FFF7FFFu};
#pragma unroll
      for (int k = 0; k < 4; ++k) m = max(m, max(w[k] << 16, w[k] & 0xFFFF0000u));
    }
  }
  for (; i < n16; i += stride) {
    const uint4 a = x[i];
    const uint32_t w[4] = {a.x & 0x7FFF7FFFu, a.y & 0x7FFF7FFFu, a.z & 0x7FFF7FFFu,
                           a.w & 0x7FFF7FFFu};
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max(w[k] << 16, w[k] & 0xFFFF0000u));
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = 0u;
#pragma unroll
    for (int k = 0; k < T / 64; ++k) b = max(b, wmax[k]);
    partial[blockIdx.x] = (uint16_t)(b >> 16);
  }
  // zeros (the identity of the max) up to a whole 16-byte unit
  const unsigned padded = (gridDim.x + 7u) & ~7u;
  if (blockIdx.x == 0 && gridDim.x + threadIdx.x < padded) partial[gridDim.x + threadIdx.x] = 0;
}

// Rows (or row groups) per launch when one takes `items` work-items: as many
// as the launch limit allows, and at least one, so that the row loop always
// advances.  At the largest accepted hidden (2^30) one row is at most 2^26
// work-items, far below the dispatch's 32-bit count, so the floor only
// matters for builds with a tiny limit (a test build splits at 4096).
__host__ inline int64_t rows_per_launch(int64_t items) {
  const int64_t n = FP4Q_MAX_LAUNCH_ITEMS / items;
  return n > 0 ? n : 1;
}

// NTC: see store_codes (the global-scale call's quantize pass).
template <int FOS, bool DQ, bool NTC>
hipError_t launch_quantize(const NvQuantArgs& a, hipStream_t st) {
  const int nblk = (int)(a.hidden / 16);
  const uint4* x = (const uint4*)a.x;
  uint2* codes = (uint2*)a.codes;
  uint4* dq = (uint4*)a.dequant;
  const float neg_zero = -0.0f;
  constexpr int NB = FP4Q_NV_NB;             // blocks per lane
  const int W = (nblk + 64 * NB - 1) / (64 * NB);  // waves per row
  if (FP4Q_NV_STREAM && !DQ && nblk == 64 * NB && a.global_partials == nullptr &&
      !FP4Q_STANDIN) {
    // a fixed grid (fewer workgroups if there are fewer rows, and within the
    // launch limit) walks all rows
    int64_t grid = (a.rows + kStreamWaves - 1) / kStreamWaves;
    if (grid > kStreamGrid) grid = kStreamGrid;
    const int64_t max_grid = rows_per_launch(64 * kStreamWaves);
    if (grid > max_grid) grid = max_grid;
    hipLaunchKernelGGL((nvfp4_quantize_stream<FOS, NB>), dim3((unsigned)grid),
                       dim3(64 * kStreamWaves), 0, st, x, (int64_t)0, a.rows, nblk, a.offsets,
                       a.num_groups, codes, a.block_scales, a.token_scales, neg_zero);
  } else if (W <= kMaxWgWaves) {
    const int R = W >= FP4Q_NV_WG_WAVES ? 1 : FP4Q_NV_WG_WAVES / W;  // rows per workgroup
    const int64_t max_rows = rows_per_launch(64 * W * R) * R;         // rows per launch
    // per wave: its reciprocal table, then its input tile (NB x 2 KiB) or,
    // without it, 2 KiB of dequant staging
    const size_t wave_lds = FP4Q_NV_LDS_LOAD ? (size_t)NB * 128
                            : (FP4Q_NV_LDS_DQ && DQ) ? 128 : 0;
    const size_t lds = (size_t)W * R * (128 * sizeof(float2v) + wave_lds * sizeof(uint4));
    for (int64_t row0 = 0; row0 < a.rows; row0 += max_rows) {
      const int64_t row_end = a.rows - row0 < max_rows ? a.rows : row0 + max_rows;
      const dim3 grid((unsigned)((row_end - row0 + R - 1) / R)), block(64 * W * R);
      hipLaunchKernelGGL((nvfp4_quantize_split<FOS, DQ, NB, NTC>), grid, block, lds, st, x,
                         a.rows, row0, row_end, nblk, W, (65536 + W - 1) / W, R, a.offsets,
                         a.num_groups, codes,
                         a.block_scales, a.token_scales, dq, neg_zero, a.global_partials,
                         a.num_partials, a.tensor_scale_out);
    }
  } else {
    const int64_t max_rows = rows_per_launch(64 * kLongWaves) * kLongWaves;
    for (int64_t row0 = 0; row0 < a.rows; row0 += max_rows) {
      const int64_t row_end = a.rows - row0 < max_rows ? a.rows : row0 + max_rows;
      const dim3 grid((unsigned)((row_end - row0 + kLongWaves - 1) / kLongWaves)),
          block(64 * kLongWaves);
      hipLaunchKernelGGL((nvfp4_quantize_long_rows<FOS, DQ, NTC>), grid, block, 0, st, x,
                         a.rows, row0, row_end, nblk, a.offsets, a.num_groups, codes,
                         a.block_scales, a.token_scales, dq, neg_zero, a.global_partials,
                         a.num_partials, a.tensor_scale_out);
    }
  }
  return hipGetLastError();
}

}  // namespace

namespace {
// Workgroups of the tensor-max pass for rows x hidden.
int64_t global_amax_grid(int64_t rows, int64_t hidden) {
  const int64_t n16 = rows * hidden / 8;  // 16-byte units
  const int64_t grid = (n16 + FP4Q_GAMAX_THREADS - 1) / FP4Q_GAMAX_THREADS;
  return grid < FP4Q_GAMAX_GRID ? grid : FP4Q_GAMAX_GRID;
}
}  // namespace

int64_t global_workspace_bytes(int64_t rows, int64_t hidden) {
  return 2 * ((global_amax_grid(rows, hidden) + 7) / 8 * 8);
}

hipError_t nvfp4_quantize_global_launch(const NvQuantArgs& args, float* tensor_scale,
                                        void* workspace, hipStream_t st) {
  NvQuantArgs a = args;
  const int64_t n16 = a.rows * a.hidden / 8;  // 16-byte units, >= 2
  const int64_t grid = global_amax_grid(a.rows, a.hidden);
  // grid 16-bit maxima, zero-padded to whole 16-byte units
  uint16_t* partial = static_cast<uint16_t*>(workspace);
  hipLaunchKernelGGL(global_amax_pass, dim3((unsigned)grid), dim3(FP4Q_GAMAX_THREADS), 0, st,
                     (const uint4*)a.x, n16, partial);
  a.global_partials = reinterpret_cast<const uint4*>(partial);
  a.num_partials = (int)((grid + 7) / 8);
  a.tensor_scale_out = tensor_scale;
  a.token_scales = nullptr;
  return nvfp4_quantize_launch(a, st);
}

namespace {
template <bool NTC>
hipError_t launch_mode(const NvQuantArgs& a, hipStream_t st) {
  if (a.four_over_six == 2)
    return a.dequant ? launch_quantize<2, true, NTC>(a, st) : launch_quantize<2, false, NTC>(a, st);
  if (a.four_over_six == 1)
    return a.dequant ? launch_quantize<1, true, NTC>(a, st) : launch_quantize<1, false, NTC>(a, st);
  return a.dequant ? launch_quantize<0, true, NTC>(a, st) : launch_quantize<0, false, NTC>(a, st);
}
}  // namespace

hipError_t nvfp4_quantize_launch(const NvQuantArgs& a, hipStream_t st) {
  return a.global_partials != nullptr ? launch_mode<true>(a, st) : launch_mode<false>(a, st);
}

hipError_t nvfp4_dequantize_launch(const uint8_t* codes, const uint8_t* scales,
                                   const float* tscale, int64_t rows, int64_t hidden, void* out,
                                   hipStream_t st) {
  const int h8 = (int)(hidden / 8);
  const int64_t per_wave = 64 * FP4Q_DQ_UNITS;
  const uint32_t wpr = (uint32_t)((h8 + per_wave - 1) / per_wave);  // waves per row
  const int64_t max_rows = rows_per_launch(64 * (int64_t)wpr);
  for (int64_t row0 = 0; row0 < rows; row0 += max_rows) {
    const int64_t n = rows - row0 < max_rows ? rows - row0 : max_rows;
    const dim3 grid((unsigned)((n * wpr + 3) / 4)), block(256);
    hipLaunchKernelGGL(nvfp4_dequantize_rows, grid, block, 0, st, (const uint32_t*)codes, scales,
                       tscale, row0, row0 + n, h8, wpr, (uint4*)out);
  }
  return hipGetLastError();
}

hipError_t nvfp4_guided_launch(const void* x, const uint8_t* guide, const uint8_t* scales,
                              const float* tscale, int64_t rows, int64_t hidden, uint8_t* codes,
                              void* dequant, hipStream_t st) {
  const int h8 = (int)(hidden / 8);
  const int64_t per_wave = 64 * FP4Q_GUIDED_UNITS;
  const uint32_t wpr = (uint32_t)((h8 + per_wave - 1) / per_wave);  // waves per row
  const int64_t max_rows = rows_per_launch(64 * (int64_t)wpr);
  for (int64_t row0 = 0; row0 < rows; row0 += max_rows) {
    const int64_t n = rows - row0 < max_rows ? rows - row0 : max_rows;
    const dim3 grid((unsigned)((n * wpr + 3) / 4)), block(256);
    // the guide's presence and the dequant output are template arguments, so
    // that each instance issues a fixed run of memory operations per unit
    auto launch = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, grid, block, 0, st, (const uint4*)x, (const uint32_t*)guide,
                         scales, tscale, row0, row0 + n, h8, wpr, (uint32_t*)codes,
                         (uint4*)dequant);
    };
    if (guide != nullptr)
      dequant != nullptr ? launch(nvfp4_guided_units<false, true>)
                         : launch(nvfp4_guided_units<false, false>);
    else
      dequant != nullptr ? launch(nvfp4_guided_units<true, true>)
                         : launch(nvfp4_guided_units<true, false>);
  }
  return hipGetLastError();
}

}  // namespace fp4q
