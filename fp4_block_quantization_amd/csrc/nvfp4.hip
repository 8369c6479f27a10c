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
// Mapping (K1): one wavefront per row, one lane per 16-element block.  The
// whole row stays in VGPRs between the amax reduction and the block pass
// (CH chunks of 64 blocks = 1024 elements), so HBM sees every input byte
// once; rows longer than 8 chunks take a second, L2-served read.
//
// Arithmetic per block and candidate k (all IEEE binary32, no contraction):
//   t = b / fl(k s)   (IEEE division)      e = E4M3(min(t, 448))
//   r = 1 / fl(e s)   (IEEE division, looked up in a per-row LDS table of
//                      all 127 E4M3 values: the same bits, computed once
//                      per row instead of once per block)
//   v = x r, q = E2M1(v) with sign, c = fl(fl(+-g e) s), err += (x - c)^2
// The E2M1/E4M3/BF16 conversions are the gfx950 conversion instructions.
#include "fp4q_device.h"
#include "fp4q_launch.h"

namespace fp4q {

namespace {

constexpr int kWaves = 4;  // wavefronts (rows) per workgroup

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Wave-wide max of a non-negative value held as its bit pattern.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}

// Max |x| over one block of 16 BF16 values, as a BF16 magnitude pattern.
__device__ __forceinline__ uint32_t block_absmax_bits(const uint32_t (&w)[8]) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = max(m, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
  return m;
}

// Per-row reciprocal table: tab[byte] = 1 / fl(e(byte) * s) for every
// E4M3 byte 0..127 (0 where the decode step is 0).  Each lane fills two
// entries; only this wave reads them.
__device__ __forceinline__ void fill_recip_table(float* tab, float s, int lane) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t byte = (uint32_t)lane + 64u * k;
    const float d = e4m3_decode(byte) * s;
    tab[byte] = (d != 0.0f) ? 1.0f / d : 0.0f;
  }
  __builtin_amdgcn_wave_barrier();
}

struct Candidate {
  uint32_t code[2];  // 16 nibbles, element 2i in the low nibble of byte i
  float err;
  float c[16];  // signed FP32 candidate values
};

// One candidate: decode step with value e and reciprocal r under token
// scale s.
__device__ __forceinline__ void candidate(const float (&x)[16], float e, float r, float s,
                                          Candidate& out) {
  if (__builtin_expect(r <= 3.4028235e38f, 1)) {
    uint32_t code[2] = {0u, 0u};
    float err = 0.0f;
    static_for<0, 8>([&](auto P) {
      constexpr int p = decltype(P)::value;
      const float v0 = x[2 * p] * r, v1 = x[2 * p + 1] * r;
      code[p >> 2] = cvt_e2m1x2<p & 3>(code[p >> 2], v0, v1);
      const float2v g = e2m1x2_values<p & 3>(code[p >> 2]);
      const float ge0 = g.x * e, ge1 = g.y * e;  // exact: <= 6 significant bits
      const float c0 = ge0 * s, c1 = ge1 * s;
      const float d0 = x[2 * p] - c0, d1 = x[2 * p + 1] - c1;
      const float q0 = d0 * d0, q1 = d1 * d1;
      err = err + q0;
      err = err + q1;
      out.c[2 * p] = c0;
      out.c[2 * p + 1] = c1;
    });
    out.code[0] = code[0];
    out.code[1] = code[1];
    out.err = err;
  } else {
    // r = +inf (a decode step below 2^-128): x * r is +-inf for nonzero x
    // and NaN for zeros, which the portable rounding maps to code 0.
    uint32_t code[2] = {0u, 0u};
    float err = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float g;
      const uint32_t q = e2m1_code_sw(fabsf(x[i]) * r, g);
      const uint32_t neg = __float_as_uint(x[i]) >> 31;
      const float ge = g * e;
      float c = ge * s;
      c = neg ? -c : c;
      const float d = x[i] - c;
      const float sq = d * d;
      err = err + sq;
      code[i >> 3] |= (q | (neg << 3)) << (4 * (i & 7));
      out.c[i] = c;
    }
    out.code[0] = code[0];
    out.code[1] = code[1];
    out.err = err;
  }
}

template <bool FOS, bool DQ>
__device__ __forceinline__ void quantize_block(const uint32_t (&w)[8], uint32_t bbits, float s,
                                               float ks6, float ks4, const float* tab,
                                               int64_t blk, uint2* __restrict__ codes,
                                               uint8_t* __restrict__ scales,
                                               uint4* __restrict__ dq) {
  float x[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[2 * k] = bf16_lo(w[k]);
    x[2 * k + 1] = bf16_hi(w[k]);
  }
  const float b = __uint_as_float(bbits << 16);
  // both candidate block scales in one conversion (byte 0: map to 6,
  // byte 1: map to 4); E4M3 saturates at 448
  const float t6 = fminf(b / ks6, 448.0f);
  const float t4 = FOS ? fminf(b / ks4, 448.0f) : 0.0f;
  const uint32_t eb = cvt_e4m3x2(t6, t4);

  Candidate c6;
  candidate(x, e4m3_value<0>(eb), tab[eb & 0xFFu], s, c6);
  bool four = false;
  Candidate c4;
  if (FOS) {
    candidate(x, e4m3_value<1>(eb), tab[eb >> 8], s, c4);
    four = c4.err < c6.err;  // strictly lower error: 4 wins; ties keep 6
  }
  codes[blk] = four ? make_uint2(c4.code[0], c4.code[1]) : make_uint2(c6.code[0], c6.code[1]);
  scales[blk] = (uint8_t)(four ? (eb >> 8) : (eb & 0xFFu));
  if (DQ) {
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      o[k] = cvt_bf16x2(four ? c4.c[2 * k] : c6.c[2 * k], four ? c4.c[2 * k + 1] : c6.c[2 * k + 1]);
    dq[2 * blk] = make_uint4(o[0], o[1], o[2], o[3]);
    dq[2 * blk + 1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
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

// Token scale and the per-row constants: ks = fl(k s); a zero row uses 1
// so that b / ks = 0 / 1 gives a zero block scale.
template <bool FOS>
__device__ __forceinline__ float token_scale(uint32_t amax_bits, float& ks6, float& ks4) {
  const float amax = __uint_as_float(amax_bits << 16);
  const float s = amax / (FOS ? 1536.0f : 2688.0f);
  ks6 = (s != 0.0f) ? 6.0f * s : 1.0f;
  ks4 = (s != 0.0f) ? 4.0f * s : 1.0f;
  return s;
}

// Register-resident row: nblk <= 64 * CH.
template <int CH, bool FOS, bool DQ>
__global__ __launch_bounds__(64 * kWaves) void nvfp4_quantize_rows(
    const uint4* __restrict__ x, int64_t rows, int nblk, const int64_t* __restrict__ offs,
    int64_t ngroups, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tscale, uint4* __restrict__ dq) {
  __shared__ float recip[kWaves][128];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  if (!row_range(row, rows, offs, ngroups)) return;

  const int64_t base = row * nblk;  // first block of the row
  uint32_t w[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j = c * 64 + lane;
    uint4 a = make_uint4(0, 0, 0, 0), bq = a;
    if (j < nblk) {
      a = x[2 * (base + j)];
      bq = x[2 * (base + j) + 1];
    }
    w[c][0] = a.x; w[c][1] = a.y; w[c][2] = a.z; w[c][3] = a.w;
    w[c][4] = bq.x; w[c][5] = bq.y; w[c][6] = bq.z; w[c][7] = bq.w;
  }

  uint32_t bmax[CH];
  uint32_t lmax = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    bmax[c] = block_absmax_bits(w[c]);
    lmax = max(lmax, bmax[c]);
  }
  float ks6, ks4;
  const float s = token_scale<FOS>(wave_max_u32(lmax), ks6, ks4);
  if (lane == 0) tscale[row] = s;
  fill_recip_table(recip[wave], s, lane);

#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j = c * 64 + lane;
    if (j < nblk)
      quantize_block<FOS, DQ>(w[c], bmax[c], s, ks6, ks4, recip[wave], base + j, codes, scales,
                              dq);
  }
}

// Any row length: a first pass for the amax, a second pass (served mostly
// by L2) for the blocks.
template <bool FOS, bool DQ>
__global__ __launch_bounds__(64 * kWaves) void nvfp4_quantize_long_rows(
    const uint4* __restrict__ x, int64_t rows, int nblk, const int64_t* __restrict__ offs,
    int64_t ngroups, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tscale, uint4* __restrict__ dq) {
  __shared__ float recip[kWaves][128];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  if (!row_range(row, rows, offs, ngroups)) return;
  const int64_t base = row * nblk;

  uint32_t lmax = 0;
  for (int j = lane; j < nblk; j += 64) {
    const uint4 a = x[2 * (base + j)], bq = x[2 * (base + j) + 1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
    lmax = max(lmax, block_absmax_bits(w));
  }
  float ks6, ks4;
  const float s = token_scale<FOS>(wave_max_u32(lmax), ks6, ks4);
  if (lane == 0) tscale[row] = s;
  fill_recip_table(recip[wave], s, lane);
  for (int j = lane; j < nblk; j += 64) {
    const uint4 a = x[2 * (base + j)], bq = x[2 * (base + j) + 1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
    quantize_block<FOS, DQ>(w, block_absmax_bits(w), s, ks6, ks4, recip[wave], base + j, codes,
                            scales, dq);
  }
}

// K2: one lane per 16-element block.
__global__ __launch_bounds__(256) void nvfp4_dequantize_blocks(
    const uint2* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tscale, int64_t nblocks, int nblk, uint4* __restrict__ out) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  const float s = tscale[blk / nblk];
  const float e = e4m3_decode(scales[blk]);
  const uint2 cw = codes[blk];
  uint32_t o[8];
  static_for<0, 8>([&](auto P) {
    constexpr int k = decltype(P)::value;
    const float2v g = e2m1x2_values<k & 3>(k < 4 ? cw.x : cw.y);
    const float ge0 = g.x * e, ge1 = g.y * e;
    o[k] = cvt_bf16x2(ge0 * s, ge1 * s);
  });
  out[2 * blk] = make_uint4(o[0], o[1], o[2], o[3]);
  out[2 * blk + 1] = make_uint4(o[4], o[5], o[6], o[7]);
}

template <bool FOS, bool DQ>
hipError_t launch_quantize(const NvQuantArgs& a, hipStream_t st) {
  const int nblk = (int)(a.hidden / 16);
  const dim3 grid((unsigned)((a.rows + kWaves - 1) / kWaves)), block(64 * kWaves);
  const uint4* x = (const uint4*)a.x;
  uint2* codes = (uint2*)a.codes;
  uint4* dq = (uint4*)a.dequant;
  const int ch = (nblk + 63) / 64;
#define FP4Q_ROWS(CHN)                                                                       \
  case CHN:                                                                                   \
    hipLaunchKernelGGL((nvfp4_quantize_rows<CHN, FOS, DQ>), grid, block, 0, st, x, a.rows,  \
                       nblk, a.offsets, a.num_groups, codes, a.block_scales, a.token_scales, \
                       dq);                                                                   \
    break;
  switch (ch) {
    FP4Q_ROWS(1)
    FP4Q_ROWS(2)
    FP4Q_ROWS(3)
    FP4Q_ROWS(4)
    FP4Q_ROWS(5)
    FP4Q_ROWS(6)
    FP4Q_ROWS(7)
    FP4Q_ROWS(8)
    default:
      hipLaunchKernelGGL((nvfp4_quantize_long_rows<FOS, DQ>), grid, block, 0, st, x, a.rows,
                         nblk, a.offsets, a.num_groups, codes, a.block_scales, a.token_scales,
                         dq);
  }
#undef FP4Q_ROWS
  return hipGetLastError();
}

}  // namespace

hipError_t nvfp4_quantize_launch(const NvQuantArgs& a, hipStream_t st) {
  if (a.four_over_six)
    return a.dequant ? launch_quantize<true, true>(a, st) : launch_quantize<true, false>(a, st);
  return a.dequant ? launch_quantize<false, true>(a, st) : launch_quantize<false, false>(a, st);
}

hipError_t nvfp4_dequantize_launch(const uint8_t* codes, const uint8_t* scales,
                                   const float* tscale, int64_t rows, int64_t hidden, void* out,
                                   hipStream_t st) {
  const int nblk = (int)(hidden / 16);
  const int64_t nblocks = rows * nblk;
  const dim3 grid((unsigned)((nblocks + 255) / 256)), block(256);
  hipLaunchKernelGGL(nvfp4_dequantize_blocks, grid, block, 0, st, (const uint2*)codes, scales,
                     tscale, nblocks, nblk, (uint4*)out);
  return hipGetLastError();
}

}  // namespace fp4q
