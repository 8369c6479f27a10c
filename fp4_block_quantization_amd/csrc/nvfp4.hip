// nvfp4.hip -- per-token NVFP4 quantization with Four-Over-Six (K1) and
// NVFP4 dequantization (K2) for gfx950.
//
// Method: "NVFP4-RL" (jianyuh.github.io), sections 2-4, and "humans&
// Open-Sources the First Stable 4-Bit RL Training Recipe at 1.73x Speedup"
// (alphasignal.ai), sections 1-3.  Each token row gets its own FP32 scale
// from its amax over the hidden dimension; the E4M3 scale of every
// 16-element block is computed in the same kernel; per block the max is
// mapped to 6 or to 4, whichever gives the lower squared error (ties keep
// 6); the BF16 dequantized values of the chosen encoding are written in the
// same pass for the dequantized backward.
//
// Mapping (K1): one wavefront per row, one lane per 16-element block.  The
// whole row stays in VGPRs between the amax reduction and the block pass
// (CH chunks of 64 blocks = 1024 elements), so HBM sees every input byte
// once; rows longer than 8 chunks take a second, L2-served read.
#include "fp4q_device.h"
#include "fp4q_launch.h"

namespace fp4q {

namespace {

constexpr int kWaves = 4;  // wavefronts (rows) per workgroup

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

struct Candidate {
  uint32_t code[2];  // 16 nibbles
  uint32_t ebyte;
  float err;
  uint32_t deq[8];  // 16 BF16 values
};

// One candidate of one block: the block max b is mapped to k via
// ks = fl(k * s) (NVFP4-RL blog, section 4).
template <bool DQ>
__device__ __forceinline__ void candidate(const float (&xv)[16], float b, float ks, float s,
                                          Candidate& c) {
  float e;
  c.ebyte = e4m3_encode(b / ks, e);
  const float d = e * s;
  const float r = (d != 0.0f) ? 1.0f / d : 0.0f;  // a zero step gives code 0 everywhere
  float err = 0.0f;
  uint32_t code[2] = {0u, 0u};
  float cv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = fabsf(xv[i]);
    float g;
    const uint32_t q = e2m1_code_sw(a * r, g);
    const float ge = g * e;  // exact: at most 6 significant bits
    float cand = ge * s;
    const uint32_t neg = __float_as_uint(xv[i]) >> 31;
    cand = neg ? -cand : cand;
    const float delta = xv[i] - cand;
    const float sq = delta * delta;
    err = err + sq;
    code[i >> 3] |= (q | (neg << 3)) << (4 * (i & 7));
    cv[i] = cand;
  }
  c.code[0] = code[0];
  c.code[1] = code[1];
  c.err = err;
  if (DQ) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c.deq[k] = pack_bf16x2(cv[2 * k], cv[2 * k + 1]);
  }
}

template <bool FOS, bool DQ>
__device__ __forceinline__ void quantize_block(const uint32_t (&w)[8], uint32_t bbits, float s,
                                               float s6, float s4, int64_t blk,
                                               uint2* __restrict__ codes,
                                               uint8_t* __restrict__ scales,
                                               uint4* __restrict__ dq) {
  float xv[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    xv[2 * k] = bf16_lo(w[k]);
    xv[2 * k + 1] = bf16_hi(w[k]);
  }
  const float b = __uint_as_float(bbits << 16);
  Candidate c6;
  candidate<DQ>(xv, b, s6, s, c6);
  if (FOS) {
    Candidate c4;
    candidate<DQ>(xv, b, s4, s, c4);
    if (c4.err < c6.err) c6 = c4;  // strictly lower error: 4 wins; ties keep 6
  }
  codes[blk] = make_uint2(c6.code[0], c6.code[1]);
  scales[blk] = (uint8_t)c6.ebyte;
  if (DQ) {
    dq[2 * blk] = make_uint4(c6.deq[0], c6.deq[1], c6.deq[2], c6.deq[3]);
    dq[2 * blk + 1] = make_uint4(c6.deq[4], c6.deq[5], c6.deq[6], c6.deq[7]);
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

// Register-resident row: nblk <= 64 * CH.
template <int CH, bool FOS, bool DQ>
__global__ __launch_bounds__(64 * kWaves) void nvfp4_quantize_rows(
    const uint4* __restrict__ x, int64_t rows, int nblk, const int64_t* __restrict__ offs,
    int64_t ngroups, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tscale, uint4* __restrict__ dq) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
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
  const float amax = __uint_as_float(wave_max_u32(lmax) << 16);
  const float s = amax / (FOS ? 1536.0f : 2688.0f);
  if (lane == 0) tscale[row] = s;
  const float s6 = 6.0f * s, s4 = 4.0f * s;

#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j = c * 64 + lane;
    if (j < nblk) quantize_block<FOS, DQ>(w[c], bmax[c], s, s6, s4, base + j, codes, scales, dq);
  }
}

// Any row length: a first pass for the amax, a second pass (served mostly
// by L2) for the blocks.
template <bool FOS, bool DQ>
__global__ __launch_bounds__(64 * kWaves) void nvfp4_quantize_long_rows(
    const uint4* __restrict__ x, int64_t rows, int nblk, const int64_t* __restrict__ offs,
    int64_t ngroups, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tscale, uint4* __restrict__ dq) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (!row_range(row, rows, offs, ngroups)) return;
  const int64_t base = row * nblk;

  uint32_t lmax = 0;
  for (int j = lane; j < nblk; j += 64) {
    const uint4 a = x[2 * (base + j)], bq = x[2 * (base + j) + 1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
    lmax = max(lmax, block_absmax_bits(w));
  }
  const float amax = __uint_as_float(wave_max_u32(lmax) << 16);
  const float s = amax / (FOS ? 1536.0f : 2688.0f);
  if (lane == 0) tscale[row] = s;
  const float s6 = 6.0f * s, s4 = 4.0f * s;
  for (int j = lane; j < nblk; j += 64) {
    const uint4 a = x[2 * (base + j)], bq = x[2 * (base + j) + 1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
    quantize_block<FOS, DQ>(w, block_absmax_bits(w), s, s6, s4, base + j, codes, scales, dq);
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
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t word = (k < 4) ? cw.x : cw.y;
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t nib = (word >> (8 * (k & 3) + 4 * h)) & 15u;
      const float ge = e2m1_value(nib & 7u) * e;
      const float c = ge * s;
      v[h] = (nib & 8u) ? -c : c;
    }
    o[k] = pack_bf16x2(v[0], v[1]);
  }
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
