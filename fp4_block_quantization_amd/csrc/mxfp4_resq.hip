// mxfp4_resq.hip -- MXFP4 quantization with a Rollout-ResQ residual (K3)
// for gfx950.
//
// Method: "HiFloat4 Format for End-To-End Reinforcement Learning
// Post-Training of Large Language Models" (agifrontier.github.io), section
// on Rollout-ResQ and hardware-aware sparsity.  The rollout projection is
// rebuilt as Q(X)Q(W)^T + S(Q(dX))Q(W)^T with dX = X - Q(X); MXFP4 keeps
// one E8M0 scale per 32 E2M1 values; S_{2:4} keeps 2 of every 4
// consecutive values of the quantized residual.  This kernel produces
// Q(X), Q(dX)'s scale and its 2:4-compressed codes in one pass; the
// residual itself never leaves registers.
//
// Mapping: one lane per 32-element block; no cross-lane work.
#include "fp4q_device.h"
#include "fp4q_launch.h"

namespace fp4q {

namespace {

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// MXFP4 of 32 FP32 values: packed nibbles (element 2i in the low nibble of
// byte i) and the exact dequantized values +-g * 2^k.  Returns the E8M0
// byte k + 127.  x * 2^-k is exact (or far below the first code), so the
// hardware E2M1 conversion of the scaled value is the reference rounding.
__device__ __forceinline__ uint32_t mx_quantize32(const float (&v)[32], uint32_t (&cw)[4],
                                                  float (&deq)[32]) {
  uint32_t mbits = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) mbits = max(mbits, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  const int k = mx_exponent(mbits);
  const float down = __uint_as_float((uint32_t)(127 - k) << 23);  // 2^-k, k in [-127, 125]
  static_for<0, 16>([&](auto P) {
    constexpr int p = decltype(P)::value;
    cw[p >> 2] = cvt_e2m1x2<p & 3>(p & 3 ? cw[p >> 2] : 0u, v[2 * p] * down,
                                    v[2 * p + 1] * down);
    const float2v g = e2m1x2_values<p & 3>(cw[p >> 2]);
    deq[2 * p] = ldexpf(g.x, k);  // exact
    deq[2 * p + 1] = ldexpf(g.y, k);
  });
  return (uint32_t)(k + 127);
}

__global__ __launch_bounds__(256) void mxfp4_resq_blocks(
    const uint4* __restrict__ x, int64_t nblocks, uint4* __restrict__ codes,
    uint8_t* __restrict__ scales, uint2* __restrict__ res_codes, uint32_t* __restrict__ res_meta,
    uint8_t* __restrict__ res_scales) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;

  float v[32];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint4 a = x[4 * blk + p];
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * p + 2 * k] = bf16_lo(w[k]);
      v[8 * p + 2 * k + 1] = bf16_hi(w[k]);
    }
  }

  uint32_t cw[4];
  float deq[32];
  scales[blk] = (uint8_t)mx_quantize32(v, cw, deq);
  codes[blk] = make_uint4(cw[0], cw[1], cw[2], cw[3]);

  // residual, exact in FP32, quantized again over all 32 values
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = v[i] - deq[i];
  res_scales[blk] = (uint8_t)mx_quantize32(v, cw, deq);

  // S_{2:4}: per group of 4 keep the two largest magnitudes, ties to the
  // lower index.  Key = magnitude * 4 + (3 - index) orders uniquely; the
  // two largest of four keys come from a max/min network.
  uint32_t rc[2] = {0u, 0u}, meta = 0u;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const uint32_t word = cw[g >> 1] >> (16 * (g & 1));  // this group's 4 nibbles
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) key[i] = (((word >> (4 * i)) & 7u) << 2) | (3u - i);
    const uint32_t p = max(key[0], key[1]), q = min(key[0], key[1]);
    const uint32_t r = max(key[2], key[3]), t = min(key[2], key[3]);
    const uint32_t k1 = max(p, r), k2 = max(min(p, r), max(q, t));
    const uint32_t ia = 3u - (k1 & 3u), ib = 3u - (k2 & 3u);
    const uint32_t i0 = min(ia, ib), i1 = max(ia, ib);
    const uint32_t n0 = (word >> (4 * i0)) & 15u, n1 = (word >> (4 * i1)) & 15u;
    rc[g >> 2] |= (n0 | (n1 << 4)) << (8 * (g & 3));
    meta |= (i0 | (i1 << 2)) << (4 * g);
  }
  res_codes[blk] = make_uint2(rc[0], rc[1]);
  res_meta[blk] = meta;
}

}  // namespace

hipError_t mxfp4_resq_launch(const void* x, int64_t rows, int64_t hidden, uint8_t* codes,
                             uint8_t* scales, uint8_t* res_codes, uint8_t* res_meta,
                             uint8_t* res_scales, hipStream_t st) {
  const int64_t nblocks = rows * (hidden / 32);
  const dim3 grid((unsigned)((nblocks + 255) / 256)), block(256);
  hipLaunchKernelGGL(mxfp4_resq_blocks, grid, block, 0, st, (const uint4*)x, nblocks,
                     (uint4*)codes, scales, (uint2*)res_codes, (uint32_t*)res_meta, res_scales);
  return hipGetLastError();
}

}  // namespace fp4q
