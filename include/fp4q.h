/*
 * fp4q.h -- C ABI of the MI355X (gfx950) fused FP4 block quantizer.
 *
 * Three operations, each one or more hand-written HIP kernels:
 *
 *   nvfp4_quantize      per-token NVFP4 with Four-Over-Six and the exact
 *                       BF16 dequantized tensor
 *   nvfp4_dequantize    BF16 dequantization of stored NVFP4 values
 *   mxfp4_resq_quantize MXFP4 with a re-quantized, 2:4-sparsified residual
 *                       (Rollout-ResQ)
 *
 * Conventions shared by every call
 *   - Every data pointer is a DEVICE pointer on the device the call's
 *     stream belongs to (the current HIP device for the NULL stream).  The
 *     caller allocates and frees all memory; the library allocates nothing
 *     and keeps no state between calls, apart from the fixed per-device
 *     scratch array of nvfp4_quantize_global_noalloc (below).
 *   - Tensors are row-major and contiguous: [rows, hidden], hidden innermost.
 *     BF16 is passed as 16-bit patterns (void*).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream).  Arguments are validated on the host before anything is
 *     launched; a rejected call returns its status and writes nothing.
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - Outputs must not alias inputs or each other.
 *   - Inputs must be finite.  NaN or infinity is outside the domain: the
 *     kernels stay memory-safe but the output values are unspecified.
 *   - Results depend only on the input values: they are bit-identical for
 *     any stream, batch composition, row order or launch, and bit-identical
 *     to the CPU reference.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stdint.h>

/* The calls below are the library's only exported symbols. */
#define FP4Q_API __attribute__((visibility("default")))

/* Bytes of device workspace nvfp4_quantize_global needs, whatever the
   tensor's size: one 2-byte partial maximum per workgroup of its tensor-max
   pass, which has at most 512 workgroups. */
#define FP4Q_GLOBAL_WORKSPACE_BYTES 1024

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4Q_SUCCESS = 0,
  FP4Q_ERROR_NULL_POINTER = 1,  /* a required pointer is NULL                */
  FP4Q_ERROR_INVALID_SHAPE = 2, /* rows < 0, hidden <= 0, hidden not a
                                   multiple of the block size, num_groups < 0,
                                   or a size too large to index              */
  FP4Q_ERROR_MISALIGNED = 3,    /* a pointer lacks the alignment stated at
                                   its argument                              */
  FP4Q_ERROR_LAUNCH = 4,        /* the HIP launch failed (no device, bad
                                   stream, ...)                             */
  FP4Q_ERROR_INVALID_ARGUMENT = 5 /* an option outside its documented
                                     values (four_over_six not 0, 1 or 2)   */
} fp4q_status;

/*
 * nvfp4_quantize -- per-token NVFP4 with Four-Over-Six.
 *
 * Definition: "humans& Open-Sources the First Stable 4-Bit RL Training
 * Recipe at 1.73x Speedup" (alphasignal.ai), sections 1-3, and "NVFP4-RL"
 * (jianyuh.github.io), section 2 (each token's FP32 scale over the hidden
 * dimension, computed together with the FP8 E4M3 block scales in one
 * kernel), section 3 (the dequantized value of the exact quantized tensor
 * feeds the BF16 backward) and section 4 (Four-Over-Six candidate formula).
 * Per row r with amax = max |x|:
 *   s = amax / 1536 (four_over_six) or amax / 2688 (6 only), FP32;
 *   per 16-element block with max b, per candidate k in {6, 4}:
 *     e_k = E4M3_RNE(b / (k*s)), d_k = e_k*s, r_k = 1/d_k,
 *     q_i = E2M1_RNE(|x_i| * r_k), c_i = +-((g(q_i) * e_k) * s),
 *     err_k = sum_i (x_i - c_i)^2 in element order;
 *   candidate 4 wins only if err_4 < err_6 (ties keep 6).
 * Every step is one IEEE binary32 operation (no FMA contraction, division
 * correctly rounded, subnormals kept).
 *
 *   x             BF16 [rows, hidden], 16-byte aligned.
 *   rows          >= 0 (0: nothing is launched).
 *   hidden        > 0, a multiple of 16.
 *   group_offsets NULL, or int64 [num_groups + 1] on the device, 8-byte
 *                 aligned, with 0 <= off[0] <= ... <= off[num_groups] <=
 *                 rows (routed tokens grouped per expert).  Only rows
 *                 [off[0], off[num_groups]) are read and written; the
 *                 others keep their contents.  The offsets are not checked
 *                 on the host (that would need a synchronisation); the
 *                 kernel clamps the range to [0, rows), so wrong offsets
 *                 cannot cause an out-of-bounds access.
 *   num_groups    0 when group_offsets is NULL, else >= 1.
 *   four_over_six 1: s = amax/1536 and the 4/6 choice per block on the
 *                    FP32 squared error above;
 *                 2: the same, but the choice is made on the FP16 fast
 *                    path's error ("NVFP4-RL", section 4, "The
 *                    optimization": products g*e in FP16, where they are
 *                    exact; the target scaled down by the inverse token
 *                    scale): y_i = FP16(|x_i| * fl(1/s)), per candidate
 *                    err16 = sum in element order, in FP32, of
 *                    FP16(y_i - g_i*e_k)^2; 4 iff err16_4 < err16_6.  Codes,
 *                    scales and dequant values are those of the chosen
 *                    candidate, as with 1; on the workloads measured the
 *                    choice differs from 1's in about 0.1% of blocks;
 *                 0: s = amax/2688 and the 6 candidate only.
 *                 Other values: FP4Q_ERROR_INVALID_ARGUMENT.
 *   codes         uint8 [rows, hidden/2], 8-byte aligned: E2M1 nibbles,
 *                 sign in bit 3, element 2i in the low nibble of byte i.
 *   block_scales  uint8 [rows, hidden/16]: OCP E4M3FN bit patterns.
 *   token_scales  float [rows], 4-byte aligned: s.
 *   dequant       BF16 [rows, hidden], 16-byte aligned, or NULL to skip:
 *                 BF16_RNE(c_i) of the chosen candidate.
 *   stream        hipStream_t or NULL.
 */
FP4Q_API fp4q_status nvfp4_quantize(const void* x, int64_t rows, int64_t hidden,
                           const int64_t* group_offsets, int64_t num_groups,
                           int four_over_six, uint8_t* codes,
                           uint8_t* block_scales, float* token_scales,
                           void* dequant, void* stream);

/*
 * nvfp4_dequantize -- BF16 values of stored NVFP4 data.
 *
 * Definition: "NVFP4-RL" (jianyuh.github.io), section 3 (dequantized
 * backward, y = x . DQ(Q(w))) and section 4 (candidate formula):
 *   out_i = BF16_RNE(+-((g(code_i & 7) * e_block) * s_row)),
 * the sign from bit 3 of the nibble.  Given the outputs of nvfp4_quantize
 * it reproduces that call's dequant tensor bit for bit.
 *
 *   codes         uint8 [rows, hidden/2], 8-byte aligned.
 *   block_scales  uint8 [rows, hidden/16].
 *   token_scales  float [rows], 4-byte aligned.
 *   rows          >= 0; hidden > 0, a multiple of 16.
 *   out           BF16 [rows, hidden], 16-byte aligned.
 */
FP4Q_API fp4q_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* block_scales,
                             const float* token_scales, int64_t rows,
                             int64_t hidden, void* out, void* stream);

/*
 * nvfp4_quantize_global -- NVFP4 with one FP32 scale for the whole tensor.
 *
 * The naive NVFP4 that "humans& Open-Sources the First Stable 4-Bit RL
 * Training Recipe" (section 1) and "NVFP4-RL" (section 2) contrast with
 * per-token scaling: s = amax over the whole tensor / 1536 (four_over_six 1
 * or 2) or / 2688 (0), then the block path of nvfp4_quantize in every row
 * under that s.  A row's outputs therefore depend on the other rows (the
 * batch dependency those pages warn about).
 *
 * Two kernels: a tensor-max pass writes one partial maximum per workgroup
 * into the workspace; the quantize pass reduces them in every wavefront,
 * derives s and quantizes the blocks under it.
 *
 *   x, codes, block_scales, dequant, four_over_six: as for nvfp4_quantize
 *                 (no ragged rows).
 *   tensor_scale  float [1], 4-byte aligned, device memory: receives s.
 *   workspace     device memory of FP4Q_GLOBAL_WORKSPACE_BYTES bytes,
 *                 16-byte aligned, owned by the caller: holds the partial
 *                 maxima between the two kernels.  Its contents on entry are
 *                 ignored and on return unspecified; it must not overlap
 *                 an input or output.
 * Concurrent calls must not share tensor_scale or workspace.
 */
FP4Q_API fp4q_status nvfp4_quantize_global(const void* x, int64_t rows, int64_t hidden,
                                  int four_over_six, uint8_t* codes, uint8_t* block_scales,
                                  float* tensor_scale, void* dequant, void* workspace,
                                  void* stream);

/*
 * nvfp4_quantize_global_noalloc -- nvfp4_quantize_global without the
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It allocates nothing: the partial maxima live in a fixed
 * 1 KiB array of the library's own (FP4Q_GLOBAL_WORKSPACE_BYTES), one per
 * device, held until the process ends; its address is looked up once per
 * device on the first call there (the stream's device, or the current
 * device for the NULL stream; that lookup briefly makes the stream's
 * device current and then restores the caller's).  The scratch need does
 * not grow with the tensor (at most 512 partial maxima), so no size within
 * the limits of nvfp4_quantize_global is refused for it.  Every call on a device shares
 * that device's array: calls that overlap on one device (other streams, or
 * other host threads) race and must not be in flight together.  Arguments,
 * outputs and results are those of nvfp4_quantize_global;
 * FP4Q_ERROR_LAUNCH also reports a failed lookup of the array.
 */
FP4Q_API fp4q_status nvfp4_quantize_global_noalloc(const void* x, int64_t rows, int64_t hidden,
                                          int four_over_six, uint8_t* codes,
                                          uint8_t* block_scales, float* tensor_scale,
                                          void* dequant, void* stream);

/*
 * nvfp4_quantize_guided -- TRACE rollout-guided rounding.
 *
 * Definition: "TRACE FP4 RL -- Rollout-guided FP4 rounding"
 * (learnaivisually.com): the training engine rounds each captured value,
 * between its two neighbouring FP4 codewords, toward the codeword the
 * rollout engine chose, under the same rollout-side scale.  With the
 * rollout's E4M3 block scale e and token scale s (as nvfp4_quantize stored
 * them), per element:
 *   v = |x_i| * fl(1 / fl(e*s))  (0 when e*s == 0);
 *   lo = the largest E2M1 magnitude code with g <= v, hi = the smallest
 *   with g >= v (equal when v is a grid value; 7 for both above 6);
 *   with G the guide's signed value and sigma the sign of x_i, the code is
 *   hi if |sigma*g(hi) - G| < |sigma*g(lo) - G|, else lo; the sign bit
 *   follows x_i.  Guided by its own round-to-nearest codes it returns them.
 *   With guide_codes NULL every element takes its nearest codeword,
 *   E2M1_RNE(v), under the same scales: the training side's own rounding
 *   that the page's worked example and its count of mismatches between
 *   adjacent codewords set guided rounding against.
 *
 *   x             BF16 [rows, hidden] (training side), 16-byte aligned.
 *   guide_codes   uint8 [rows, hidden/2], 4-byte aligned: the rollout's
 *                 codes; or NULL (round to nearest).
 *   block_scales  uint8 [rows, hidden/16], token_scales float [rows] (4-byte
 *                 aligned): the rollout's scales, read only.
 *   codes         uint8 [rows, hidden/2], 4-byte aligned: the guided codes.
 *   dequant       BF16 [rows, hidden], 16-byte aligned, or NULL:
 *                 BF16(+-((g*e)*s)) of the guided codes.
 */
FP4Q_API fp4q_status nvfp4_quantize_guided(const void* x, int64_t rows, int64_t hidden,
                                  const uint8_t* guide_codes, const uint8_t* block_scales,
                                  const float* token_scales, uint8_t* codes, void* dequant,
                                  void* stream);

/*
 * mxfp4_resq_quantize -- MXFP4 with a Rollout-ResQ residual.
 *
 * Definition: "HiFloat4 Format for End-To-End Reinforcement Learning
 * Post-Training of Large Language Models" (agifrontier.github.io), section
 * on Rollout-ResQ and hardware-aware sparsity: MXFP4 is E2M1 data under one
 * E8M0 scale per 32 elements; the residual dX = X - Q(X) is quantized
 * again and S_{2:4} keeps 2 of every 4 consecutive elements of Q(dX).  Per
 * 32-element block with max b:
 *   k = clamp(floor(log2 b) - 2, -127, 127) (b == 0: -127), E8M0 byte k+127;
 *   q_i = E2M1_RNE(|x_i| * 2^-k); DQ_i = +-g(q_i) * 2^k (exact);
 *   dX_i = x_i - DQ_i (exact in FP32); the residual gets its own k' and
 *   codes q'_i by the same rule over all 32 residuals;
 *   per group of 4 consecutive residual codes keep the two largest
 *   magnitudes (ties to the lower index), indices i0 < i1.
 *
 *   x           BF16 [rows, hidden], 16-byte aligned; hidden a multiple of 32.
 *   codes       uint8 [rows, hidden/2], 16-byte aligned: primary E2M1
 *               nibbles, element 2i in the low nibble.
 *   scales      uint8 [rows, hidden/32]: primary E8M0 (2^(byte-127)).
 *   res_codes   uint8 [rows, hidden/4], 8-byte aligned: per group of 4, the
 *               kept residual nibble at i0 (low) and at i1 (high).
 *   res_meta    uint8 [rows, hidden/8], 4-byte aligned: per group the
 *               nibble i0 | i1 << 2; group 2m in the low nibble of byte m.
 *   res_scales  uint8 [rows, hidden/32]: residual E8M0.
 */
FP4Q_API fp4q_status mxfp4_resq_quantize(const void* x, int64_t rows, int64_t hidden,
                                uint8_t* codes, uint8_t* scales,
                                uint8_t* res_codes, uint8_t* res_meta,
                                uint8_t* res_scales, void* stream);

/*
 * mxfp4_resq_dense_quantize -- Rollout-ResQ-Dense: the same primary MXFP4
 * and residual quantization as mxfp4_resq_quantize, with every residual
 * code kept (the dense correction Q(X)Q(W)^T + Q(dX)Q(W)^T that the same
 * HiFloat4 page compares with the S_{2:4} one).
 *
 *   x, codes, scales, res_scales: as for mxfp4_resq_quantize.
 *   res_codes   uint8 [rows, hidden/2], 16-byte aligned: residual E2M1
 *               nibbles, packed like codes.
 */
FP4Q_API fp4q_status mxfp4_resq_dense_quantize(const void* x, int64_t rows, int64_t hidden,
                                      uint8_t* codes, uint8_t* scales,
                                      uint8_t* res_codes, uint8_t* res_scales,
                                      void* stream);

/*
 * mxfp4_resq_reconstruct -- the tensor the Rollout-ResQ projection sees,
 * X_hat = DQ(Q(X)) + DQ(S(Q(dX))) (same HiFloat4 page section), for error
 * analysis of the residual correction:
 *   residual 0: X_hat = DQ(Q(X)); res_* are not read (may be NULL);
 *   residual 1: + DQ(S(Q(dX))) from mxfp4_resq_quantize's res_codes
 *               [rows, hidden/4] (8-byte aligned), res_meta [rows, hidden/8]
 *               and res_scales; the two dropped elements of a group add 0;
 *   residual 2: + DQ(Q(dX)) from mxfp4_resq_dense_quantize's res_codes
 *               [rows, hidden/2] (16-byte aligned) and res_scales; res_meta
 *               is not read.
 * Each term is +-g * 2^(byte-127), exact in FP32; their sum is one FP32
 * addition.  Other residual values: FP4Q_ERROR_INVALID_ARGUMENT.
 *
 *   codes       uint8 [rows, hidden/2], 16-byte aligned; scales [rows, hidden/32].
 *   rows >= 0; hidden > 0, a multiple of 32.
 *   out         float [rows, hidden], 16-byte aligned.
 */
FP4Q_API fp4q_status mxfp4_resq_reconstruct(const uint8_t* codes, const uint8_t* scales,
                                   const uint8_t* res_codes, const uint8_t* res_meta,
                                   const uint8_t* res_scales, int64_t rows, int64_t hidden,
                                   int residual, float* out, void* stream);

/* Static description of a status (never NULL). */
FP4Q_API const char* fp4q_status_string(fp4q_status status);

#ifdef __cplusplus
}
#endif
#endif /* FP4Q_H */
