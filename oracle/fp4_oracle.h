/*
 * fp4_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded CPU reference of the fused FP4 block
 * quantizer.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark may load it.  The GPU library never includes, links or
 * calls anything here, and nothing here is shared with the GPU library.
 *
 * Every floating-point step is one IEEE binary32 operation with
 * round-to-nearest-even, in the order written in fp4_oracle.c; build with
 * -O2 -ffp-contract=off and no fast-math so that the compiler keeps it so.
 *
 * All pointers are HOST pointers.  BF16 values travel as their uint16_t bit
 * patterns.  Functions return 0 on success and a positive status on a
 * rejected argument (same numbering as the GPU library's fp4q_status).
 */
#ifndef FP4_ORACLE_H
#define FP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- primitives ------------------------------------------------------- */

/* E2M1 magnitude code 0..7 of a >= 0 (round to nearest, ties to the even
 * code, saturating at 6; NaN gives 0). */
int oracle_e2m1_code(float a);
/* Magnitude of E2M1 code q (0..7): {0, 0.5, 1, 1.5, 2, 3, 4, 6}. */
float oracle_e2m1_value(int q);
/* OCP E4M3FN byte of t >= 0 (round to nearest, ties to even mantissa,
 * saturating at 448, t == 0 or NaN gives 0x00). */
uint8_t oracle_e4m3_encode(float t);
/* Exact value of an E4M3FN byte (sign bit honoured, 0x7F/0xFF give NaN). */
float oracle_e4m3_decode(uint8_t byte);
/* FP32 -> BF16 bit pattern, round to nearest even, subnormals kept. */
uint16_t oracle_bf16_rne(float f);
/* MX shared exponent of a block whose max magnitude is b >= 0:
 * floor(log2 b) - 2 clamped to [-127, 127]; b == 0 gives -127. */
int oracle_e8m0_exponent(float b);

/* IEEE binary16 round-to-nearest-even of v, returned as a double. */
double oracle_fp16_rne(double v);

/* ---- NVFP4, one block, with its internals (for tests) ------------------ */

typedef struct {
  float t[2];      /* [0]: 6-candidate, [1]: 4-candidate target scale t_k   */
  float e[2];      /* E4M3 value e_k                                        */
  uint8_t e_byte[2];
  float err[2];    /* summed squared error of the candidate                 */
  float err16[2];  /* the FP16 fast path's error (four_over_six == 2)       */
  float cand[2][16]; /* signed FP32 candidate dequant values                */
  uint8_t code[2][16]; /* nibbles (sign << 3 | magnitude code)              */
  int choice;      /* 6 or 4                                                */
} oracle_nvfp4_block_t;

/* Quantize one 16-element block x16 (FP32 values, exactly BF16) under the
 * token scale s.  four_over_six: 0, the 6-candidate only; 1, 4 and 6
 * compete on the FP32 squared error; 2, 4 and 6 compete on the FP16 fast
 * path's error (same codes and scales, possibly a different choice). */
void oracle_nvfp4_block(const float* x16, float s, int four_over_six,
                        oracle_nvfp4_block_t* out);

/* ---- whole-tensor entry points (twins of the GPU library's calls) ------ */

int nvfp4_quantize_ref(const uint16_t* x, int64_t rows, int64_t hidden,
                       const int64_t* group_offsets, int64_t num_groups,
                       int four_over_six, uint8_t* codes, uint8_t* block_scales,
                       float* token_scales, uint16_t* dequant);

int nvfp4_dequantize_ref(const uint8_t* codes, const uint8_t* block_scales,
                         const float* token_scales, int64_t rows,
                         int64_t hidden, uint16_t* out);

int mxfp4_resq_quantize_ref(const uint16_t* x, int64_t rows, int64_t hidden,
                            uint8_t* codes, uint8_t* scales,
                            uint8_t* res_codes, uint8_t* res_meta,
                            uint8_t* res_scales);

/* Rollout-ResQ-Dense: res_codes [rows, hidden/2] keeps every residual code. */
int mxfp4_resq_dense_quantize_ref(const uint16_t* x, int64_t rows, int64_t hidden,
                                  uint8_t* codes, uint8_t* scales,
                                  uint8_t* res_codes, uint8_t* res_scales);

/* FP32 reconstruction DQ(Q(X)) (+ DQ(S(Q(dX))) for residual 1, + DQ(Q(dX))
 * for residual 2). */
int mxfp4_resq_reconstruct_ref(const uint8_t* codes, const uint8_t* scales,
                               const uint8_t* res_codes, const uint8_t* res_meta,
                               const uint8_t* res_scales, int64_t rows, int64_t hidden,
                               int residual, float* out);

/* One FP32 scale for the whole tensor (the naive baseline). */
int nvfp4_quantize_global_ref(const uint16_t* x, int64_t rows, int64_t hidden,
                              int four_over_six, uint8_t* codes, uint8_t* block_scales,
                              float* tensor_scale, uint16_t* dequant);

/* TRACE rollout-guided rounding under the rollout's scales (guide_codes
 * NULL: round-to-nearest under those scales). */
int nvfp4_quantize_guided_ref(const uint16_t* x, int64_t rows, int64_t hidden,
                              const uint8_t* guide_codes, const uint8_t* block_scales,
                              const float* token_scales, uint8_t* codes,
                              uint16_t* dequant);

#ifdef __cplusplus
}
#endif
#endif /* FP4_ORACLE_H */
