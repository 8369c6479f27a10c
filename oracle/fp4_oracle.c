/*
 * fp4_oracle.c -- TEST INFRASTRUCTURE ONLY (see fp4_oracle.h).
 *
 * A plain CPU statement of what the fused FP4 quantizer computes, written
 * step by step from the pages it follows:
 *
 *  - "humans& Open-Sources the First Stable 4-Bit RL Training Recipe at
 *    1.73x Speedup" (alphasignal.ai), sections 1 (per-token activation
 *    scaling), 2 (dequantized gradients) and 3 (Four-Over-Six scaling);
 *  - "NVFP4-RL" (jianyuh.github.io, 2026-07-11), section 2 (per-token
 *    scales, FP8 E4M3 block scales fused into the quantization kernel),
 *    section 3 (dequantized backward, y = x . DQ(Q(w))) and section 4 (the
 *    Four-Over-Six candidate formula);
 *  - "TRACE FP4 RL -- Rollout-guided FP4 rounding" (learnaivisually.com),
 *    Jargon (the E2M1 magnitude set; round-to-nearest) and the worked
 *    example (the halfway line at 2.5 between codewords 2 and 3);
 *  - "HiFloat4 Format for End-To-End Reinforcement Learning Post-Training
 *    of Large Language Models" (agifrontier.github.io), section on
 *    Rollout-ResQ and hardware-aware sparsity (residual
 *    dX = X - Q(X), its re-quantization, the S_{2:4} sparsifier, and MXFP4
 *    as 32-element blocks with one E8M0 scale over E2M1 data).
 *
 * Where those pages leave a step open, the reading taken here is stated at
 * the step.  The fixed numeric conventions are:
 *   - token scale s = amax / 1536 (= 6 * 256) with Four-Over-Six on and
 *     amax / 2688 (= 6 * 448) with it off, so that both candidate block
 *     scales of the row-max block fit E4M3's 448 (the blog names the
 *     constant E4M3_4OVER6_MAXVAL without a value; 256 is the reading);
 *   - block scales are OCP E4M3FN rounded to nearest even;
 *   - every FP32 operation is separately IEEE-rounded (no FMA), division
 *     included.
 *
 * Deliberately slow: one row, one block, one element at a time.
 */
#include "fp4_oracle.h"

#include <math.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* primitives                                                               */
/* ------------------------------------------------------------------------ */

static float bf16_bits_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16; /* BF16 is the top half of an FP32 */
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* The E2M1 magnitudes, from the TRACE page's Jargon entry on FP4 (E2M1):
 * 0, 0.5, 1, 1.5, 2, 3, 4 and 6.  The code of a magnitude is its index in
 * this sorted list (the OCP E2M1 bit pattern: 2 exponent bits, 1 mantissa
 * bit); the sign is a separate bit 3. */
static const float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float oracle_e2m1_value(int q) { return kE2M1[q & 7]; }

/* Round-to-nearest onto the E2M1 grid (TRACE page, Jargon: RTN maps a value
 * to the closest codeword; worked example: 2.49 -> 2, 2.51 -> 3).  The code
 * is the number of grid midpoints lying below a.  An exact midpoint goes to
 * the neighbour with the even code, so each comparison is strict (">") where
 * the lower neighbour's code is even and non-strict (">=") where it is odd.
 * Values above 6 saturate to code 7; a NaN fails every test and gives 0. */
int oracle_e2m1_code(float a) {
  int q = 0;
  q += (a > 0.25f);  /* between 0   (code 0) and 0.5 (code 1) */
  q += (a >= 0.75f); /* between 0.5 (code 1) and 1   (code 2) */
  q += (a > 1.25f);  /* between 1   (code 2) and 1.5 (code 3) */
  q += (a >= 1.75f); /* between 1.5 (code 3) and 2   (code 4) */
  q += (a > 2.5f);   /* between 2   (code 4) and 3   (code 5) */
  q += (a >= 3.5f);  /* between 3   (code 5) and 4   (code 6) */
  q += (a > 5.0f);   /* between 4   (code 6) and 6   (code 7) */
  return q;
}

/* OCP E4M3FN: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; normal
 * binades 2^-6 .. 2^8, subnormal step 2^-9, largest finite value 448
 * (byte 0x7E), no infinity (0x7F is NaN).  The NVFP4-RL blog section 2 calls
 * the block scale "FP8 E4M3"; the OCP variant with max 448 is the reading. */
uint8_t oracle_e4m3_encode(float t) {
  double a = (double)t;
  if (!(a > 0.0)) return 0x00; /* zero (either sign) and NaN */
  if (a > 448.0) return 0x7E;  /* saturate at the largest finite value */

  int ex;
  (void)frexp(a, &ex); /* 2^(ex-1) <= a < 2^ex */
  int binade = ex - 1;
  if (binade < -6) binade = -6; /* subnormals share the step of binade -6 */
  double step = ldexp(1.0, binade - 3); /* 3 fraction bits per binade */

  /* Round a / step (exact in double) to the nearest integer, ties to even:
   * the parity of that integer is the parity of the mantissa. */
  double n = a / step;
  double lo = floor(n);
  double frac = n - lo;
  if (frac > 0.5 || (frac == 0.5 && fmod(lo, 2.0) != 0.0)) lo += 1.0;
  double v = lo * step;
  if (v > 448.0) v = 448.0;
  if (v == 0.0) return 0x00;

  if (v < ldexp(1.0, -6)) /* subnormal: exponent field 0 */
    return (uint8_t)(int)(v / ldexp(1.0, -9));
  (void)frexp(v, &ex);
  binade = ex - 1;
  int mant = (int)(v / ldexp(1.0, binade - 3)) - 8; /* 0..7 */
  return (uint8_t)(((binade + 7) << 3) | mant);
}

float oracle_e4m3_decode(uint8_t byte) {
  int negative = (byte >> 7) & 1;
  int expo = (byte >> 3) & 15;
  int mant = byte & 7;
  if (expo == 15 && mant == 7) return NAN;
  double v = (expo == 0) ? ldexp((double)mant, -9)
                         : ldexp((double)(8 + mant), expo - 7 - 3);
  return (float)(negative ? -v : v);
}

/* FP32 -> BF16 with round to nearest even: keep the top 16 bits of the
 * binary32 pattern; the dropped low 16 bits decide -- above one half of the
 * last kept place rounds up, exactly one half rounds to the even kept
 * pattern.  A carry into the exponent field is the correctly rounded result
 * (the next binade, or infinity past the largest finite value). */
uint16_t oracle_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t hi = u >> 16;
  uint32_t lo = u & 0xFFFFu;
  if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

/* IEEE binary16 rounding to nearest even of a double (11 significant bits,
 * normal binades 2^-14 .. 2^15, subnormal step 2^-24, largest finite
 * 65504; at or above 65520 in magnitude the result is infinity).  Returns
 * the rounded value as a double. */
double oracle_fp16_rne(double v) {
  if (v != v) return v;
  double a = fabs(v);
  if (a == 0.0 || isinf(a)) return v;
  int ex;
  (void)frexp(a, &ex); /* 2^(ex-1) <= a < 2^ex */
  int binade = ex - 1;
  if (binade < -14) binade = -14; /* subnormals share the step of 2^-14 */
  double step = ldexp(1.0, binade - 10);
  double n = a / step; /* exact: a has at most 53 bits, step a power of 2 */
  double lo = floor(n);
  double frac = n - lo;
  if (frac > 0.5 || (frac == 0.5 && fmod(lo, 2.0) != 0.0)) lo += 1.0;
  double r = lo * step;
  if (r > 65504.0) r = INFINITY;
  return v < 0 ? -r : r;
}

/* MX shared exponent (HiFloat4 page, Rollout-ResQ section: MXFP4 keeps one
 * E8M0 scale per 32 elements).  The page gives no rule; the reading is the
 * OCP MX one -- the largest power of two not above the block max, divided
 * by the largest power of two of E2M1 (2^2) -- so k = floor(log2 b) - 2,
 * clamped to the E8M0 range.  An all-zero block gets the smallest scale. */
int oracle_e8m0_exponent(float b) {
  if (!(b > 0.0f)) return -127;
  int ex;
  (void)frexp((double)b, &ex); /* floor(log2 b) = ex - 1, subnormals too */
  int k = (ex - 1) - 2;
  if (k < -127) k = -127;
  if (k > 127) k = 127;
  return k;
}

/* ------------------------------------------------------------------------ */
/* NVFP4 with Four-Over-Six                                                 */
/* ------------------------------------------------------------------------ */

/* One 16-element block under the token scale s.
 *
 * Candidates (NVFP4-RL blog section 4; humans& article section 3): the
 * block max is mapped either to 6 (the usual NVFP4 mapping) or to 4; the
 * candidate that gives the lower squared error wins, and a tie keeps 6.
 *
 * Per candidate k in {6, 4}:
 *   t_k = b / (k * s)            target block scale (FP32, IEEE division)
 *   e_k = E4M3(t_k)              stored block scale
 *   d_k = e_k * s                decode step of the block
 *   r_k = 1 / d_k                the blog's "scale the target down by its
 *                                inverse": one reciprocal per block
 *   q_i = E2M1(|x_i| * r_k)      magnitude code of each element
 *   c_i = +-((g(q_i) * e_k) * s) the blog's candidate formula
 *                                fp4_value * fp8_scale * amax / (6 * 256),
 *                                read left to right with the stored token
 *                                scale s standing for amax / (6 * 256)
 *   err_k = sum_i (x_i - c_i)^2  squared error in the x domain, summed in
 *                                element order 0..15
 * A zero block (or a zero token scale) gives e_k = 0; a zero decode step
 * gives magnitude code 0 for every element. */
void oracle_nvfp4_block(const float* x, float s, int four_over_six,
                        oracle_nvfp4_block_t* out) {
  static const float kMapTo[2] = {6.0f, 4.0f};
  memset(out, 0, sizeof *out);

  float b = 0.0f;
  for (int i = 0; i < 16; ++i) {
    float a = fabsf(x[i]);
    if (a > b) b = a;
  }

  int candidates = four_over_six ? 2 : 1;
  for (int k = 0; k < 2; ++k) out->err[k] = out->err16[k] = NAN;

  for (int k = 0; k < candidates; ++k) {
    float t = 0.0f;
    uint8_t e_byte = 0x00;
    if (b != 0.0f && s != 0.0f) {
      float ks = kMapTo[k] * s;
      t = b / ks;
      e_byte = oracle_e4m3_encode(t);
    }
    float e = oracle_e4m3_decode(e_byte);
    float d = e * s;
    float r = 0.0f;
    if (d != 0.0f) r = 1.0f / d;

    float err = 0.0f;
    for (int i = 0; i < 16; ++i) {
      float a = fabsf(x[i]);
      int q = 0;
      if (d != 0.0f) {
        float v = a * r;
        q = oracle_e2m1_code(v);
      }
      float ge = oracle_e2m1_value(q) * e; /* exact: <= 6 significant bits */
      float c = ge * s;
      int negative = signbit(x[i]) ? 1 : 0;
      if (negative) c = -c;
      float delta = x[i] - c;
      float sq = delta * delta;
      err = err + sq;
      out->cand[k][i] = c;
      out->code[k][i] = (uint8_t)((negative << 3) | q);
    }
    out->t[k] = t;
    out->e[k] = e;
    out->e_byte[k] = e_byte;
    out->err[k] = err;
  }
  /* Strictly lower error picks 4; equality (and NaN) keeps 6. */
  out->choice = (four_over_six && out->err[1] < out->err[0]) ? 4 : 6;

  /* four_over_six == 2: the NVFP4-RL blog's FP16 fast path for the same
   * decision (section 4, "The optimization").  The blog keeps the E2M1 x
   * E4M3 products in FP16, where they are exact, and scales the target
   * down by the inverse token scale instead of scaling the candidate up.
   * The reading taken here, with every step one IEEE rounding:
   *   inv_s = 1 / s                         (FP32, once per row)
   *   y_i   = FP16(|x_i| * inv_s)           target in units of s
   *   ge_i  = g(q_i) * e_k                  exact in FP16
   *   d_i   = FP16(y_i - ge_i)              FP16 difference
   *   err16_k = sum_i d_i^2                 in FP32, element order; d_i^2
   *                                         is exact in FP32, so only the
   *                                         additions round
   * Squares are summed in FP32 because in FP16 they overflow for the
   * largest blocks (d up to ~256 in units of s).  Codes, scales and
   * candidate values are those of the exact path; only the choice
   * differs, and 4 wins only with a strictly lower err16. */
  if (four_over_six == 2) {
    float inv_s = 1.0f / s;
    for (int k = 0; k < 2; ++k) {
      float err16 = 0.0f;
      for (int i = 0; i < 16; ++i) {
        float scaled = fabsf(x[i]) * inv_s;
        double y = oracle_fp16_rne((double)scaled);
        double ge = (double)oracle_e2m1_value(out->code[k][i] & 7) * (double)out->e[k];
        double d = oracle_fp16_rne(y - ge); /* y - ge exact in double */
        float sq = (float)(d * d);          /* exact: <= 22 significant bits */
        err16 = err16 + sq;
      }
      out->err16[k] = err16;
    }
    out->choice = (out->err16[1] < out->err16[0]) ? 4 : 6;
  }
}

/* One token row.  Per-token scaling (humans& article section 1; NVFP4-RL
 * blog section 2): each row takes its own FP32 scale from the max magnitude
 * over its hidden dimension, so nothing outside the row matters. */
static void nvfp4_row_with_scale(const uint16_t* xrow, int64_t hidden, int four_over_six,
                                 float s, uint8_t* codes, uint8_t* block_scales,
                                 uint16_t* dequant);

static void nvfp4_row(const uint16_t* xrow, int64_t hidden, int four_over_six,
                      uint8_t* codes, uint8_t* block_scales, float* token_scale,
                      uint16_t* dequant) {
  float amax = 0.0f;
  for (int64_t i = 0; i < hidden; ++i) {
    float a = fabsf(bf16_bits_to_float(xrow[i]));
    if (a > amax) amax = a;
  }
  float s = amax / (four_over_six ? 1536.0f : 2688.0f); /* 1 and 2: 4/6 on */
  *token_scale = s;
  nvfp4_row_with_scale(xrow, hidden, four_over_six, s, codes, block_scales, dequant);
}

/* The blocks of one row under a given FP32 scale s (the row's own, or the
 * whole tensor's). */
static void nvfp4_row_with_scale(const uint16_t* xrow, int64_t hidden, int four_over_six,
                                 float s, uint8_t* codes, uint8_t* block_scales,
                                 uint16_t* dequant) {

  for (int64_t j = 0; j < hidden / 16; ++j) {
    float x16[16];
    for (int i = 0; i < 16; ++i) x16[i] = bf16_bits_to_float(xrow[j * 16 + i]);
    oracle_nvfp4_block_t blk;
    oracle_nvfp4_block(x16, s, four_over_six, &blk);
    int k = (blk.choice == 4) ? 1 : 0;
    block_scales[j] = blk.e_byte[k];
    for (int i = 0; i < 16; i += 2) /* element 2m in the low nibble */
      codes[j * 8 + i / 2] =
          (uint8_t)(blk.code[k][i] | (blk.code[k][i + 1] << 4));
    if (dequant)
      for (int i = 0; i < 16; ++i)
        dequant[j * 16 + i] = oracle_bf16_rne(blk.cand[k][i]);
  }
}

int nvfp4_quantize_ref(const uint16_t* x, int64_t rows, int64_t hidden,
                       const int64_t* group_offsets, int64_t num_groups,
                       int four_over_six, uint8_t* codes, uint8_t* block_scales,
                       float* token_scales, uint16_t* dequant) {
  if (rows < 0 || hidden <= 0 || hidden % 16 != 0 || num_groups < 0) return 2;
  if (four_over_six < 0 || four_over_six > 2) return 5;
  if (rows == 0) return 0;
  if (!x || !codes || !block_scales || !token_scales) return 1;
  if (num_groups > 0 && !group_offsets) return 1;

  int64_t first = 0, last = rows;
  if (num_groups > 0) { /* ragged groups only bound the processed row range */
    first = group_offsets[0];
    last = group_offsets[num_groups];
    if (first < 0 || last > rows) return 2;
    for (int64_t g = 0; g < num_groups; ++g)
      if (group_offsets[g + 1] < group_offsets[g]) return 2;
  }
  for (int64_t r = first; r < last; ++r)
    nvfp4_row(x + r * hidden, hidden, four_over_six, codes + r * (hidden / 2),
              block_scales + r * (hidden / 16), token_scales + r,
              dequant ? dequant + r * hidden : NULL);
  return 0;
}

/* Dequantized backward (NVFP4-RL blog section 3; humans& article section 2)
 * needs the BF16 value of exactly what was stored: the same candidate
 * formula applied to the stored code, block scale and token scale. */
int nvfp4_dequantize_ref(const uint8_t* codes, const uint8_t* block_scales,
                         const float* token_scales, int64_t rows,
                         int64_t hidden, uint16_t* out) {
  if (rows < 0 || hidden <= 0 || hidden % 16 != 0) return 2;
  if (rows == 0) return 0;
  if (!codes || !block_scales || !token_scales || !out) return 1;
  for (int64_t r = 0; r < rows; ++r) {
    float s = token_scales[r];
    for (int64_t i = 0; i < hidden; ++i) {
      uint8_t byte = codes[r * (hidden / 2) + i / 2];
      int nibble = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
      float e = oracle_e4m3_decode(block_scales[r * (hidden / 16) + i / 16]);
      float ge = oracle_e2m1_value(nibble & 7) * e;
      float c = ge * s;
      if (nibble & 8) c = -c;
      out[r * hidden + i] = oracle_bf16_rne(c);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 with Rollout-ResQ residual and 2:4 sparsity                        */
/* ------------------------------------------------------------------------ */

/* MXFP4 of one 32-element block of FP32 values: shared exponent k, nibbles
 * (sign << 3 | code) and the exact dequantized values +-g(q) * 2^k. */
static int mx_block(const float* x, uint8_t* nibble, float* dq) {
  float b = 0.0f;
  for (int i = 0; i < 32; ++i) {
    float a = fabsf(x[i]);
    if (a > b) b = a;
  }
  int k = oracle_e8m0_exponent(b);
  float down = ldexpf(1.0f, -k); /* exact power of two for k in [-127, 127] */
  for (int i = 0; i < 32; ++i) {
    float v = fabsf(x[i]) * down;
    int q = oracle_e2m1_code(v);
    int negative = signbit(x[i]) ? 1 : 0;
    nibble[i] = (uint8_t)((negative << 3) | q);
    float m = ldexpf(oracle_e2m1_value(q), k); /* exact */
    dq[i] = negative ? -m : m;
  }
  return k;
}

/* Rollout-ResQ (HiFloat4 page): the rollout projection becomes
 * Q(X)Q(W)^T + S(Q(dX))Q(W)^T with dX = X - Q(X), where Q(X) means the
 * dequantized value of the quantized X, and S keeps 2 of every 4
 * consecutive elements of the quantized residual.  The page does not say
 * which two; the two largest magnitudes are kept, ties to the lower index,
 * and the residual's block scale is taken over all 32 residuals before S
 * (S acts on Q(dX)). */
int mxfp4_resq_quantize_ref(const uint16_t* x, int64_t rows, int64_t hidden,
                            uint8_t* codes, uint8_t* scales,
                            uint8_t* res_codes, uint8_t* res_meta,
                            uint8_t* res_scales) {
  if (rows < 0 || hidden <= 0 || hidden % 32 != 0) return 2;
  if (rows == 0) return 0;
  if (!x || !codes || !scales || !res_codes || !res_meta || !res_scales)
    return 1;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t j = 0; j < hidden / 32; ++j) {
      float xb[32], dq[32], delta[32], rdq[32];
      uint8_t nib[32], rnib[32];
      for (int i = 0; i < 32; ++i)
        xb[i] = bf16_bits_to_float(x[r * hidden + j * 32 + i]);

      int k = mx_block(xb, nib, dq);
      for (int i = 0; i < 32; ++i) delta[i] = xb[i] - dq[i];
      int kr = mx_block(delta, rnib, rdq);

      scales[r * (hidden / 32) + j] = (uint8_t)(k + 127);
      res_scales[r * (hidden / 32) + j] = (uint8_t)(kr + 127);
      for (int i = 0; i < 32; i += 2)
        codes[r * (hidden / 2) + j * 16 + i / 2] =
            (uint8_t)(nib[i] | (nib[i + 1] << 4));

      for (int g = 0; g < 8; ++g) { /* groups of 4 consecutive elements */
        const uint8_t* grp = rnib + 4 * g;
        int i0 = -1, i1 = -1;
        /* first pick: largest magnitude, lowest index among equals */
        for (int i = 0; i < 4; ++i)
          if (i0 < 0 || (grp[i] & 7) > (grp[i0] & 7)) i0 = i;
        /* second pick: the same rule over the other three */
        for (int i = 0; i < 4; ++i)
          if (i != i0 && (i1 < 0 || (grp[i] & 7) > (grp[i1] & 7))) i1 = i;
        if (i1 < i0) { int tmp = i0; i0 = i1; i1 = tmp; }
        int64_t group = j * 8 + g; /* group index within the row */
        res_codes[r * (hidden / 4) + group] =
            (uint8_t)(grp[i0] | (grp[i1] << 4));
        uint8_t meta = (uint8_t)(i0 | (i1 << 2));
        uint8_t* mb = &res_meta[r * (hidden / 8) + group / 2];
        if (group % 2 == 0) *mb = (uint8_t)((*mb & 0xF0) | meta);
        else *mb = (uint8_t)((*mb & 0x0F) | (meta << 4));
      }
    }
  }
  return 0;
}

/* Rollout-ResQ-Dense (HiFloat4 page, the dense residual correction
 * Q(X)Q(W)^T + Q(dX)Q(W)^T that the sparse variant is compared with): the
 * same primary and residual quantization, with every residual code kept.
 * res_codes is [rows, hidden/2], packed like the primary codes. */
int mxfp4_resq_dense_quantize_ref(const uint16_t* x, int64_t rows, int64_t hidden,
                                  uint8_t* codes, uint8_t* scales,
                                  uint8_t* res_codes, uint8_t* res_scales) {
  if (rows < 0 || hidden <= 0 || hidden % 32 != 0) return 2;
  if (rows == 0) return 0;
  if (!x || !codes || !scales || !res_codes || !res_scales) return 1;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t j = 0; j < hidden / 32; ++j) {
      float xb[32], dq[32], delta[32], rdq[32];
      uint8_t nib[32], rnib[32];
      for (int i = 0; i < 32; ++i)
        xb[i] = bf16_bits_to_float(x[r * hidden + j * 32 + i]);
      int k = mx_block(xb, nib, dq);
      for (int i = 0; i < 32; ++i) delta[i] = xb[i] - dq[i];
      int kr = mx_block(delta, rnib, rdq);
      scales[r * (hidden / 32) + j] = (uint8_t)(k + 127);
      res_scales[r * (hidden / 32) + j] = (uint8_t)(kr + 127);
      for (int i = 0; i < 32; i += 2) {
        codes[r * (hidden / 2) + j * 16 + i / 2] = (uint8_t)(nib[i] | (nib[i + 1] << 4));
        res_codes[r * (hidden / 2) + j * 16 + i / 2] = (uint8_t)(rnib[i] | (rnib[i + 1] << 4));
      }
    }
  }
  return 0;
}

/* The dequantized value of an MX code under the E8M0 byte: +-g * 2^(byte -
 * 127), exact in FP32 for every code and byte. */
static float mx_value(uint8_t nibble, uint8_t scale_byte) {
  float m = ldexpf(oracle_e2m1_value(nibble & 7), (int)scale_byte - 127);
  return (nibble & 8) ? -m : m;
}

/* Reconstruction of the rollout input from what Rollout-ResQ stores (the
 * HiFloat4 page's Q(X) + S(Q(dX)), or + Q(dX) for the dense variant):
 *   residual 0: X_hat = DQ(Q(X))                      (primary only)
 *   residual 1: X_hat = DQ(Q(X)) + DQ(S(Q(dX)))        res_codes/res_meta
 *                                                      of the sparse call
 *   residual 2: X_hat = DQ(Q(X)) + DQ(Q(dX))           res_codes of the
 *                                                      dense call
 * Both terms are exact FP32 values; their sum is one FP32 addition.  The
 * two elements S drops in each group of four contribute +0.  With the
 * primary only there is no addition, so a negative zero stays -0. */
int mxfp4_resq_reconstruct_ref(const uint8_t* codes, const uint8_t* scales,
                               const uint8_t* res_codes, const uint8_t* res_meta,
                               const uint8_t* res_scales, int64_t rows, int64_t hidden,
                               int residual, float* out) {
  if (rows < 0 || hidden <= 0 || hidden % 32 != 0) return 2;
  if (residual < 0 || residual > 2) return 5;
  if (rows == 0) return 0;
  if (!codes || !scales || !out) return 1;
  if (residual != 0 && (!res_codes || !res_scales)) return 1;
  if (residual == 1 && !res_meta) return 1;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t i = 0; i < hidden; ++i) {
      int64_t blk = r * (hidden / 32) + i / 32;
      uint8_t byte = codes[r * (hidden / 2) + i / 2];
      float v = mx_value((i % 2) ? (byte >> 4) : (byte & 15), scales[blk]);
      float rv = 0.0f;
      if (residual == 2) {
        uint8_t rb = res_codes[r * (hidden / 2) + i / 2];
        rv = mx_value((i % 2) ? (rb >> 4) : (rb & 15), res_scales[blk]);
      } else if (residual == 1) {
        int64_t group = i / 4; /* within the row */
        uint8_t mb = res_meta[r * (hidden / 8) + group / 2];
        int meta = (group % 2) ? (mb >> 4) : (mb & 15);
        int i0 = meta & 3, i1 = meta >> 2, pos = (int)(i % 4);
        uint8_t kept = res_codes[r * (hidden / 4) + group];
        if (pos == i0) rv = mx_value(kept & 15, res_scales[blk]);
        else if (pos == i1) rv = mx_value(kept >> 4, res_scales[blk]);
      }
      out[r * hidden + i] = residual == 0 ? v : v + rv; /* primary only: DQ itself */
    }
  }
  return 0;
}

/* TRACE rollout-guided FP4 rounding ("TRACE FP4 RL -- Rollout-guided FP4
 * rounding", learnaivisually.com: the training engine rounds each captured
 * value, between its two neighbouring codewords, toward the codeword the
 * rollout engine chose, instead of to its own nearest one; the guarantee
 * holds with the rollout's codeword, the same rollout-side scale and the same
 * two candidates).
 *
 * Inputs: the training-side values x, the rollout's codes (guide) and the
 * rollout's block and token scales, used as the scale here too.  Per
 * element, with d = fl(e * s) and r = fl(1 / d) as in the quantizer:
 *   v = |x| * r;  lo = the largest E2M1 magnitude code with g <= v,
 *   hi = the smallest with g >= v (the same code when v is a grid value;
 *   v > 6 gives 7 for both; d == 0 gives 0 for both);
 *   with sigma the sign of x and G the guide's signed value, the code is hi
 *   when |sigma g(hi) - G| < |sigma g(lo) - G|, else lo.
 * The sign bit follows x, as in the quantizer; dequant (optional) is
 * BF16(+-((g * e) * s)).  Codes outside [off0, off1) of a ragged call are
 * not part of this entry point: every row is processed.
 *
 * guide_codes NULL: the training side's own round-to-nearest under the same
 * rollout-side scale, the rounding the page sets guided rounding against
 * (its worked example and its count of mismatches on adjacent codewords):
 * the code is E2M1(v), the quantizer's rounding of the same v. */
int nvfp4_quantize_guided_ref(const uint16_t* x, int64_t rows, int64_t hidden,
                              const uint8_t* guide_codes, const uint8_t* block_scales,
                              const float* token_scales, uint8_t* codes,
                              uint16_t* dequant) {
  if (rows < 0 || hidden <= 0 || hidden % 16 != 0) return 2;
  if (rows == 0) return 0;
  if (!x || !block_scales || !token_scales || !codes) return 1;
  for (int64_t r = 0; r < rows; ++r) {
    float s = token_scales[r];
    for (int64_t i = 0; i < hidden; ++i) {
      float e = oracle_e4m3_decode(block_scales[r * (hidden / 16) + i / 16]);
      float d = e * s;
      float xi = bf16_bits_to_float(x[r * hidden + i]);
      int neg = signbit(xi) ? 1 : 0;
      int lo = 0, hi = 0, nearest = 0;
      if (d != 0.0f) {
        float rr = 1.0f / d;
        float v = fabsf(xi) * rr;
        lo = 0;
        for (int q = 1; q < 8; ++q)
          if (oracle_e2m1_value(q) <= v) lo = q;
        hi = lo;
        if (oracle_e2m1_value(lo) < v && lo < 7) hi = lo + 1;
        nearest = oracle_e2m1_code(v);
      }
      int q = nearest;
      if (guide_codes) {
        uint8_t gb = guide_codes[r * (hidden / 2) + i / 2];
        int gn = (i % 2) ? (gb >> 4) : (gb & 15);
        double G =
            (gn & 8) ? -(double)oracle_e2m1_value(gn & 7) : (double)oracle_e2m1_value(gn & 7);
        double sigma = neg ? -1.0 : 1.0;
        double dlo = fabs(sigma * oracle_e2m1_value(lo) - G);
        double dhi = fabs(sigma * oracle_e2m1_value(hi) - G);
        q = (dhi < dlo) ? hi : lo;
      }
      uint8_t nib = (uint8_t)((neg << 3) | q);
      uint8_t* cb = &codes[r * (hidden / 2) + i / 2];
      if (i % 2 == 0) *cb = (uint8_t)((*cb & 0xF0) | nib);
      else *cb = (uint8_t)((*cb & 0x0F) | (nib << 4));
      if (dequant) {
        float ge = oracle_e2m1_value(q) * e;
        float c = ge * s;
        dequant[r * hidden + i] = oracle_bf16_rne(neg ? -c : c);
      }
    }
  }
  return 0;
}

/* The naive NVFP4 the pages contrast with per-token scaling (humans&
 * article section 1; NVFP4-RL blog section 2): one FP32 scale for the whole
 * activation tensor, s = amax_tensor / 1536 (4/6 on) or / 2688, then the
 * same block path in every row.  A row's outputs then depend on the other
 * rows of the tensor (the batch dependency the pages warn about). */
int nvfp4_quantize_global_ref(const uint16_t* x, int64_t rows, int64_t hidden,
                              int four_over_six, uint8_t* codes, uint8_t* block_scales,
                              float* tensor_scale, uint16_t* dequant) {
  if (rows < 0 || hidden <= 0 || hidden % 16 != 0) return 2;
  if (four_over_six < 0 || four_over_six > 2) return 5;
  if (rows == 0) return 0;
  if (!x || !codes || !block_scales || !tensor_scale) return 1;
  float amax = 0.0f;
  for (int64_t i = 0; i < rows * hidden; ++i) {
    float a = fabsf(bf16_bits_to_float(x[i]));
    if (a > amax) amax = a;
  }
  float s = amax / (four_over_six ? 1536.0f : 2688.0f);
  *tensor_scale = s;
  for (int64_t r = 0; r < rows; ++r)
    nvfp4_row_with_scale(x + r * hidden, hidden, four_over_six, s, codes + r * (hidden / 2),
                         block_scales + r * (hidden / 16), dequant ? dequant + r * hidden : NULL);
  return 0;
}
