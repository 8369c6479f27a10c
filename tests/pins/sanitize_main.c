/* Drives every entry point of the CPU oracle (oracle/fp4_oracle.c) on
 * seeded finite inputs -- zeros, signed zeros, BF16 subnormals, the largest
 * finite BF16, grid points and midpoints, heavy tails -- over row lengths
 * from one block to a long row, plus the rejected-argument paths, so that
 * a build with AddressSanitizer and UndefinedBehaviorSanitizer sees every
 * buffer index and conversion the oracle performs.  Prints "sanitize ok"
 * and returns 0 when every call returns the expected status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp4_oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) { /* xorshift64* */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return state * 0x2545F4914F6CDD1Dull;
}

static uint16_t bf16_of(float f) { return oracle_bf16_rne(f); }

/* one row of `hidden` BF16 values of kind k */
static void fill_row(uint16_t* r, int64_t hidden, int k) {
  for (int64_t i = 0; i < hidden; ++i) {
    uint64_t u = next();
    float f;
    switch (k % 8) {
      case 0: f = 0.0f; break;
      case 1: f = (i & 1) ? -0.0f : 0.0f; break;
      case 2: r[i] = (uint16_t)((u & 0x7F) | ((u >> 8) & 1) << 15); continue; /* subnormals */
      case 3: r[i] = (uint16_t)(0x7F7F | ((u & 1) << 15)); continue;         /* largest */
      case 4: {
        static const float g[] = {0, .25f, .5f, .75f, 1, 1.25f, 1.5f, 1.75f, 2, 2.5f, 3, 3.5f, 4, 5, 6};
        f = g[u % 15] * ldexpf(1.0f, (int)((u >> 8) % 40) - 20) * ((u >> 16) & 1 ? -1.0f : 1.0f);
        break;
      }
      case 5: f = (float)((int64_t)(u % 2001) - 1000) * 1e-3f; break;
      case 6: { /* heavy tail: ratio of uniforms */
        double a = (double)(u >> 11) / 9007199254740992.0 - 0.5;
        double b = (double)(next() >> 11) / 9007199254740992.0 + 1e-6;
        f = (float)(a / b);
        break;
      }
      default: r[i] = (uint16_t)(u % 0x7F80 | ((u >> 20) & 1) << 15); continue; /* any finite */
    }
    r[i] = bf16_of(f);
  }
}

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static void run_shape(int64_t rows, int64_t hidden) {
  const int64_t n = rows * hidden;
  uint16_t* x = malloc(n * sizeof *x);
  uint8_t* codes = malloc(n / 2);
  uint8_t* scales = malloc(n / 16);
  float* ts = malloc(rows * sizeof *ts);
  uint16_t* dq = malloc(n * sizeof *dq);
  uint16_t* back = malloc(n * sizeof *back);
  uint8_t* gcodes = malloc(n / 2);
  for (int64_t r = 0; r < rows; ++r) fill_row(x + r * hidden, hidden, (int)(r + hidden));

  for (int fos = 0; fos <= 2; ++fos) {
    EXPECT(nvfp4_quantize_ref(x, rows, hidden, NULL, 0, fos, codes, scales, ts, dq) == 0);
    EXPECT(nvfp4_quantize_ref(x, rows, hidden, NULL, 0, fos, codes, scales, ts, NULL) == 0);
    EXPECT(nvfp4_dequantize_ref(codes, scales, ts, rows, hidden, back) == 0);
    EXPECT(nvfp4_quantize_guided_ref(x, rows, hidden, codes, scales, ts, gcodes, back) == 0);
    for (int64_t i = 0; i < n / 2; ++i) gcodes[i] = (uint8_t)next();
    EXPECT(nvfp4_quantize_guided_ref(x, rows, hidden, gcodes, scales, ts, codes, NULL) == 0);
    EXPECT(nvfp4_quantize_guided_ref(x, rows, hidden, NULL, scales, ts, codes, back) == 0);
    float s1;
    EXPECT(nvfp4_quantize_global_ref(x, rows, hidden, fos, codes, scales, &s1, dq) == 0);
  }
  /* a ragged group range inside the rows */
  int64_t offs[4] = {rows / 3, rows / 3, rows / 2 + 1 > rows ? rows : rows / 2 + 1, rows};
  EXPECT(nvfp4_quantize_ref(x, rows, hidden, offs, 3, 1, codes, scales, ts, dq) == 0);

  if (hidden % 32 == 0) {
    uint8_t* c = malloc(n / 2);
    uint8_t* sc = malloc(n / 32);
    uint8_t* rc = malloc(n / 4);
    uint8_t* rm = malloc(n / 8);
    uint8_t* rs = malloc(n / 32);
    uint8_t* dc = malloc(n / 2);    /* dense: primary codes and scales, */
    uint8_t* dsc = malloc(n / 32);
    uint8_t* drc = malloc(n / 2);   /* every residual code, residual scales */
    uint8_t* drs = malloc(n / 32);
    float* xh = malloc(n * sizeof *xh);
    EXPECT(mxfp4_resq_quantize_ref(x, rows, hidden, c, sc, rc, rm, rs) == 0);
    EXPECT(mxfp4_resq_dense_quantize_ref(x, rows, hidden, dc, dsc, drc, drs) == 0);
    EXPECT(mxfp4_resq_reconstruct_ref(c, sc, NULL, NULL, NULL, rows, hidden, 0, xh) == 0);
    EXPECT(mxfp4_resq_reconstruct_ref(c, sc, rc, rm, rs, rows, hidden, 1, xh) == 0);
    EXPECT(mxfp4_resq_reconstruct_ref(dc, dsc, drc, NULL, drs, rows, hidden, 2, xh) == 0);
    free(c); free(sc); free(rc); free(rm); free(rs); free(dc); free(dsc); free(drc); free(drs);
    free(xh);
  }
  free(x); free(codes); free(scales); free(ts); free(dq); free(back); free(gcodes);
}

int main(void) {
  /* primitives over wide ranges of their inputs */
  for (uint32_t b = 0; b < 0x7F800000u; b += 0x00001001u) {
    float f;
    memcpy(&f, &b, 4);
    (void)oracle_e2m1_code(f);
    (void)oracle_e4m3_encode(f);
    (void)oracle_bf16_rne(f);
    (void)oracle_bf16_rne(-f);
    (void)oracle_e8m0_exponent(f);
    (void)oracle_fp16_rne((double)f);
  }
  for (int q = 0; q < 8; ++q) (void)oracle_e2m1_value(q);
  for (int b = 0; b < 256; ++b) (void)oracle_e4m3_decode((uint8_t)b);

  /* single blocks under extreme token scales */
  float x16[16];
  oracle_nvfp4_block_t blk;
  const float svals[] = {0.0f, 1e-45f, 1e-38f, 1e-30f, 1.0f / 1536, 1.0f, 1e20f, 2e38f};
  for (int k = 0; k < 64; ++k) {
    uint16_t r[16];
    fill_row(r, 16, k);
    for (int i = 0; i < 16; ++i) {
      uint32_t w = (uint32_t)r[i] << 16;
      memcpy(&x16[i], &w, 4);
    }
    for (size_t j = 0; j < sizeof svals / sizeof svals[0]; ++j)
      for (int fos = 0; fos <= 2; ++fos) oracle_nvfp4_block(x16, svals[j], fos, &blk);
  }

  const int64_t shapes[][2] = {{3, 16}, {5, 32}, {9, 48}, {4, 2048}, {2, 7168}, {1, 33024}};
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) run_shape(shapes[i][0], shapes[i][1]);

  /* rejected arguments */
  uint16_t x[64] = {0};
  uint8_t c[32], s[4];
  float t[2];
  EXPECT(nvfp4_quantize_ref(x, 2, 24, NULL, 0, 1, c, s, t, NULL) != 0);
  EXPECT(nvfp4_quantize_ref(x, 2, 32, NULL, 0, 3, c, s, t, NULL) != 0);
  EXPECT(nvfp4_quantize_ref(NULL, 2, 32, NULL, 0, 1, c, s, t, NULL) != 0);
  EXPECT(mxfp4_resq_quantize_ref(x, 2, 16, c, s, c, c, s) != 0);
  EXPECT(nvfp4_quantize_ref(x, 0, 32, NULL, 0, 1, NULL, NULL, NULL, NULL) == 0);

  if (failures) return 1;
  puts("sanitize ok");
  return 0;
}
