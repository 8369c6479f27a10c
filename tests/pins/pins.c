/*
 * pins.c -- exhaustive checks of the CPU oracle's number-format primitives
 * against independent brute-force definitions evaluated exactly in double.
 *
 * Nothing here includes or links the oracle: the test passes the oracle's
 * primitive in as a function pointer, and this file decides what the right
 * answer is from first principles (nearest representable value, ties to the
 * even code / even mantissa).  Each function walks a range of binary32 bit
 * patterns and returns the number of disagreements, storing the first
 * offending pattern.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef int (*e2m1_code_fn)(float);
typedef uint8_t (*e4m3_encode_fn)(float);
typedef uint16_t (*bf16_fn)(float);
typedef int (*e8m0_fn)(float);

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* E2M1 magnitudes, listed as sign-less 1.m x 2^e values of a 2-bit-exponent,
 * 1-bit-mantissa float with bias 1 (code 1 is the subnormal 0.5). */
static double e2m1_grid(int q) {
  int ex = q >> 1, man = q & 1;
  return ex == 0 ? man * 0.5 : ldexp(1.0 + 0.5 * man, ex - 1);
}

/* Nearest grid value to a (exact in double), ties to the even code;
 * values past the top saturate. */
static int e2m1_nearest(const double* grid, double a) {
  int best = 0;
  double bestd = fabs(a - grid[0]);
  for (int q = 1; q < 8; ++q) {
    double d = fabs(a - grid[q]);
    if (d < bestd || (d == bestd && (q % 2 == 0) && (best % 2 != 0))) {
      best = q;
      bestd = d;
    }
  }
  return best;
}

/* The range is split into chunks walked by OpenMP threads; the count of
 * disagreements and the lowest offending pattern do not depend on it. */
#define CHUNK (1u << 20)

int64_t pin_e2m1(e2m1_code_fn f, uint32_t lo, uint32_t hi, uint32_t* first) {
  double grid[8];
  for (int q = 0; q < 8; ++q) grid[q] = e2m1_grid(q);
  int64_t bad = 0;
  uint32_t first_bad = 0xFFFFFFFFu;
  int64_t nchunks = ((int64_t)hi - lo) / CHUNK + 1;
#pragma omp parallel for schedule(dynamic) reduction(+ : bad) reduction(min : first_bad)
  for (int64_t c = 0; c < nchunks; ++c) {
    uint64_t a0 = (uint64_t)lo + (uint64_t)c * CHUNK;
    uint64_t a1 = a0 + CHUNK - 1 > hi ? hi : a0 + CHUNK - 1;
    for (uint64_t u = a0; u <= a1; ++u) {
      float a = from_bits((uint32_t)u);
      if (f(a) != e2m1_nearest(grid, (double)a)) {
        if ((uint32_t)u < first_bad) first_bad = (uint32_t)u;
        ++bad;
      }
    }
  }
  if (bad) *first = first_bad;
  return bad;
}

/* All 127 non-negative finite E4M3FN values in increasing order, built from
 * the format's fields as 2^(E-7) * (1 + m/8) (normal) or 2^-6 * m/8
 * (subnormal); byte pattern == index. */
static double e4m3_table[127];
static void build_e4m3_table(void) {
  for (int byte = 0; byte < 127; ++byte) {
    int E = byte >> 3, m = byte & 7;
    e4m3_table[byte] = E == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, E - 7);
  }
}

/* Walk the patterns in increasing order with a moving bracket
 * table[j] <= a < table[j+1]; nearest with ties to the even byte,
 * saturation above 448. */
int64_t pin_e4m3(e4m3_encode_fn f, uint32_t lo, uint32_t hi, uint32_t* first) {
  build_e4m3_table();
  int64_t bad = 0;
  uint32_t first_bad = 0xFFFFFFFFu;
  int64_t nchunks = ((int64_t)hi - lo) / CHUNK + 1;
#pragma omp parallel for schedule(dynamic) reduction(+ : bad) reduction(min : first_bad)
  for (int64_t c = 0; c < nchunks; ++c) {
    uint64_t a0 = (uint64_t)lo + (uint64_t)c * CHUNK;
    uint64_t a1 = a0 + CHUNK - 1 > hi ? hi : a0 + CHUNK - 1;
    int j = 0;
    for (uint64_t u = a0; u <= a1; ++u) {
      double a = (double)from_bits((uint32_t)u);
      while (j < 126 && e4m3_table[j + 1] <= a) ++j;
      int want;
      if (j == 126) {
        want = 126; /* at or past 448 */
      } else {
        double dl = a - e4m3_table[j], dh = e4m3_table[j + 1] - a;
        if (dl < dh) want = j;
        else if (dh < dl) want = j + 1;
        else want = (j % 2 == 0) ? j : j + 1;
      }
      if (f((float)a) != want) {
        if ((uint32_t)u < first_bad) first_bad = (uint32_t)u;
        ++bad;
      }
    }
  }
  if (bad) *first = first_bad;
  return bad;
}

/* Nearest BF16 to a finite float: the two BF16 neighbours are the pattern
 * truncated to its top 16 bits and the next one up in magnitude; compare
 * distances exactly in double, ties to the even pattern.  Overflow past
 * the largest finite BF16 is decided the same way against 2^128 (the
 * infinity pattern 0x7F80 is the "next" value). */
int64_t pin_bf16(bf16_fn f, uint32_t lo, uint32_t hi, uint32_t* first) {
  int64_t bad = 0;
  uint32_t first_bad = 0xFFFFFFFFu;
  int64_t nchunks = ((int64_t)hi - lo) / CHUNK + 1;
#pragma omp parallel for schedule(dynamic) reduction(+ : bad) reduction(min : first_bad)
  for (int64_t c = 0; c < nchunks; ++c) {
    uint64_t a0 = (uint64_t)lo + (uint64_t)c * CHUNK;
    uint64_t a1 = a0 + CHUNK - 1 > hi ? hi : a0 + CHUNK - 1;
    for (uint64_t u = a0; u <= a1; ++u) {
      uint32_t bits = (uint32_t)u;
      if ((bits & 0x7F800000u) == 0x7F800000u) continue; /* Inf/NaN */
      float x = from_bits(bits);
      uint32_t t = bits & 0xFFFF0000u;
      double lo_v = (double)from_bits(t);
      uint32_t up = t + 0x10000u;
      double hi_v = ((up & 0x7F800000u) == 0x7F800000u)
                        ? copysign(ldexp(1.0, 128), lo_v)
                        : (double)from_bits(up);
      double dl = fabs((double)x - lo_v), dh = fabs(hi_v - (double)x);
      uint16_t want;
      if (dl < dh) want = (uint16_t)(t >> 16);
      else if (dh < dl) want = (uint16_t)(up >> 16);
      else want = ((t >> 16) & 1u) ? (uint16_t)(up >> 16) : (uint16_t)(t >> 16);
      if (f(x) != want) {
        if (bits < first_bad) first_bad = bits;
        ++bad;
      }
    }
  }
  if (bad) *first = first_bad;
  return bad;
}

/* E8M0 exponent k of a block max b > 0: k = floor(log2 b) - 2, so that
 * 4 * 2^k <= b < 8 * 2^k when unclamped; checked as that inequality. */
int64_t pin_e8m0(e8m0_fn f, uint32_t lo, uint32_t hi, uint32_t step,
                 uint32_t* first) {
  int64_t bad = 0;
  for (uint64_t u = lo; u <= hi; u += step) {
    float b = from_bits((uint32_t)u);
    if (!(b > 0.0f) || isinf(b)) continue;
    int k = f(b);
    int ok;
    double lo_b = ldexp(4.0, k), hi_b = ldexp(8.0, k);
    if (k == -127) ok = (double)b < ldexp(8.0, -127);
    else if (k == 127) ok = (double)b >= ldexp(4.0, 127);
    else ok = lo_b <= (double)b && (double)b < hi_b;
    if (!ok) {
      if (!bad) *first = (uint32_t)u;
      ++bad;
    }
  }
  return bad;
}

/* ---- comparison of GPU conversion results with the oracle's primitives --
 * Pairs: result i covers the binary32 patterns (lo + 2i) ^ flip (first /
 * low part) and (lo + 2i + 1) ^ flip (second / high part).  NaN patterns
 * are skipped.  Returns the number of mismatching results and the index of
 * the first one. */

static int is_nan_bits(uint32_t u) { return (u & 0x7FFFFFFFu) > 0x7F800000u; }

int64_t cmp_fp4(e2m1_code_fn f, uint32_t lo, uint32_t flip, uint64_t n,
                const uint8_t* got, uint64_t* first) {
  int64_t bad = 0;
  uint64_t first_bad = UINT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : first_bad)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    int ok = 1;
    for (int h = 0; h < 2; ++h) {
      uint32_t u = (uint32_t)(lo + 2 * (uint64_t)i + h) ^ flip;
      if (is_nan_bits(u)) continue;
      float v = from_bits(u);
      int want = f(fabsf(v)) | ((u >> 31) << 3);
      int have = (got[i] >> (4 * h)) & 15;
      if (want != have) ok = 0;
    }
    if (!ok) {
      ++bad;
      if ((uint64_t)i < first_bad) first_bad = (uint64_t)i;
    }
  }
  *first = first_bad;
  return bad;
}

/* got[i]: two codes of the patterns (2i) << 13 (low nibble) and
 * (2i + 1) << 13 from an encode that divides by 2^k; the oracle's code of
 * |a| * 2^-k (the product rounded to binary32, as the oracle forms it) with
 * the sign bit kept.  Only inputs the MX kernels can feed it are compared:
 * finite |a| < 2^(k+3), the bound every element of a block whose shared
 * exponent is k satisfies. */
int64_t cmp_fp4_scaled(e2m1_code_fn f, int k, uint64_t n, const uint8_t* got, uint64_t* first) {
  int64_t bad = 0;
  uint64_t first_bad = UINT64_MAX;
  const float down = ldexpf(1.0f, -k);
  const double bound = ldexp(1.0, k + 3);
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : first_bad)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    int ok = 1;
    for (int h = 0; h < 2; ++h) {
      uint32_t u = (uint32_t)(2 * (uint64_t)i + h) << 13;
      float a = from_bits(u);
      if (!(fabs((double)a) < bound)) continue; /* also skips Inf and NaN */
      int want = f(fabsf(a) * down) | ((u >> 31) << 3);
      if (((got[i] >> (4 * h)) & 15) != want) ok = 0;
    }
    if (!ok) {
      ++bad;
      if ((uint64_t)i < first_bad) first_bad = (uint64_t)i;
    }
  }
  *first = first_bad;
  return bad;
}

/* E2M1 code of the largest grid point at or below a >= 0 (7 above 6): the
 * number of nonzero grid points 0.5, 1, 1.5, 2, 3, 4, 6 that are <= a. */
static int e2m1_floor_code(float a) {
  static const float g[7] = {0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  int q = 0;
  for (int k = 0; k < 7; ++k) q += a >= g[k];
  return q;
}

/* got[i]: two floor codes, of patterns lo + 2i (low nibble) and lo + 2i + 1
 * (non-negative patterns; NaN patterns skipped). */
int64_t cmp_fp4_floor(uint32_t lo, uint64_t n, const uint8_t* got, uint64_t* first) {
  int64_t bad = 0;
  uint64_t first_bad = UINT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : first_bad)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    int ok = 1;
    for (int h = 0; h < 2; ++h) {
      uint32_t u = (uint32_t)(lo + 2 * (uint64_t)i + h);
      if (is_nan_bits(u)) continue;
      if (((got[i] >> (4 * h)) & 15) != e2m1_floor_code(from_bits(u))) ok = 0;
    }
    if (!ok) {
      ++bad;
      if ((uint64_t)i < first_bad) first_bad = (uint64_t)i;
    }
  }
  *first = first_bad;
  return bad;
}

/* got[i]: a reciprocal of the pattern lo + i; it must equal the IEEE
 * binary32 quotient 1 / d, which C's division gives. */
int64_t cmp_recip(uint32_t lo, uint64_t n, const float* got, uint64_t* first) {
  int64_t bad = 0;
  uint64_t first_bad = UINT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : first_bad)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    float want = 1.0f / from_bits((uint32_t)(lo + (uint64_t)i));
    if (memcmp(&want, &got[i], 4) != 0) {
      ++bad;
      if ((uint64_t)i < first_bad) first_bad = (uint64_t)i;
    }
  }
  *first = first_bad;
  return bad;
}

int64_t cmp_bf16(bf16_fn f, uint32_t lo, uint64_t n, const uint32_t* got,
                 uint64_t* first) {
  int64_t bad = 0;
  uint64_t first_bad = UINT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : first_bad)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    int ok = 1;
    for (int h = 0; h < 2; ++h) {
      uint32_t u = (uint32_t)(lo + 2 * (uint64_t)i + h);
      if (is_nan_bits(u)) continue;
      if ((uint32_t)f(from_bits(u)) != ((got[i] >> (16 * h)) & 0xFFFFu)) ok = 0;
    }
    if (!ok) {
      ++bad;
      if ((uint64_t)i < first_bad) first_bad = (uint64_t)i;
    }
  }
  *first = first_bad;
  return bad;
}

int64_t cmp_fp8(e4m3_encode_fn f, uint32_t lo, uint64_t n, const uint16_t* got,
                uint64_t* first) {
  int64_t bad = 0;
  uint64_t first_bad = UINT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : first_bad)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    int ok = 1;
    for (int h = 0; h < 2; ++h) {
      uint32_t u = (uint32_t)(lo + 2 * (uint64_t)i + h);
      if (is_nan_bits(u)) continue;
      if ((uint32_t)f(from_bits(u)) != ((uint32_t)(got[i] >> (8 * h)) & 0xFFu)) ok = 0;
    }
    if (!ok) {
      ++bad;
      if ((uint64_t)i < first_bad) first_bad = (uint64_t)i;
    }
  }
  *first = first_bad;
  return bad;
}

/* ---- IEEE binary16 rounding --------------------------------------------- */

typedef double (*fp16_fn)(double);

/* Value of a positive binary16 pattern (0x0000 .. 0x7C00 = infinity) from
 * its fields: exponent field 0 is subnormal (m * 2^-24), else
 * (1024 + m) * 2^(field - 25). */
static double fp16_value(int pattern) {
  int field = pattern >> 10, m = pattern & 1023;
  if (field == 31) return INFINITY;
  return field == 0 ? ldexp((double)m, -24) : ldexp(1024.0 + m, field - 25);
}

/* Every binary32 pattern in [lo, hi] (non-negative values): the oracle's
 * rounding must give the nearest binary16 value, found by binary search in
 * the table of all non-negative patterns, ties to the even pattern; past
 * the largest finite value the candidate above is infinity. */
int64_t pin_fp16(fp16_fn f, uint32_t lo, uint32_t hi, uint32_t* first) {
  static double table[0x7C01];
  for (int p = 0; p <= 0x7C00; ++p) table[p] = fp16_value(p);
  int64_t bad = 0;
  uint32_t first_bad = 0xFFFFFFFFu;
  int64_t nchunks = ((int64_t)hi - lo) / CHUNK + 1;
#pragma omp parallel for schedule(dynamic) reduction(+ : bad) reduction(min : first_bad)
  for (int64_t c = 0; c < nchunks; ++c) {
    uint64_t a0 = (uint64_t)lo + (uint64_t)c * CHUNK;
    uint64_t a1 = a0 + CHUNK - 1 > hi ? hi : a0 + CHUNK - 1;
    for (uint64_t u = a0; u <= a1; ++u) {
      double a = (double)from_bits((uint32_t)u);
      double want;
      if (a >= table[0x7BFF] + 16.0) {  /* 65520 and above: infinity */
        want = INFINITY;
      } else {
        int l = 0, h = 0x7BFF;  /* largest pattern with value <= a */
        while (l < h) {
          int mid = (l + h + 1) / 2;
          if (table[mid] <= a) l = mid; else h = mid - 1;
        }
        if (table[l] == a || l == 0x7BFF) {
          want = table[l];
        } else {
          double dl = a - table[l], dh = table[l + 1] - a;
          want = (dl < dh || (dl == dh && (l % 2 == 0))) ? table[l] : table[l + 1];
        }
      }
      double got = f(a);
      if (!(got == want)) {
        bad++;
        if (u < first_bad) first_bad = (uint32_t)u;
      }
    }
  }
  *first = first_bad;
  return bad;
}
