/*
 * gen.c -- seeded synthetic inputs for the quantizer's workloads.
 *
 * Holds no quantizer arithmetic: it only draws random FP32 values.  Every
 * row has its own random stream (xoshiro256** seeded through splitmix64
 * from the workload seed and the row index), so any subset of rows can be
 * regenerated on its own and the result does not depend on the number of
 * threads.
 *
 *   splitmix64, xoshiro256**: Blackman & Vigna, "Scrambled linear
 *     pseudorandom number generators" (2018 reference code description).
 *   Normal variates: Box-Muller in double.
 *   Student-t(3): Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3).
 *   LogNormal(mu, sigma): exp(mu + sigma * Z).
 *
 * Draw order within a row: the row gain (if any), then per element its
 * value (one normal, or four normals for Student-t), then its outlier
 * uniform (if element outliers are on).  Values are returned as FP32.
 */
#include <math.h>
#include <stdint.h>

typedef struct { uint64_t s[4]; int have_spare; double spare; } stream_t;

static uint64_t splitmix64(uint64_t* x) {
  uint64_t z = (*x += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint64_t rotl(uint64_t x, int k) { return (x << k) | (x >> (64 - k)); }

static uint64_t next_u64(stream_t* st) {
  uint64_t* s = st->s;
  uint64_t result = rotl(s[1] * 5, 7) * 9;
  uint64_t t = s[1] << 17;
  s[2] ^= s[0];
  s[3] ^= s[1];
  s[1] ^= s[2];
  s[0] ^= s[3];
  s[2] ^= t;
  s[3] = rotl(s[3], 45);
  return result;
}

static void stream_init(stream_t* st, uint64_t seed, uint64_t index) {
  uint64_t x = seed * 0xD1B54A32D192ED03ull ^ (index + 0x632BE59BD9B4E019ull);
  for (int i = 0; i < 4; ++i) st->s[i] = splitmix64(&x);
  st->have_spare = 0;
  st->spare = 0.0;
}

/* uniform in [0, 1) with 53 random bits */
static double uniform(stream_t* st) {
  return (double)(next_u64(st) >> 11) * (1.0 / 9007199254740992.0);
}

static double normal(stream_t* st) {
  if (st->have_spare) {
    st->have_spare = 0;
    return st->spare;
  }
  double u1 = uniform(st), u2 = uniform(st);
  if (u1 < 1e-300) u1 = 1e-300;
  double rad = sqrt(-2.0 * log(u1));
  double ang = 6.283185307179586476925286766559 * u2;
  st->spare = rad * sin(ang);
  st->have_spare = 1;
  return rad * cos(ang);
}

static double student_t3(stream_t* st) {
  double z = normal(st);
  double a = normal(st), b = normal(st), c = normal(st);
  return z / sqrt((a * a + b * b + c * c) / 3.0);
}

/* dist: 0 = normal, 1 = Student-t with 3 degrees of freedom.
 * value = scale * draw * col_mult[col] * row_gain, and with probability
 * elem_p the element is further multiplied by elem_mult. */
void wl_fill_rows(uint64_t seed, int64_t row0, int64_t nrows, int64_t hidden,
                  int dist, double scale, double row_gain_sigma,
                  double elem_p, double elem_mult, const float* col_mult,
                  float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    stream_t st;
    stream_init(&st, seed, (uint64_t)(row0 + r));
    double gain = 1.0;
    if (row_gain_sigma > 0.0) gain = exp(row_gain_sigma * normal(&st));
    float* o = out + r * hidden;
    for (int64_t i = 0; i < hidden; ++i) {
      double v = dist == 1 ? student_t3(&st) : normal(&st);
      v *= scale * gain;
      if (col_mult) v *= (double)col_mult[i];
      if (elem_p > 0.0 && uniform(&st) < elem_p) v *= elem_mult;
      o[i] = (float)v;
    }
  }
}

/* Seeded Fisher-Yates: the first `count` entries of a random permutation
 * of 0..n-1 (distinct channel indices). */
void wl_pick_channels(uint64_t seed, int64_t n, int64_t count, int64_t* out,
                      int64_t* scratch) {
  stream_t st;
  stream_init(&st, seed, 0xC0FFEEull);
  for (int64_t i = 0; i < n; ++i) scratch[i] = i;
  for (int64_t i = 0; i < count; ++i) {
    int64_t j = i + (int64_t)(uniform(&st) * (double)(n - i));
    int64_t t = scratch[i];
    scratch[i] = scratch[j];
    scratch[j] = t;
    out[i] = scratch[i];
  }
}

/* Routing: each of n_draws routed rows picks one of n_bins experts from the
 * top bits of a 64-bit draw (n_bins a power of two); counts per expert. */
void wl_route_counts(uint64_t seed, int64_t n_draws, int log2_bins,
                     int64_t* counts) {
  stream_t st;
  stream_init(&st, seed, 0x5EEDull);
  for (int64_t b = 0; b < ((int64_t)1 << log2_bins); ++b) counts[b] = 0;
  for (int64_t i = 0; i < n_draws; ++i)
    counts[next_u64(&st) >> (64 - log2_bins)] += 1;
}
