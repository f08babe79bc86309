/*
 * Seeded, counter-based synthetic input generator.
 *
 * Serves both the oracle and the HIP library's tests and benchmark: it writes
 * plain fp32 (or fp64) host arrays, and the caller rounds them to bf16/fp16
 * with a library cast.  It holds none of the FP8 method's arithmetic.
 *
 * Random bits: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  Draw i of stream
 * (seed, stream) is the i-th output of SplitMix64 started from the state
 * seed * 2^32 + stream, computed directly from i (counter-based), so any
 * element can be produced on its own and in any order.
 * Normals: Box-Muller transform in fp64.
 */
#include <math.h>
#include <stdint.h>

#define SYN_API __attribute__((visibility("default")))

static const uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* The i-th (0-based) SplitMix64 output from the given initial state. */
static uint64_t draw(uint64_t state0, uint64_t i) { return mix64(state0 + (i + 1) * GAMMA); }

static uint64_t state_of(uint64_t seed, uint64_t stream) { return (seed << 32) + stream; }

/* uniform in [0, 1) with 53 random bits */
static double u01(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }
/* uniform in (0, 1] */
static double u01_open0(uint64_t r) { return (double)((r >> 11) + 1) * 0x1.0p-53; }

SYN_API void syn_u64(uint64_t seed, uint64_t stream, int64_t start, int64_t n, uint64_t* out) {
  uint64_t s0 = state_of(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = draw(s0, (uint64_t)(start + i));
}

SYN_API void syn_uniform_f64(uint64_t seed, uint64_t stream, int64_t start, int64_t n,
                             double* out) {
  uint64_t s0 = state_of(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = u01(draw(s0, (uint64_t)(start + i)));
}

/*
 * out[i] = sigma * z_i * (outlier_i ? outlier_mult : 1), z_i ~ N(0,1) from
 * draws 3i and 3i+1 (Box-Muller, cosine branch); element i is an outlier when
 * draw 3i+2, as a uniform in [0,1), is below outlier_p.
 */
SYN_API void syn_normal_f32(uint64_t seed, uint64_t stream, int64_t start, int64_t n,
                            double sigma, double outlier_p, double outlier_mult, float* out) {
  uint64_t s0 = state_of(seed, stream);
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t e = (uint64_t)(start + i);
    double u1 = u01_open0(draw(s0, 3 * e));
    double u2 = u01(draw(s0, 3 * e + 1));
    double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
    double v = sigma * z;
    if (outlier_p > 0.0 && u01(draw(s0, 3 * e + 2)) < outlier_p) v *= outlier_mult;
    out[i] = (float)v;
  }
}

/* Random sign times a magnitude 10^U(lo10, hi10) (log-uniform), from draws 2i
 * (exponent) and 2i+1 (sign). */
SYN_API void syn_logmag_f32(uint64_t seed, uint64_t stream, int64_t start, int64_t n,
                            double lo10, double hi10, float* out) {
  uint64_t s0 = state_of(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t e = (uint64_t)(start + i);
    double u = u01(draw(s0, 2 * e));
    double mag = pow(10.0, lo10 + (hi10 - lo10) * u);
    int neg = (int)(draw(s0, 2 * e + 1) >> 63);
    out[i] = (float)(neg ? -mag : mag);
  }
}
