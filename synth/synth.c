/*
 * Seeded synthetic inputs for the gated delta-rule scan workloads.
 *
 * This file only draws random numbers and shapes their distribution; it holds
 * none of the scan's arithmetic.  It serves both the double-precision oracle
 * and the GPU library's tests and benchmark, so both sides see identical bits.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used counter-style: draw i of stream s is
 * mix(base(seed, s) + (i + 1) * GAMMA), so every element can be produced
 * independently, in any order and on any number of threads.  Normals come from
 * the Box-Muller transform (cosine branch only; one normal per pair of draws).
 *
 * bf16 values are produced by round-to-nearest-even of the double-precision
 * sample, done through an exact integer construction so that no double
 * rounding occurs.
 */
#include <stdint.h>
#include <math.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed * GAMMA + 0x632BE59BD9B4E019ULL) ^ (stream * 0xD1B54A32D192ED03ULL));
}

/* uniform in the open interval (0, 1) */
static inline double uniform_at(uint64_t base, uint64_t i) {
  uint64_t x = mix64(base + (i + 1) * GAMMA);
  return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t base, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = uniform_at(base, 2 * i);
  double u2 = uniform_at(base, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* Round a double to bf16 (nearest, ties to even) with no double rounding:
   first round to fp32 by round-to-odd (truncate, then set the sticky lowest
   bit if anything was dropped), then round that fp32 to bf16 to nearest-even.
   fp32 keeps 16 more significand bits than bf16, so the two-step result
   equals the direct correctly rounded one. */
static inline uint16_t double_to_bf16_bits(double x) {
  uint32_t u;
  float f = (float)x;
  if (!isnan(x) && (double)f != x) {
    if (fabs((double)f) > fabs(x)) f = nextafterf(f, 0.0f);
    memcpy(&u, &f, 4);
    u |= 1u;
  } else {
    memcpy(&u, &f, 4);
  }
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline double softplus(double x) {
  return x > 0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

/*
 * Fill a [rows, d] block of vectors: each row ~ N(0, I_d) (element index
 * row*d + j of the stream), optionally scaled to unit L2 norm in double
 * before rounding.  dtype 0 writes float, dtype 1 writes bf16 bits.
 */
void synth_vectors(uint64_t seed, uint64_t stream, int64_t rows, int64_t d,
                   int unit_norm, int dtype, void* dst, int64_t row0) {
  uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double buf[1024]; /* d <= 1024 is checked by the Python wrapper */
    int64_t gr = row0 + r;
    double ss = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      double z = normal_at(base, (uint64_t)(gr * d + j));
      buf[j] = z;
      ss += z * z;
    }
    double scale = 1.0;
    if (unit_norm) scale = 1.0 / sqrt(ss);
    if (dtype == 0) {
      float* o = (float*)dst + r * d;
      for (int64_t j = 0; j < d; ++j) o[j] = (float)(buf[j] * scale);
    } else {
      uint16_t* o = (uint16_t*)dst + r * d;
      for (int64_t j = 0; j < d; ++j) o[j] = double_to_bf16_bits(buf[j] * scale);
    }
  }
}

/*
 * Raw (un-normalised) vectors for testing a consumer's own normalisation:
 * each row ~ N(0, I_d) times a per-row scale 10^(6u - 3), u ~ U(0, 1) from
 * stream `scale_stream` (row norms from about 1e-3 sqrt(d) to 1e3 sqrt(d)),
 * except every 37th row (global row index 5 mod 37), which is rescaled to an
 * L2 norm of 10^(-6 + 0.6 (u - 0.5)) -- between about 0.5e-6 and 2e-6, on
 * both sides of a 1e-6 norm clamp.  dtype as for synth_vectors.
 */
void synth_vectors_raw(uint64_t seed, uint64_t stream, uint64_t scale_stream, int64_t rows, int64_t d,
                       int dtype, void* dst, int64_t row0) {
  uint64_t base = stream_base(seed, stream);
  uint64_t sbase = stream_base(seed, scale_stream);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double buf[1024]; /* d <= 1024 is checked by the Python wrapper */
    int64_t gr = row0 + r;
    double ss = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      double z = normal_at(base, (uint64_t)(gr * d + j));
      buf[j] = z;
      ss += z * z;
    }
    double u = uniform_at(sbase, (uint64_t)gr);
    double scale = (gr % 37 == 5) ? pow(10.0, -6.0 + 0.6 * (u - 0.5)) / sqrt(ss) : pow(10.0, 6.0 * u - 3.0);
    if (dtype == 0) {
      float* o = (float*)dst + r * d;
      for (int64_t j = 0; j < d; ++j) o[j] = (float)(buf[j] * scale);
    } else {
      uint16_t* o = (uint16_t*)dst + r * d;
      for (int64_t j = 0; j < d; ++j) o[j] = double_to_bf16_bits(buf[j] * scale);
    }
  }
}

/*
 * Fill n scalars from stream `stream` with one of these distributions:
 *   kind 0: N(0,1) * p0                         (plain normal, std p0)
 *   kind 1: sigmoid(N(0,1))                     (write-strength gates)
 *   kind 2: -softplus(N(0,1) + p0)              (log decay gates)
 *   kind 3: constant p0
 * Output is float.
 */
void synth_scalars(uint64_t seed, uint64_t stream, int64_t n, int kind, double p0,
                   float* dst, int64_t i0) {
  uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double z = (kind == 3) ? 0.0 : normal_at(base, (uint64_t)(i0 + i));
    double y;
    switch (kind) {
      case 0: y = z * p0; break;
      case 1: y = 1.0 / (1.0 + exp(-z)); break;
      case 2: y = -softplus(z + p0); break;
      default: y = p0; break;
    }
    dst[i] = (float)y;
  }
}

/* Exact widening of bf16 bit patterns to float (for handing inputs to the oracle). */
void synth_bf16_to_f32(const uint16_t* src, float* dst, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)src[i] << 16;
    memcpy(&dst[i], &u, 4);
  }
}

int synth_abi_version(void) { return 1; }
