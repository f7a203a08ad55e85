/*
 * Seeded, counter-based input generator for the CSA2 workloads.
 *
 * This module holds none of the CSA2 method's arithmetic: it only draws
 * random numbers and shapes them like the latents the method consumes.
 * Both the HIP path and the CPU oracle take their inputs from here, so the
 * two sides see the same numbers without either one depending on the other.
 *
 * Generator: every value is a pure function of (seed, tensor id, index).
 *   mix()  is the SplitMix64 output function (Steele, Lea & Flood,
 *          "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014):
 *          add the golden gamma 0x9e3779b97f4a7c15, then two xor-shift-multiply
 *          rounds and a final xor-shift.
 *   hash(seed, tensor, index) = mix(mix(mix(seed) ^ tensor) ^ index).
 *   uniform  U[0,1): top 24 bits of hash(...) times 2^-24 (exact in fp32).
 *   normal   N(0,1): Box-Muller on the pair index p = index / 2 with
 *          u1 = (top 53 bits of hash(seed,tensor,p) + 1) * 2^-53 in (0,1],
 *          u2 = top 53 bits of mix(hash(seed,tensor,p)) * 2^-53,
 *          even index -> r cos(2 pi u2), odd index -> r sin(2 pi u2),
 *          r = sqrt(-2 ln u1); evaluated in fp64, rounded to fp32.
 *
 * Latent rows (the compressed main-KV / SWA latents): N(0,1) per channel,
 * RMS-normalised with unit weight (eps 1e-6), then rotary position embedding
 * on the last `rope_dims` channels (pairs of adjacent channels, base 10^4,
 * position = row * pos_mult), all in fp64, rounded once to fp32.
 *
 * Built with gcc -O2 -fopenmp; deterministic for any thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix(uint64_t z) {
  z += 0x9e3779b97f4a7c15ULL;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t hash3(uint64_t seed, uint64_t tensor, uint64_t index) {
  return mix(mix(mix(seed) ^ tensor) ^ index);
}

uint64_t synth_hash(uint64_t seed, uint64_t tensor, uint64_t index) {
  return hash3(seed, tensor, index);
}

static inline double normal_at(uint64_t seed, uint64_t tensor, uint64_t index) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t h = hash3(seed, tensor, index >> 1);
  uint64_t h2 = mix(h);
  double u1 = ((double)(h >> 11) + 1.0) * 0x1.0p-53;
  double u2 = (double)(h2 >> 11) * 0x1.0p-53;
  double r = sqrt(-2.0 * log(u1));
  return (index & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
}

void synth_normal_f32(uint64_t seed, uint64_t tensor, uint64_t first, int64_t count,
                      float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = (float)normal_at(seed, tensor, first + (uint64_t)i);
}

void synth_uniform_f32(uint64_t seed, uint64_t tensor, uint64_t first, int64_t count,
                       float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i)
    out[i] = (float)((double)(hash3(seed, tensor, first + (uint64_t)i) >> 40) * 0x1.0p-24);
}

/* fp32 -> bf16 bit pattern, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

void synth_normal_bf16(uint64_t seed, uint64_t tensor, uint64_t first, int64_t count,
                       uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i)
    out[i] = f32_to_bf16_rne((float)normal_at(seed, tensor, first + (uint64_t)i));
}

/*
 * rows [row0, row0+rows) of a [*, dim] latent tensor; counter index of
 * channel c of row r is r*dim + c, so any row range reproduces the same values.
 */
void synth_latent_rows(uint64_t seed, uint64_t tensor, int64_t row0, int64_t rows, int dim,
                       int rope_dims, int64_t pos_mult, float* out) {
  const double base = 10000.0;
  double inv_freq[2048];
  for (int p = 0; p < rope_dims / 2; ++p) inv_freq[p] = pow(base, -2.0 * p / rope_dims);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < rows; ++i) {
    double x[4096];
    int64_t r = row0 + i;
    double ss = 0.0;
    for (int c = 0; c < dim; ++c) {
      x[c] = normal_at(seed, tensor, (uint64_t)r * (uint64_t)dim + (uint64_t)c);
      ss += x[c] * x[c];
    }
    double inv = 1.0 / sqrt(ss / dim + 1e-6);
    for (int c = 0; c < dim; ++c) x[c] *= inv;
    double pos = (double)(r * pos_mult);
    int off = dim - rope_dims;
    for (int p = 0; p < rope_dims / 2; ++p) {
      double theta = pos * inv_freq[p];
      double cs = cos(theta), sn = sin(theta);
      double a = x[off + 2 * p], b = x[off + 2 * p + 1];
      x[off + 2 * p] = a * cs - b * sn;
      x[off + 2 * p + 1] = a * sn + b * cs;
    }
    for (int c = 0; c < dim; ++c) out[i * dim + c] = (float)x[c];
  }
}
