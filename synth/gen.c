/*
 * Seeded synthetic input generators shared by the test harness, the bench
 * and the oracle's callers.  Nothing here computes any step of the Engram
 * method: it only draws token streams, table values, weights and hidden
 * states so that both the GPU library and the CPU oracle read the same
 * arrays.
 *
 * Counter-based stream: splitmix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), element-indexed: the i-th
 * value of stream s is the splitmix64 output for state s + (i+1)*gamma.
 * Normals: Box-Muller (1958) in double on the uniform pair of elements
 * 2p and 2p+1; element 2p takes the cosine branch and 2p+1 the sine branch.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t sm_at(uint64_t seed, uint64_t i) {
  return sm_mix(seed + (i + 1) * SM_GAMMA);
}

/* uniform in [0,1) from the top 53 bits */
static inline double sm_unit(uint64_t x) { return (double)(x >> 11) * (1.0 / 9007199254740992.0); }

static inline double sm_normal(uint64_t seed, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = sm_unit(sm_at(seed, 2 * p));
  double u2 = sm_unit(sm_at(seed, 2 * p + 1));
  double r = sqrt(-2.0 * log(1.0 - u1)); /* 1-u1 lies in (0,1] */
  double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

/* float -> bf16 bits, round to nearest even (inputs are finite) */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

void synth_u64(uint64_t seed, uint64_t offset, int64_t n, uint64_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = sm_at(seed, offset + (uint64_t)i);
}

void synth_unit(uint64_t seed, uint64_t offset, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = sm_unit(sm_at(seed, offset + (uint64_t)i));
}

void synth_normal_f64(uint64_t seed, uint64_t offset, int64_t n, double stdev, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = stdev * sm_normal(seed, offset + (uint64_t)i);
}

void synth_normal_f32(uint64_t seed, uint64_t offset, int64_t n, double stdev, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(stdev * sm_normal(seed, offset + (uint64_t)i));
}

void synth_normal_bf16(uint64_t seed, uint64_t offset, int64_t n, double stdev, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16((float)(stdev * sm_normal(seed, offset + (uint64_t)i)));
}

/*
 * Finite-support Zipf over ranks 1..V with p(r) proportional to r^-s;
 * the sampled id is r-1.  Inverse CDF by binary search over `cdf`
 * (cdf[r-1] = P(rank <= r), filled by synth_zipf_cdf).
 */
void synth_zipf_cdf(int64_t V, double s, double* cdf) {
  double acc = 0.0;
  for (int64_t r = 1; r <= V; ++r) {
    acc += pow((double)r, -s);
    cdf[r - 1] = acc;
  }
  for (int64_t r = 0; r < V; ++r) cdf[r] /= acc;
  cdf[V - 1] = 1.0;
}

void synth_zipf(uint64_t seed, uint64_t offset, int64_t n, int64_t V, const double* cdf, int32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double u = sm_unit(sm_at(seed, offset + (uint64_t)i));
    int64_t lo = 0, hi = V - 1; /* first r with cdf[r] > u */
    while (lo < hi) {
      int64_t mid = (lo + hi) >> 1;
      if (cdf[mid] > u) hi = mid; else lo = mid + 1;
    }
    out[i] = (int32_t)lo;
  }
}
