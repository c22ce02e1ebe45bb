// Shared device/host helpers of the Engram HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engram.h"

namespace engram {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ----------------------------------------------------------- number formats
// bf16 <-> fp32 on raw bits: widening is exact; narrowing rounds to nearest
// even (inputs are finite).
__host__ __device__ inline float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
__host__ __device__ inline uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// Two floats -> packed bf16 pair (a in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950, the same result as f32_to_bf16_bits for
// finite inputs.
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 r = __builtin_convertvector(floatx2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// ------------------------------------------------------- exact x mod prime
// x mod p for a 64-bit x and 1 <= p < 2^31 without a 64-bit divide.
// recip = floor((2^64 - 1) / p).  With q = floor(x * recip / 2^64):
// x*recip/2^64 = x/p - x*(1+s)/(p*2^64) where 2^64-1 = recip*p + s, s < p,
// so x/p - 1 < x*recip/2^64 <= x/p and q is floor(x/p) or floor(x/p) - 1:
// one conditional subtraction restores the exact remainder.
__host__ __device__ inline uint64_t mulhi_u64(uint64_t a, uint64_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __umul64hi(a, b);
#else
  return (uint64_t)(((unsigned __int128)a * b) >> 64);
#endif
}
__host__ __device__ inline uint32_t mod_prime(uint64_t x, uint32_t p, uint64_t recip) {
  uint64_t q = mulhi_u64(x, recip);
  uint64_t r = x - q * (uint64_t)p;
  if (r >= p) r -= p;
  return (uint32_t)r;
}
inline uint64_t mod_recip(uint32_t p) { return ~0ull / (uint64_t)p; }

// ------------------------------------------------------- hash parameters
struct HashArgs {
  int32_t J;
  int32_t num_orders;
  int32_t heads;
  int32_t max_order;
  int32_t pad_id;
  int32_t orders[ENGRAM_MAX_ORDERS];
  uint32_t prime[ENGRAM_MAX_TABLES];
  uint64_t recip[ENGRAM_MAX_TABLES];
  uint64_t mult[ENGRAM_MAX_TABLES * ENGRAM_MAX_ORDERS];  // [j][i], i < max_order
  // id check (null: ids are trusted): an id outside [0, vocab) is counted
  // into *bad and read as canonical pad_id, so canon_map is never indexed
  // out of bounds
  uint32_t* bad;
  int32_t vocab;
};

#if defined(__HIPCC__)
// Canonical id of raw token x under the id check of a (see HashArgs::bad).
// Several lanes may read one token (context windows); only the read that
// owns it (own = true) counts it, so *bad ends up as the number of bad ids.
__device__ inline uint32_t canon_of(const int32_t* __restrict__ canon, int32_t x, const HashArgs& a,
                                    bool own) {
  if (a.bad != nullptr && (uint32_t)x >= (uint32_t)a.vocab) {
    if (own) atomicAdd(a.bad, 1u);
    return (uint32_t)a.pad_id;
  }
  return (uint32_t)canon[x];
}
#endif

// idx_j for one token given its canonical context c[i] = c_{t-i} (i < max_order).
__host__ __device__ inline uint32_t hash_one(const HashArgs& a, int j, int n, const uint32_t* c) {
  uint64_t x = 0;
  for (int i = 0; i < n; ++i) x ^= a.mult[j * a.max_order + i] * (uint64_t)c[i];
  return mod_prime(x, a.prime[j], a.recip[j]);
}

inline size_t dtype_size(int32_t dt) { return dt == ENGRAM_BF16 ? 2 : 4; }

}  // namespace engram
