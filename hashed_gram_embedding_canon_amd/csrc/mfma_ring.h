// Pieces shared by the matrix-core kernels: the MFMA wrappers, accumulator
// reads, direct-to-LDS global loads, a fence-free workgroup barrier and
// explicit vmcnt waits.
#pragma once
#include "kernels.h"

namespace engram {

template <int GT>
struct Mma;

// run0: c = a b with a zero accumulator (an inline-constant C operand, so a
// tile's accumulators need no zeroing writes)
template <>
struct Mma<GEMM_BF16> {
  __device__ static inline void run(const u32x4& a, const u32x4& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline void run0(const u32x4& a, const u32x4& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), floatx16{}, 0, 0, 0);
  }
};

template <>
struct Mma<GEMM_F16> {
  __device__ static inline void run(const u32x4& a, const u32x4& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                               __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
  }
  __device__ static inline void run0(const u32x4& a, const u32x4& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                               __builtin_bit_cast(halfx8, b), floatx16{}, 0, 0, 0);
  }
};

// E4M3 x E4M3 (format codes 0 and 0, no block scales): lanes 0-31 hold
// k = 0..31 of a 64-element K slice, lanes 32-63 hold k = 32..63.
template <>
struct Mma<GEMM_FP8> {
  __device__ static inline void run(const u32x8& a, const u32x8& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                         __builtin_bit_cast(i32x8, b), c, 0, 0, 0, 0,
                                                         0, 0);
  }
  __device__ static inline void run0(const u32x8& a, const u32x8& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                         __builtin_bit_cast(i32x8, b), floatx16{}, 0,
                                                         0, 0, 0, 0, 0);
  }
};

// fp32: lanes 0-31 hold k = 0..3 of the 32-byte K slice, lanes 32-63 hold
// k = 4..7; step i multiplies the pair (i, 4+i), so four steps cover all 8.
template <>
struct Mma<GEMM_F32> {
  __device__ static inline void run(const u32x4& a, const u32x4& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
  __device__ static inline void run0(const u32x4& a, const u32x4& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), floatx16{}, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

// One accumulator value copied out of its AGPR at the point of use.  Left to
// itself the register allocator moves all 256 accumulators into VGPRs when
// the epilogue does arithmetic on them, and spills.
__device__ inline float acc_read(float x) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}

// LDS byte address of a __shared__ object.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Wave-uniform 64-bit value, held in SGPRs.
__device__ inline const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// 16-byte direct-to-LDS global loads: lane l's 16 bytes land at LDS address
// m0v + 16*l (m0v is wave-uniform and goes through M0).  Written as asm so
// that the compiler does not treat every later LDS read as aliasing the write
// and wait for all loads in flight; the ring below waits with explicit vmcnt
// counts.  The instructions have no destination register, so nothing the
// compiler allocates can be overwritten while they are in flight.  M0 is a
// register the compiler reserves and assumes unchanged across asm, so each
// block restores it (the load reads M0 when it issues).
//   load_lds16:   per-lane 64-bit address
//   load_lds16_s: wave-uniform 64-bit base (SGPRs) + per-lane 32-bit offset,
//                 so a stage's loads need no per-lane address arithmetic
__device__ inline void load_lds16(const void* src, uint32_t m0v) {
  m0v = __builtin_amdgcn_readfirstlane(m0v);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(src), "s"(m0v)
               : "memory");
}
__device__ inline void load_lds16_s(uint32_t voff, const void* sbase, uint32_t m0v) {
  m0v = __builtin_amdgcn_readfirstlane(m0v);
  sbase = uniform_ptr(sbase);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(voff), "s"(sbase), "s"(m0v)
               : "memory");
}

// The same load for a caller that keeps M0 for a group of loads: it saves M0
// once (M0Keep) and restores it when the group ends (two scalar moves per
// group instead of per load).
__device__ inline void load_lds16_s_kept(uint32_t voff, const void* sbase, uint32_t m0v) {
  m0v = __builtin_amdgcn_readfirstlane(m0v);
  sbase = uniform_ptr(sbase);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0v)
               : "memory");
}
struct M0Keep {
  uint32_t saved;
  __device__ M0Keep() { asm volatile("s_mov_b32 %0, m0" : "=s"(saved)); }
  __device__ ~M0Keep() { asm volatile("s_mov_b32 m0, %0" : : "s"(saved) : "memory"); }
};

// Workgroup barrier without a memory fence: LDS written by this wave's
// direct-to-LDS loads is complete once vmcnt says so (waited for explicitly
// before the barrier), and LDS reads of the previous stage were consumed by
// MFMAs before it.  __syncthreads() would also wait for every load in flight.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier (the s_barrier builtin itself is not a memory operation
// to the optimizer).
#define ENGRAM_BARRIER()                 \
  do {                                   \
    asm volatile("" ::: "memory");       \
    __builtin_amdgcn_sched_barrier(0);   \
    __builtin_amdgcn_s_barrier();        \
    __builtin_amdgcn_sched_barrier(0);   \
    asm volatile("" ::: "memory");       \
  } while (0)

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding)
#define ENGRAM_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(((n)&0xF) | ((((n) >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8))
// the same, and all of this wave's LDS operations complete
#define ENGRAM_WAIT_VM_LDS(n) \
  __builtin_amdgcn_s_waitcnt(((n)&0xF) | ((((n) >> 4) & 3) << 14) | (0x7 << 4))

}  // namespace engram
