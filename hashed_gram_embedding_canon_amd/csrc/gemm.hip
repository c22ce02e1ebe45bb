// Key/value projections ("DeepSeek AI II", section "DeepSeek Engram": the
// retrieved memory e_t is the shared input of the key and value
// projections W_K, W_V) and the backward contraction de = W_K^T dk + W_V^T dv,
// on CDNA4 matrix cores.
//
// Formulation: C^T[f][m] = sum_k A[f][k] B[m][k] with A = the weight rows
// (output features f, K contiguous) and B = the token rows (K contiguous).
// Features are the MFMA row dimension and tokens the column dimension, so
// each lane of a 32x32 accumulator block owns one token and 16 of its
// features.  That makes the gate's per-token reductions (sum k^2,
// sum g_q g_k h k, sum h^2) plain in-register sums in the epilogue: the key
// never goes to HBM, and h is read exactly once, here.
//
// Tiling: 256 features x 256 tokens per workgroup, 128 bytes of K per stage
// (64 bf16/fp16 or 32 fp32 values), double-buffered in LDS with a 16-byte row
// pad (conflict-free ds_read_b128 of the 32-row MFMA fragments).  Matrix
// cores: v_mfma_f32_32x32x16_bf16 / _f16; fp32 inputs use four
// v_mfma_f32_32x32x2f32 per 16-byte fragment.  Workgroup ids are spread over
// the 8 XCDs round-robin by the hardware; the id -> tile map keeps the
// f-tiles of a small group of token tiles on one XCD so that their e rows
// and weight slabs are shared through that XCD's L2.
#include "kernels.h"

namespace engram {

template <int GT>
struct Mma;

template <>
struct Mma<GEMM_BF16> {
  __device__ static inline void run(const u32x4& a, const u32x4& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mma<GEMM_F16> {
  __device__ static inline void run(const u32x4& a, const u32x4& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                               __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
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
};

// 4 consecutive values of an io tensor (bf16 or fp32) as floats.
__device__ inline floatx4 load4(const uint8_t* base, int64_t i, int io) {
  if (io == ENGRAM_BF16) {
    const u32x2 u = *reinterpret_cast<const u32x2*>(base + i * 2);
    return floatx4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                   __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
  }
  return *reinterpret_cast<const floatx4*>(base + i * 4);
}

__device__ inline void store4(uint8_t* base, int64_t i, int io, float a, float b, float c, float d) {
  if (io == ENGRAM_BF16) {
    u32x2 u;
    u.x = (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
    u.y = (uint32_t)f32_to_bf16_bits(c) | ((uint32_t)f32_to_bf16_bits(d) << 16);
    *reinterpret_cast<u32x2*>(base + i * 2) = u;
  } else {
    *reinterpret_cast<floatx4*>(base + i * 4) = floatx4{a, b, c, d};
  }
}

template <int GT, int EPI, int BF, int BT, int WF, int WT>
__global__ __launch_bounds__(WF * WT * 64) void gemm_kernel(GemmArgs g) {
  constexpr int NT = WF * WT * 64;
  constexpr int BKB = 128;          // bytes of K per stage
  constexpr int PITCH = BKB + 16;   // LDS row pitch
  constexpr int FB = BF / WF / 32;  // 32-row MFMA blocks per wave along f
  constexpr int TB = BT / WT / 32;  // 32-column blocks per wave along tokens
  constexpr int CPR = BKB / 16;     // 16-byte chunks per row and stage
  constexpr int ACH = BF * CPR / NT;
  constexpr int BCH = BT * CPR / NT;
  static_assert(ACH * NT == BF * CPR && BCH * NT == BT * CPR, "tile/thread mismatch");
  constexpr int ES = (GT == GEMM_F32) ? 4 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (BF + BT) * PITCH];

  // ---- workgroup id -> (token tile, feature tile), XCD-grouped
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int tiles_f = g.F / BF;
  const int gm = g.group_m;
  const int per_group = gm * tiles_f;
  const int grp = slot / per_group;
  const int in_g = slot - grp * per_group;
  const int tf = in_g / gm;
  const int tm_local = in_g - tf * gm;
  const int64_t tm = (int64_t)(grp * gm + tm_local) * 8 + xcd;
  const int64_t tiles_m = (g.M + BT - 1) / BT;
  if (tm >= tiles_m) return;
  const int f0 = tf * BF;
  const int64_t m0 = tm * BT;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wf = wave % WF;
  const int wt = wave / WF;
  const int64_t row_bytes = (int64_t)g.K * ES;
  const uint8_t* __restrict__ gA = g.A;
  const uint8_t* __restrict__ gB = g.B;

  u32x4 ra[ACH], rb[BCH];
#define ENGRAM_GLOAD(kt)                                                                      \
  do {                                                                                        \
    const int64_t kb_ = (int64_t)(kt) * BKB;                                                  \
    _Pragma("unroll") for (int i = 0; i < ACH; ++i) {                                         \
      const int c_ = tid + i * NT;                                                            \
      ra[i] = *reinterpret_cast<const u32x4*>(gA + (int64_t)(f0 + c_ / CPR) * row_bytes + kb_ + \
                                              (c_ % CPR) * 16);                               \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < BCH; ++i) {                                         \
      const int c_ = tid + i * NT;                                                            \
      int64_t m_ = m0 + c_ / CPR;                                                             \
      m_ = m_ < g.M ? m_ : g.M - 1; /* ragged tail: valid row, result masked later */         \
      rb[i] = *reinterpret_cast<const u32x4*>(gB + m_ * row_bytes + kb_ + (c_ % CPR) * 16);   \
    }                                                                                         \
  } while (0)
#define ENGRAM_LSTORE(buf)                                                                    \
  do {                                                                                        \
    uint8_t* la_ = lds + (buf) * (BF + BT) * PITCH;                                           \
    uint8_t* lb_ = la_ + BF * PITCH;                                                          \
    _Pragma("unroll") for (int i = 0; i < ACH; ++i) {                                         \
      const int c_ = tid + i * NT;                                                            \
      *reinterpret_cast<u32x4*>(la_ + (c_ / CPR) * PITCH + (c_ % CPR) * 16) = ra[i];          \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < BCH; ++i) {                                         \
      const int c_ = tid + i * NT;                                                            \
      *reinterpret_cast<u32x4*>(lb_ + (c_ / CPR) * PITCH + (c_ % CPR) * 16) = rb[i];          \
    }                                                                                         \
  } while (0)

  floatx16 acc[FB][TB];
#pragma unroll
  for (int a = 0; a < FB; ++a)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[a][b] = floatx16{};

  const int nk = (int)(row_bytes / BKB);
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  ENGRAM_GLOAD(0);
  ENGRAM_LSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) ENGRAM_GLOAD(kt + 1);
    const uint8_t* la = lds + cur * (BF + BT) * PITCH;
    const uint8_t* lb = la + BF * PITCH;
#pragma unroll
    for (int s = 0; s < BKB / 32; ++s) {
      u32x4 af[FB], bfr[TB];
#pragma unroll
      for (int a = 0; a < FB; ++a)
        af[a] = *reinterpret_cast<const u32x4*>(la + ((wf * FB + a) * 32 + lrow) * PITCH + s * 32 +
                                                lhalf * 16);
#pragma unroll
      for (int b = 0; b < TB; ++b)
        bfr[b] = *reinterpret_cast<const u32x4*>(lb + ((wt * TB + b) * 32 + lrow) * PITCH + s * 32 +
                                                 lhalf * 16);
#pragma unroll
      for (int a = 0; a < FB; ++a)
#pragma unroll
        for (int b = 0; b < TB; ++b) Mma<GT>::run(af[a], bfr[b], acc[a][b]);
    }
    if (kt + 1 < nk) ENGRAM_LSTORE(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogues.  acc[a][b][q*4+r] holds C^T[f][m] with
  //      f = f0 + (wf*FB + a)*32 + q*8 + lhalf*4 + r,  m = m0 + (wt*TB + b)*32 + lrow
  if constexpr (EPI == EPI_KV) {
    const int io = g.io_dtype;
    const int d = g.d;
    if (f0 < d) {
      // key tile: per-token partial sums of the gate; k itself only if asked
      float skk[TB], shk[TB], shh[TB];
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        skk[b] = 0.f;
        shk[b] = 0.f;
        shh[b] = 0.f;
        const int64_t m = m0 + (wt * TB + b) * 32 + lrow;
        const bool valid = m < g.M;
        const int64_t mc = valid ? m : g.M - 1;
#pragma unroll
        for (int a = 0; a < FB; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = f0 + (wf * FB + a) * 32 + q * 8 + lhalf * 4;
            const floatx4 hv = load4(g.h, mc * d + f, io);
            floatx4 gg = floatx4{1.f, 1.f, 1.f, 1.f};
            if (g.gamma_q) gg *= *reinterpret_cast<const floatx4*>(g.gamma_q + f);
            if (g.gamma_k) gg *= *reinterpret_cast<const floatx4*>(g.gamma_k + f);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float kv = acc[a][b][q * 4 + r];
              skk[b] += kv * kv;
              shk[b] += gg[r] * hv[r] * kv;
              shh[b] += hv[r] * hv[r];
            }
            if (g.k_out && valid)
              store4(g.k_out, m * d + f, io, acc[a][b][q * 4], acc[a][b][q * 4 + 1],
                     acc[a][b][q * 4 + 2], acc[a][b][q * 4 + 3]);
            // keep the h loads of later fragments from being hoisted here: the
            // 128 accumulator registers leave little room
            __builtin_amdgcn_sched_barrier(0);
          }
        skk[b] += __shfl_xor(skk[b], 32);
        shk[b] += __shfl_xor(shk[b], 32);
        shh[b] += __shfl_xor(shh[b], 32);
      }
      // combine the WF waves that share these tokens
      float* red = reinterpret_cast<float*>(lds);  // [WF][WT][TB][32][3]
      if (lhalf == 0) {
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          float* p = red + ((((wf * WT) + wt) * TB + b) * 32 + lrow) * 3;
          p[0] = skk[b];
          p[1] = shk[b];
          p[2] = shh[b];
        }
      }
      __syncthreads();
      if (wf == 0 && lhalf == 0) {
        const int nkt = d / BF;
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const int64_t m = m0 + (wt * TB + b) * 32 + lrow;
          if (m >= g.M) continue;
          float s0 = 0.f, s1 = 0.f, s2 = 0.f;
#pragma unroll
          for (int w = 0; w < WF; ++w) {
            const float* p = red + ((((w * WT) + wt) * TB + b) * 32 + lrow) * 3;
            s0 += p[0];
            s1 += p[1];
            s2 += p[2];
          }
          float* out = g.partials + (m * nkt + tf) * 3;
          out[0] = s0;
          out[1] = s1;
          out[2] = s2;
        }
      }
    } else {
      // value tile
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        const int64_t m = m0 + (wt * TB + b) * 32 + lrow;
        if (m >= g.M) continue;
#pragma unroll
        for (int a = 0; a < FB; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = f0 - d + (wf * FB + a) * 32 + q * 8 + lhalf * 4;
            store4(g.v_out, m * d + f, io, acc[a][b][q * 4], acc[a][b][q * 4 + 1],
                   acc[a][b][q * 4 + 2], acc[a][b][q * 4 + 3]);
          }
      }
    }
  } else {
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const int64_t m = m0 + (wt * TB + b) * 32 + lrow;
      if (m >= g.M) continue;
#pragma unroll
      for (int a = 0; a < FB; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = f0 + (wf * FB + a) * 32 + q * 8 + lhalf * 4;
          *reinterpret_cast<floatx4*>(g.c_out + m * g.F + f) =
              floatx4{acc[a][b][q * 4], acc[a][b][q * 4 + 1], acc[a][b][q * 4 + 2],
                      acc[a][b][q * 4 + 3]};
        }
    }
  }
}

#undef ENGRAM_GLOAD
#undef ENGRAM_LSTORE

template <int GT, int EPI>
static hipError_t launch_one(const GemmArgs& g, hipStream_t s) {
  constexpr int BF = kGemmBF, BT = 256, WF = 2, WT = 4;
  const int64_t tiles_m = (g.M + BT - 1) / BT;
  const int tiles_f = g.F / BF;
  const int64_t tiles_m_x = (tiles_m + 7) / 8;
  const int64_t groups = (tiles_m_x + g.group_m - 1) / g.group_m;
  const int64_t blocks = 8 * groups * g.group_m * tiles_f;
  hipLaunchKernelGGL((gemm_kernel<GT, EPI, BF, BT, WF, WT>), dim3((unsigned)blocks),
                     dim3(WF * WT * 64), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm(GemmType type, GemmEpilogue epi, const GemmArgs& g, hipStream_t s) {
  if (g.M == 0) return hipSuccess;
  if (epi == EPI_KV) {
    if (type == GEMM_BF16) return launch_one<GEMM_BF16, EPI_KV>(g, s);
    if (type == GEMM_F32) return launch_one<GEMM_F32, EPI_KV>(g, s);
  } else {
    if (type == GEMM_F16) return launch_one<GEMM_F16, EPI_STORE_F32>(g, s);
    if (type == GEMM_F32) return launch_one<GEMM_F32, EPI_STORE_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace engram
