// Context-aware gate and short causal depthwise convolution ("DeepSeek AI
// II", section "DeepSeek Engram": RMSNorm on query h_t and key k_t, scalar
// gate alpha_t in (0,1), gated value alpha_t v_t, then a short-kernel
// depthwise causal convolution for a wider receptive field and extra
// non-linearity, added back residually).
//
// One workgroup owns R consecutive tokens of one sequence and all d
// features (a lane holds VEC neighbouring features).  The gate of each token
// comes from the per-feature-tile partial sums that the projection epilogue
// left behind (sum k^2, sum g_q g_k h k, sum h^2), so k and h are never read
// here.  The conv walks the tokens in order with the last taps-1 values of v
// in registers, so v is read once for all branches (plus a taps-1 token halo
// per workgroup) and each branch's Y is written once: an HBM-streaming kernel.
#include "kernels.h"

namespace engram {

constexpr int kGcTokens = 64;   // R (32 and 128 measured slower)
constexpr int kMaxTaps = 8;

// raw 16 bytes of VEC features (8 bf16 or 4 fp32), widened at use
template <int VEC, bool BF16>
__device__ inline u32x4 load_raw(const uint8_t* base, int64_t elem) {
  return *reinterpret_cast<const u32x4*>(base + elem * (BF16 ? 2 : 4));
}
template <int VEC, bool BF16>
__device__ inline void widen(const u32x4 u, float* out) {
  if constexpr (BF16) {
    static_assert(VEC == 8, "");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(u[i] << 16);
      out[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    static_assert(VEC == 4, "");
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(u[i]);
  }
}

template <int VEC, bool BF16>
__device__ inline void store_vec(uint8_t* base, int64_t elem, const float* v) {
  if constexpr (BF16) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4*>(base + elem * 2) = u;
  } else {
    *reinterpret_cast<floatx4*>(base + elem * 4) = floatx4{v[0], v[1], v[2], v[3]};
  }
}

template <int VEC, bool BF16, int TAPS>
__global__ __launch_bounds__(1024) void gate_conv_kernel(GateConvArgs a) {
  constexpr int R = kGcTokens;
  constexpr int NW = TAPS > 1 ? TAPS - 1 : 1;  // window length
  constexpr int RH = R + kMaxTaps;             // gates kept per branch
  // gates of every branch for this tile and its taps-1 token halo
  __shared__ float alpha_s[ENGRAM_MAX_BRANCHES * RH];
  const int nbr = a.branches > 0 ? a.branches : 1;
  const int64_t b = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * R;
  const int nh = TAPS - 1;
  const int d = a.d;
  const int64_t N = a.B * a.T;
  const float inv_d = 1.0f / (float)d;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);

  // ---- gate of tokens t0-nh .. t0+R-1 of each branch (zero before the
  // sequence start); branch m has its own partial sums and stats
  for (int e = threadIdx.x; e < nbr * (R + nh); e += blockDim.x) {
    const int m = e / (R + nh);
    const int i = e - m * (R + nh);
    const int64_t t = t0 - nh + i;
    float al = 0.f;
    if (t >= 0 && t < a.T) {
      const float* p = a.partials + (m * N + b * a.T + t) * a.nkt * 3;
      float skk = 0.f, shk = 0.f, shh = 0.f;
      for (int q = 0; q < a.nkt; ++q) {
        skk += p[3 * q];
        shk += p[3 * q + 1];
        shh += p[3 * q + 2];
      }
      const float rq = 1.0f / sqrtf(shh * inv_d + a.eps);
      const float rk = 1.0f / sqrtf(skk * inv_d + a.eps);
      const float s = shk * rq * rk * inv_sqrt_d;
      al = 1.0f / (1.0f + expf(-s));
      if (a.stats && t >= t0) {
        float* st = a.stats + (m * N + b * a.T + t) * 4;
        *reinterpret_cast<floatx4*>(st) = floatx4{al, rq, rk, shk};
      }
    }
    alpha_s[m * RH + i] = al;
  }
  __syncthreads();

  // ---- causal conv, VEC features per lane.  The branches share v and the
  // conv weights, so one pass over v serves all of them: the lane keeps the
  // last taps-1 raw v values, and branch m's conv input at t-i is
  // alpha_m(t-i) v(t-i), i.e. z_m = sum_i alpha_m(t-i) (w_i v(t-i)).
  const int f = threadIdx.x * VEC;
  if (f >= d) return;
  float w[VEC][TAPS];
#pragma unroll
  for (int c = 0; c < VEC; ++c)
#pragma unroll
    for (int i = 0; i < TAPS; ++i) w[c][i] = a.conv_w[(f + c) * TAPS + i];
  float win[NW][VEC];  // win[i] = raw v at t-1-i
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int c = 0; c < VEC; ++c) win[i][c] = 0.f;

  const int64_t tbeg = t0 - nh > 0 ? t0 - nh : 0;
  const int64_t tend = (t0 + R < a.T) ? t0 + R : a.T;
  const uint8_t* __restrict__ vsrc = a.v;
  const int64_t ystride = N * d * (BF16 ? 2 : 4);  // bytes between branch outputs
  const int64_t row0 = b * a.T;
  // v rows stream through a ring of PD tokens loaded ahead (each wave keeps
  // PD 1 KB loads in flight; HBM latency, not bandwidth, bounds a shallower
  // ring at this occupancy)
  constexpr int PD = 4;  // 8 measured slower (fewer waves fit)
  u32x4 ring[PD];
#pragma unroll
  for (int u = 0; u < PD; ++u)
    if (tbeg + u < tend) ring[u] = load_raw<VEC, BF16>(vsrc, (row0 + tbeg + u) * d + f);
  for (int64_t tb = tbeg; tb < tend; tb += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int64_t t = tb + u;
      if (t < tend) {
        float cur[VEC];
        widen<VEC, BF16>(ring[u], cur);
        if (t + PD < tend) ring[u] = load_raw<VEC, BF16>(vsrc, (row0 + t + PD) * d + f);
        if (t >= t0) {
          // weighted taps, shared by the branches
          float p[TAPS][VEC];
#pragma unroll
          for (int c = 0; c < VEC; ++c) {
            p[0][c] = w[c][0] * cur[c];
#pragma unroll
            for (int i = 1; i < TAPS; ++i) p[i][c] = w[c][i] * win[i - 1][c];
          }
          const int li = (int)(t - (t0 - nh));
          uint8_t* ydst = a.y;
          for (int m = 0; m < nbr; ++m, ydst += ystride) {
            const float* al = alpha_s + m * RH + li;  // al[-i] = alpha_m(t-i)
            float out[VEC];
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
              float z = al[0] * p[0][c];
#pragma unroll
              for (int i = 1; i < TAPS; ++i) z += al[-i] * p[i][c];
              // SiLU with the hardware exp2 and reciprocal (about 1 ulp each)
              out[c] = z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)) + al[0] * cur[c];
            }
            store_vec<VEC, BF16>(ydst, (row0 + t) * d + f, out);
          }
        }
#pragma unroll
        for (int i = NW - 1; i > 0; --i)
#pragma unroll
          for (int c = 0; c < VEC; ++c) win[i][c] = win[i - 1][c];
#pragma unroll
        for (int c = 0; c < VEC; ++c) win[0][c] = cur[c];
      }
    }
  }
}

hipError_t launch_gate_conv(const GateConvArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  const bool bf = a.io_dtype == ENGRAM_BF16;
  const int vec = bf ? 8 : 4;
  int threads = (a.d / vec + 63) / 64 * 64;
  if (threads > 1024) return hipErrorInvalidValue;
  if (a.branches > ENGRAM_MAX_BRANCHES) return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.T + kGcTokens - 1) / kGcTokens), (unsigned)a.B);
  switch (a.taps) {
#define ENGRAM_TAPS_CASE(K)                                                                      \
  case K:                                                                                        \
    if (bf)                                                                                      \
      hipLaunchKernelGGL((gate_conv_kernel<8, true, K>), grid, dim3(threads), 0, s, a);         \
    else                                                                                         \
      hipLaunchKernelGGL((gate_conv_kernel<4, false, K>), grid, dim3(threads), 0, s, a);        \
    break;
    ENGRAM_TAPS_CASE(1)
    ENGRAM_TAPS_CASE(2)
    ENGRAM_TAPS_CASE(3)
    ENGRAM_TAPS_CASE(4)
    ENGRAM_TAPS_CASE(5)
    ENGRAM_TAPS_CASE(6)
    ENGRAM_TAPS_CASE(7)
    ENGRAM_TAPS_CASE(8)
#undef ENGRAM_TAPS_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace engram
