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

// R tokens per workgroup and v rows loaded ahead per lane.  Measured at the
// 27B shape (d = 2560): R = 24 with 8 rows ahead 0.255 ms; R = 16, 32 and 48
// 0.260-0.264; R = 64 with 2, 4, 8 and 12 rows ahead 0.290, 0.269, 0.265 and
// 0.277; R = 128 0.282.
#ifndef ENGRAM_GC_TOKENS
#define ENGRAM_GC_TOKENS 24
#endif
constexpr int kGcTokens = ENGRAM_GC_TOKENS;
#ifndef ENGRAM_GC_RING
#define ENGRAM_GC_RING 8
#endif
// Non-temporal stores of Y (bit 2; bit 1 would make the v loads
// non-temporal): Y is not read again here, and keeping it out of the 256 MB
// Infinity Cache leaves the table rows of the Zipf head there for the next
// batch's gather (0.170 -> 0.150 ms on distinct batches) at the cost of 3 %
// in this kernel (0.286 -> 0.294 ms).
#ifndef ENGRAM_GC_NT
#define ENGRAM_GC_NT 2
#endif
constexpr int kMaxTaps = 8;
// feature tiles of partial sums loaded in one burst (d <= 16 * 256)
#ifndef ENGRAM_GC_MAX_TILES
#define ENGRAM_GC_MAX_TILES 16
#endif
constexpr int kGcMaxTiles = ENGRAM_GC_MAX_TILES;

// raw 16 bytes of VEC features (8 bf16 or 4 fp32), widened at use
template <int VEC, bool BF16>
__device__ inline u32x4 load_raw(const uint8_t* base, int64_t elem) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base + elem * (BF16 ? 2 : 4));
  if constexpr ((ENGRAM_GC_NT & 1) != 0)
    return __builtin_nontemporal_load(p);
  else
    return *p;
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
    u32x4* p = reinterpret_cast<u32x4*>(base + elem * 2);
    if constexpr ((ENGRAM_GC_NT & 2) != 0)
      __builtin_nontemporal_store(u, p);
    else
      *p = u;
  } else {
    *reinterpret_cast<floatx4*>(base + elem * 4) = floatx4{v[0], v[1], v[2], v[3]};
  }
}

// SINGLE: one branch.  Its window then holds the gated values
// vt = alpha v themselves, so a token's conv is taps multiply-adds per
// feature instead of a product per tap and a gate-weighted sum of them.
template <int VEC, bool BF16, int TAPS, bool SINGLE>
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

  const int f = threadIdx.x * VEC;
  const int64_t tend = (t0 + R < a.T) ? t0 + R : a.T;
  const uint8_t* __restrict__ vsrc = a.v;
  const int64_t row0 = b * a.T;
  constexpr int PD = ENGRAM_GC_RING;
  u32x4 ring[PD];

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
      if (a.nkt <= kGcMaxTiles) {
        // all of the token's partial sums in flight at once, added in tile order
        float pv[kGcMaxTiles * 3];
#pragma unroll
        for (int q = 0; q < kGcMaxTiles * 3; ++q) pv[q] = q < a.nkt * 3 ? p[q] : 0.f;
#pragma unroll
        for (int q = 0; q < kGcMaxTiles; ++q) {
          if (q < a.nkt) {
            skk += pv[3 * q];
            shk += pv[3 * q + 1];
            shh += pv[3 * q + 2];
          }
        }
      } else {
        for (int q = 0; q < a.nkt; ++q) {
          skk += p[3 * q];
          shk += p[3 * q + 1];
          shh += p[3 * q + 2];
        }
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
  if (f >= d) return;
  float w[VEC][TAPS];
#pragma unroll
  for (int c = 0; c < VEC; ++c)
#pragma unroll
    for (int i = 0; i < TAPS; ++i) w[c][i] = a.conv_w[(f + c) * TAPS + i];
  float win[NW][VEC];  // win[i] = raw v (SINGLE: alpha v) at t-1-i
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int c = 0; c < VEC; ++c) win[i][c] = 0.f;

  const int64_t ystride = N * d * (BF16 ? 2 : 4);  // bytes between branch outputs
  // The window starts with the taps-1 tokens before t0 (zero gate before the
  // sequence start); v rows then stream through a ring of PD tokens loaded
  // ahead (each wave keeps PD 1 KB loads in flight).  Every load is
  // unconditional, its row clamped into the tile, so the compiler can count
  // the loads in flight instead of draining them at the loop's back edge.
  // Load order: conv weights, halo, ring.  Waiting for the halo then also
  // completes the weights, so no load from before the loop is still pending
  // at its head (a pending one would make every iteration drain the ring).
  const int64_t last = tend - 1;
  __builtin_amdgcn_sched_barrier(0);
  u32x4 halo[NW];
  if constexpr (TAPS > 1) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int64_t th = t0 - NW + i;
      halo[i] = load_raw<VEC, BF16>(vsrc, (row0 + (th > 0 ? th : 0)) * d + f);
    }
  }
#pragma unroll
  for (int u = 0; u < PD; ++u) {
    const int64_t t = t0 + u < last ? t0 + u : last;
    ring[u] = load_raw<VEC, BF16>(vsrc, (row0 + t) * d + f);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (TAPS > 1) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int64_t th = t0 - NW + i;  // gate 0 before the sequence start
      float cur[VEC];
      widen<VEC, BF16>(halo[i], cur);
      const float al0 = SINGLE ? alpha_s[(int)(th - (t0 - nh))] : 1.f;
#pragma unroll
      for (int c = 0; c < VEC; ++c) win[NW - 1 - i][c] = th >= 0 ? al0 * cur[c] : 0.f;
    }
  }
  const int n_out = (int)(tend - t0);
  // conv, SiLU and residual of token t from its raw v, then the window shift
  auto token = [&](int64_t t, const float* cur) __attribute__((always_inline)) {
    const int li = (int)(t - (t0 - nh));
    if constexpr (SINGLE) {
      const float al0 = alpha_s[li];
      float vt[VEC];
#pragma unroll
      for (int c = 0; c < VEC; ++c) vt[c] = al0 * cur[c];
      float out[VEC];
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        float z = w[c][0] * vt[c];
#pragma unroll
        for (int k = 1; k < TAPS; ++k) z += w[c][k] * win[k - 1][c];
        // SiLU with the hardware exp2 and reciprocal (about 1 ulp each)
        out[c] = z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)) + vt[c];
      }
      store_vec<VEC, BF16>(a.y, (row0 + t) * d + f, out);
#pragma unroll
      for (int k = NW - 1; k > 0; --k)
#pragma unroll
        for (int c = 0; c < VEC; ++c) win[k][c] = win[k - 1][c];
#pragma unroll
      for (int c = 0; c < VEC; ++c) win[0][c] = vt[c];
    } else {
      // weighted taps, shared by the branches
      float p[TAPS][VEC];
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        p[0][c] = w[c][0] * cur[c];
#pragma unroll
        for (int k = 1; k < TAPS; ++k) p[k][c] = w[c][k] * win[k - 1][c];
      }
      uint8_t* ydst = a.y;
      for (int m = 0; m < nbr; ++m, ydst += ystride) {
        const float* al = alpha_s + m * RH + li;  // al[-k] = alpha_m(t-k)
        float out[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
          float z = al[0] * p[0][c];
#pragma unroll
          for (int k = 1; k < TAPS; ++k) z += al[-k] * p[k][c];
          // SiLU with the hardware exp2 and reciprocal (about 1 ulp each)
          out[c] = z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)) + al[0] * cur[c];
        }
        store_vec<VEC, BF16>(ydst, (row0 + t) * d + f, out);
      }
#pragma unroll
      for (int k = NW - 1; k > 0; --k)
#pragma unroll
        for (int c = 0; c < VEC; ++c) win[k][c] = win[k - 1][c];
#pragma unroll
      for (int c = 0; c < VEC; ++c) win[0][c] = cur[c];
    }
  };
  // whole groups of PD tokens: one path, no branch inside
  const int n_full = n_out - n_out % PD;
  for (int i = 0; i < n_full; i += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int64_t t = t0 + i + u;
      float cur[VEC];
      widen<VEC, BF16>(ring[u], cur);
      // the slot's next load after its value is read, into the same registers
      // (hoisted above the read, it would need others and a copy that waits
      // for it at the loop's back edge)
      __builtin_amdgcn_sched_barrier(0);
      {
        const int64_t tn = t + PD < last ? t + PD : last;
        ring[u] = load_raw<VEC, BF16>(vsrc, (row0 + tn) * d + f);
      }
      token(t, cur);
    }
  }
  // the rest of a tile at the end of a sequence: already in the ring
#pragma unroll
  for (int u = 0; u < PD; ++u) {
    if (n_full + u < n_out) {
      float cur[VEC];
      widen<VEC, BF16>(ring[u], cur);
      token(t0 + n_full + u, cur);
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
  const bool single = a.branches <= 1;
  switch (a.taps) {
#define ENGRAM_TAPS_CASE(K)                                                                      \
  case K:                                                                                        \
    if (bf && single)                                                                            \
      hipLaunchKernelGGL((gate_conv_kernel<8, true, K, true>), grid, dim3(threads), 0, s, a);   \
    else if (bf)                                                                                 \
      hipLaunchKernelGGL((gate_conv_kernel<8, true, K, false>), grid, dim3(threads), 0, s, a);  \
    else if (single)                                                                             \
      hipLaunchKernelGGL((gate_conv_kernel<4, false, K, true>), grid, dim3(threads), 0, s, a);  \
    else                                                                                         \
      hipLaunchKernelGGL((gate_conv_kernel<4, false, K, false>), grid, dim3(threads), 0, s, a); \
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
