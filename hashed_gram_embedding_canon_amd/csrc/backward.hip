// Backward of the gate and the causal conv down to the projection outputs.
//
// The pages ("DeepSeek AI II", system-efficiency part) only say that
// training sends the gradients of the gathered rows back to the table rows;
// the chain rule through the forward of section "DeepSeek Engram" gives, for
// G = dL/dY:
//   dz_u   = G_u * s(z_u) * (1 + z_u (1 - s(z_u)))          (SiLU')
//   dvt_t  = G_t + sum_i w[:,i] * dz_{t+i}                    (residual + conv)
//   dalpha = <dvt_t, v_t>,   dv_t = alpha_t dvt_t
//   ds     = dalpha alpha (1 - alpha)
//   dk_t   = ca g_k g_q h_t - cb k_t,  ca = ds rq rk / sqrt(d),
//            cb = rk^3 ds rq P / (sqrt(d) d),  P = <g_q h_t, g_k k_t>
// (the RMSNorm backward of the key with its projection onto k folded into
// cb).  One workgroup owns R tokens and all d features of one sequence, a
// lane 4 neighbouring features, in two passes:
//   A: walk u = t0-taps+1 .. t0+R+taps-2 with the last taps-1 gated values
//      and the last taps dz in registers; v and G stream through a ring of
//      loads issued a few tokens ahead.  Token t = u-taps+1 is then final:
//      dv_t = alpha_t dvt_t goes out, and the lane's share of dalpha_t joins
//      a batch of 8 tokens that is summed over the wave in 10 shuffles.
//   B: dalpha_t from the per-wave sums; dk_t from h_t and k_t, whose loads
//      do not depend on each other.
// dk and dv leave as fp16 (bf16 io) or fp32 (fp32 io): the de GEMM operands.
// With PARAMS the same passes also give what the module's own parameters
// need: pass A sums dz_t vt_{t-i} per tap over the workgroup's tokens (the
// conv weights' gradient), pass B writes the gate's part of dh_t,
//   dh_t = ca g_q g_k k_t - cq h_t,  cq = rq^3 ds rk P / (sqrt(d) d)
// (the query's RMSNorm backward, the mirror of dk), and sums
// ca h_t k_t, of which the RMSNorm scales' gradients are g_k and g_q times.
// With M branches the kernel runs once per branch m (its dY, h, k, stats):
// dk of branch m goes to its columns of the [dk_0 .. dk_{M-1} | dv] row, and
// the shared v's gradient sum_m alpha_m dvt_m gathers in an fp32 buffer that
// the last branch rounds into the row (dv_mode).
#include <type_traits>

#include "kernels.h"

namespace engram {

// Where the conv weights and the tap sums live: 0 registers; 1 LDS in the
// 1024-lane variants; 2 also in the 768-lane multi-branch variants (the
// shapes whose registers run out; the others keep them in registers)
#ifndef ENGRAM_BW_LDS
#define ENGRAM_BW_LDS 2
#endif

constexpr int kBwTokens = 64;   // R
constexpr int kBwBatch = 8;     // tokens per dalpha reduction batch
constexpr int kBwMaxWaves = 16; // d / 4 / 64
// dv of this launch: written (one branch), or gathered over the branches
enum { kDvDirect = 0, kDvFirst = 1, kDvAdd = 2, kDvLast = 3 };

template <bool BF16>
using raw4_t = typename std::conditional<BF16, u32x2, u32x4>::type;

template <bool BF16>
__device__ inline raw4_t<BF16> ld4_raw(const uint8_t* base, int64_t elem) {
  return *reinterpret_cast<const raw4_t<BF16>*>(base + elem * (BF16 ? 2 : 4));
}
template <bool BF16>
__device__ inline void widen4(const raw4_t<BF16> u, float* out) {
  if constexpr (BF16) {
    out[0] = __uint_as_float(u[0] << 16);
    out[1] = __uint_as_float(u[0] & 0xFFFF0000u);
    out[2] = __uint_as_float(u[1] << 16);
    out[3] = __uint_as_float(u[1] & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = __uint_as_float(u[c]);
  }
}

// fp16 (for the fp16 GEMM) or fp32 store of 4 values
template <bool BF16>
__device__ inline void st4_grad(uint8_t* base, int64_t elem, const float* v) {
  if constexpr (BF16) {
    typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
    halfx4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<halfx4*>(base + elem * 2) = h;
  } else {
    *reinterpret_cast<floatx4*>(base + elem * 4) = floatx4{v[0], v[1], v[2], v[3]};
  }
}

// bf16 (round to nearest even) or fp32 store of 4 values in the io dtype
template <bool BF16>
__device__ inline void st4_io(uint8_t* base, int64_t elem, const float* v) {
  if constexpr (BF16) {
    *reinterpret_cast<u32x2*>(base + elem * 2) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  } else {
    *reinterpret_cast<floatx4*>(base + elem * 4) = floatx4{v[0], v[1], v[2], v[3]};
  }
}

// p[0..7]: this lane's shares of 8 tokens.  Returns the wave-wide sum of
// token 4*b5 + 2*b4 + b3 (b = lane bits): each halving step sends the half
// of the values that the partner keeps.
__device__ inline float wave_sum8(float p[8], int lane) {
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
  float q[4], r[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float send = b5 ? p[k] : p[k + 4];
    const float keep = b5 ? p[k + 4] : p[k];
    q[k] = keep + __shfl_xor(send, 32);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float send = b4 ? q[k] : q[k + 2];
    const float keep = b4 ? q[k + 2] : q[k];
    r[k] = keep + __shfl_xor(send, 16);
  }
  float x = (b3 ? r[1] : r[0]) + __shfl_xor(b3 ? r[0] : r[1], 8);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 1);
  return x;
}

// MAXT: the largest block it is launched with.  One workgroup of d/4 lanes
// fits a CU at d = 2560 whatever the register count up to 168, and the
// parameter sums need more than the 128 that 1024 threads leave.
// MULTI: one of several branches (dv gathers in dv_acc); else dv is written.
template <bool BF16, int TAPS, bool PARAMS, int MAXT, bool MULTI>
__global__ __launch_bounds__(MAXT) void bwd_gate_conv_kernel(BwdArgs a) {
  constexpr int R = kBwTokens;
  constexpr int NH = TAPS - 1;
  constexpr int NW = NH > 0 ? NH : 1;
  constexpr int PD = TAPS <= 4 ? 4 : (TAPS <= 6 ? 2 : 1);  // tokens of v / G loaded ahead
  static_assert(R % kBwBatch == 0, "");
  __shared__ floatx4 st_s[R + 2 * NH + PD];
  __shared__ float pdw[R][kBwMaxWaves];
  __shared__ float dal_s[R];
  __shared__ float sc_s[R];  // the tokens' fp16 range factors (1 without)
  // With 1024 lanes (128 registers each), and in the multi-branch variants,
  // the conv weights and the tap sums live in LDS, one slot per lane, read
  // and updated where they are used: held in registers they made the kernel
  // spill, and every reload from scratch waited for the whole ring of v / G
  // loads.  Same arithmetic in the same order, so the same results.
  constexpr bool kLdsW = ENGRAM_BW_LDS && (MAXT > 768 || (ENGRAM_BW_LDS > 1 && MULTI)) &&
                         TAPS * 4 * MAXT * 4 * (PARAMS ? 2 : 1) <= 136 * 1024;
  __shared__ float w_s[kLdsW ? TAPS * 4 * MAXT : 1];               // [i][c][lane]
  __shared__ float dcw_s[kLdsW && PARAMS ? TAPS * 4 * MAXT : 1];   // [i][c][lane]
  const int64_t b = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * R;
  const int d = a.d;
  const int64_t T = a.T;
  const float inv_d = 1.0f / (float)d;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  for (int i = threadIdx.x; i < R + 2 * NH + PD; i += blockDim.x) {
    const int64_t u = t0 - NH + i;
    st_s[i] = (u >= 0 && u < T) ? *reinterpret_cast<const floatx4*>(a.stats + (b * T + u) * 4)
                                : floatx4{0.f, 0.f, 0.f, 0.f};
  }
  for (int i = threadIdx.x; i < R; i += blockDim.x)
    sc_s[i] = a.scale && t0 + i < T ? a.scale[b * T + t0 + i] : 1.f;
  __syncthreads();

  const int f = threadIdx.x * 4;  // blockDim.x * 4 == d
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  const int64_t row0 = b * T;
  const int64_t tend = t0 + R < T ? t0 + R : T;  // tokens [t0, tend) are this block's
  // elements of a [dk_0 .. | dv] row, and where this launch's dk and the dv sit in it
  const int64_t ld = MULTI ? (int64_t)(a.branches + 1) * d : 2 * (int64_t)d;
  const int dk_col = MULTI ? a.branch * d : 0;
  const int dv_col = MULTI ? a.branches * d : d;
  float w[kLdsW ? 1 : 4][kLdsW ? 1 : TAPS];
  // a lane's own LDS slot (written and read by that lane only)
  auto lslot = [&](float* arr, int c, int i) __attribute__((always_inline)) -> float* {
    return reinterpret_cast<float*>(arr) + (i * 4 + c) * MAXT + threadIdx.x;
  };
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < TAPS; ++i) {
      const float x = a.conv_w[(f + c) * TAPS + i];
      if constexpr (kLdsW)
        *lslot(w_s, c, i) = x;
      else
        w[c][i] = x;
    }
  auto W = [&](int c, int i) __attribute__((always_inline)) -> float {
    if constexpr (kLdsW)
      return *lslot(w_s, c, i);
    else
      return w[c][i];
  };
  // the weights' loads before the ring's, so that none of them is pending at
  // the loop head (one would make every iteration wait for the whole ring)
  __builtin_amdgcn_sched_barrier(0);

  // ---- pass A
  float vtw[NW][4];  // gated value at u-1-i
  float dzw[TAPS][4];  // dz at u-i
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int i = 0; i < NW; ++i) vtw[i][c] = 0.f;
#pragma unroll
    for (int i = 0; i < TAPS; ++i) dzw[i][c] = 0.f;
  }
  const int64_t ubeg = t0 - NH;
  // Ring of raw v / G rows: token u sits in slot (u - ubeg) % RS from its
  // load at step u - PD until finish at step u + NH (RS > PD + NH).  The
  // loads are unconditional, the row clamped into [0, T), so that the
  // compiler counts them in flight instead of draining the ring: outside
  // [0, T) the gate is zero, and G enters only tokens in [t0, T).
  constexpr int RS = (PD + NH + 1 <= 8) ? 8 : 16;
  static_assert(RS % kBwBatch == 0 && R % RS == 0, "");
  raw4_t<BF16> rv[RS], rg[RS];
  auto fetch = [&](int64_t u, raw4_t<BF16>& v, raw4_t<BF16>& g) __attribute__((always_inline)) {
    const int64_t uc = u < 0 ? 0 : (u < T ? u : T - 1);
    v = ld4_raw<BF16>(a.v, (row0 + uc) * d + f);
    g = ld4_raw<BF16>(a.dy, (row0 + uc) * d + f);
  };
#pragma unroll
  for (int k = 0; k < PD; ++k) fetch(ubeg + k, rv[k], rg[k]);
  float pb[kBwBatch];
#pragma unroll
  for (int k = 0; k < kBwBatch; ++k) pb[k] = 0.f;
  // PARAMS: sum over this block's tokens of dz_u vt_{u-i} (tap i); written
  // out after pass A
  float dcw[PARAMS && !kLdsW ? 4 : 1][PARAMS && !kLdsW ? TAPS : 1];
  if constexpr (PARAMS) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < TAPS; ++i) {
        if constexpr (kLdsW)
          *lslot(dcw_s, c, i) = 0.f;
        else
          dcw[c][i] = 0.f;
      }
  }
  auto dcw_add = [&](int c, int i, float x) __attribute__((always_inline)) {
    if constexpr (kLdsW) {
      float* q = lslot(dcw_s, c, i);
      *q = *q + x;
    } else {
      dcw[c][i] += x;
    }
  };
  float* const pdst = PARAMS && a.pacc ? a.pacc + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) *
                                                      d * (TAPS + 1) + (int64_t)f * (TAPS + 1)
                                       : nullptr;

  // one step of pass A at u (slot k = (u - ubeg) % RS, compile-time)
  auto step = [&](int64_t u, int k) __attribute__((always_inline)) {
    fetch(u + PD, rv[(k + PD) % RS], rg[(k + PD) % RS]);
    float v[4], G[4];
    widen4<BF16>(rv[k], v);
    widen4<BF16>(rg[k], G);
    const float al = st_s[u - ubeg][0];
    float vt[4], dz[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) vt[c] = al * v[c];
    const bool live = u >= t0 && u < T;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float z = W(c, 0) * vt[c];
#pragma unroll
      for (int i = 1; i < TAPS; ++i) z += W(c, i) * vtw[i - 1][c];
      const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
      dz[c] = live ? G[c] * sg * (1.0f + z * (1.0f - sg)) : 0.f;
    }
    if constexpr (PARAMS) {
      // u's own tokens only: u in [tend, tend + NH) belongs to the next block
      if (u < tend) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          dcw_add(c, 0, dz[c] * vt[c]);
#pragma unroll
          for (int i = 1; i < TAPS; ++i) dcw_add(c, i, dz[c] * vtw[i - 1][c]);
        }
      }
    }
#pragma unroll
    for (int i = TAPS - 1; i > 0; --i)
#pragma unroll
      for (int c = 0; c < 4; ++c) dzw[i][c] = dzw[i - 1][c];
#pragma unroll
    for (int c = 0; c < 4; ++c) dzw[0][c] = dz[c];
#pragma unroll
    for (int i = NW - 1; i > 0; --i)
#pragma unroll
      for (int c = 0; c < 4; ++c) vtw[i][c] = vtw[i - 1][c];
    if (NH > 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) vtw[0][c] = vt[c];
    }
  };
  // token t = u - NH (slot kt) is final after step(u): dv_t out, its dalpha
  // share into pb[pslot]
  auto finish = [&](int64_t t, int kt, int pslot) __attribute__((always_inline)) {
    if (t >= tend) return;  // uniform
    float v[4], G[4];
    widen4<BF16>(rv[kt], v);
    widen4<BF16>(rg[kt], G);
    const float alpha = st_s[t - ubeg][0];
    float dv[4], pd = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float acc = G[c];
#pragma unroll
      for (int i = 0; i < TAPS; ++i) acc += W(c, i) * dzw[NH - i][c];
      pd += acc * v[c];
      dv[c] = alpha * acc;
    }
    pb[pslot] = pd;
    const float sc = sc_s[t - t0];  // the token's fp16 range factor
    if constexpr (!MULTI) {
#pragma unroll
      for (int c = 0; c < 4; ++c) dv[c] *= sc;
      st4_grad<BF16>(a.dkv, (row0 + t) * ld + dv_col + f, dv);
    } else {
      floatx4* acc = reinterpret_cast<floatx4*>(a.dv_acc + (row0 + t) * d + f);
      if (a.dv_mode == kDvFirst) {
        *acc = floatx4{dv[0], dv[1], dv[2], dv[3]};
      } else {
        const floatx4 prev = *acc;
#pragma unroll
        for (int c = 0; c < 4; ++c) dv[c] += prev[c];
        if (a.dv_mode == kDvAdd) {
          *acc = floatx4{dv[0], dv[1], dv[2], dv[3]};
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) dv[c] *= sc;
          st4_grad<BF16>(a.dkv, (row0 + t) * ld + dv_col + f, dv);
        }
      }
    }
  };

  // warm-up: u = t0-NH .. t0+NH-1 (no token final yet)
#pragma unroll
  for (int k = 0; k < 2 * NH; ++k) step(ubeg + k, k % RS);
  for (int tb = 0; tb < R; tb += RS) {
#pragma unroll
    for (int k = 0; k < RS; ++k) {
      // u = t0 + NH + tb + k, slot (2NH + tb + k) % RS; token t = t0 + tb + k
      const int64_t u = t0 + NH + tb + k;
      step(u, (2 * NH + k) % RS);
      finish(u - NH, (NH + k) % RS, k % kBwBatch);
      if (k % kBwBatch == kBwBatch - 1) {
        const float s8 = wave_sum8(pb, lane);
        if ((lane & 7) == 0) pdw[tb + (k - (kBwBatch - 1)) + ((lane >> 3) & 7)][wave] = s8;
#pragma unroll
        for (int q = 0; q < kBwBatch; ++q) pb[q] = 0.f;
      }
    }
  }
  if constexpr (PARAMS) {
    if (pdst) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < TAPS; ++i) {
          if constexpr (kLdsW)
            pdst[c * (TAPS + 1) + i] = *lslot(dcw_s, c, i);
          else
            pdst[c * (TAPS + 1) + i] = dcw[c][i];
        }
    }
  }
  __syncthreads();
  if (threadIdx.x < R) {
    float s = 0.f;
    for (int i = 0; i < nwaves; ++i) s += pdw[threadIdx.x][i];
    dal_s[threadIdx.x] = s;
  }
  __syncthreads();

  // ---- pass B: dk from h, k and the summed dalpha
  float gqk[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    gqk[c] = (a.gamma_q ? a.gamma_q[f + c] : 1.f) * (a.gamma_k ? a.gamma_k[f + c] : 1.f);
  float sgs[PARAMS ? 4 : 1];  // PARAMS: sum over tokens of ca h k
  if constexpr (PARAMS) {
#pragma unroll
    for (int c = 0; c < 4; ++c) sgs[c] = 0.f;
  }
  constexpr int UB = 4;
  for (int i0 = 0; i0 < R; i0 += UB) {
    raw4_t<BF16> rh[UB], rk[UB];
#pragma unroll
    for (int q = 0; q < UB; ++q) {
      const int64_t t = t0 + i0 + q < tend ? t0 + i0 + q : tend - 1;  // unconditional, clamped
      rh[q] = ld4_raw<BF16>(a.h, (row0 + t) * d + f);
      rk[q] = ld4_raw<BF16>(a.k, (row0 + t) * d + f);
    }
#pragma unroll
    for (int q = 0; q < UB; ++q) {
      const int64_t t = t0 + i0 + q;
      if (t >= tend) break;
      const floatx4 st = st_s[t - ubeg];
      const float alpha = st[0], rq = st[1], rkk = st[2], P = st[3];
      const float ds = dal_s[i0 + q] * alpha * (1.0f - alpha);
      const float ca = ds * rq * rkk * inv_sqrt_d;
      const float cb = rkk * rkk * rkk * ds * rq * P * inv_sqrt_d * inv_d;
      float hv[4], kv[4], dk[4];
      widen4<BF16>(rh[q], hv);
      widen4<BF16>(rk[q], kv);
      const float sc = sc_s[i0 + q];
#pragma unroll
      for (int c = 0; c < 4; ++c) dk[c] = ca * gqk[c] * hv[c] - cb * kv[c];
      float dks[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) dks[c] = dk[c] * sc;
      st4_grad<BF16>(a.dkv, (row0 + t) * ld + dk_col + f, dks);
      if constexpr (PARAMS) {
        const float cq = rq * rq * rq * ds * rkk * P * inv_sqrt_d * inv_d;
        float dh[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          dh[c] = ca * gqk[c] * kv[c] - cq * hv[c];
          sgs[c] += ca * hv[c] * kv[c];
        }
        if (a.dh) st4_io<BF16>(a.dh, (row0 + t) * d + f, dh);
      }
    }
  }
  if constexpr (PARAMS) {
    if (pdst) {
#pragma unroll
      for (int c = 0; c < 4; ++c) pdst[c * (TAPS + 1) + TAPS] = sgs[c];
    }
    // zero rows after the last token, for the weight-gradient GEMM's last stage
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      const float z4[4] = {0.f, 0.f, 0.f, 0.f};
      const int64_t N = a.B * T;
      for (int r = 0; r < a.pad_rows; ++r)
        for (int c = 0; c <= (MULTI ? a.branches : 1); ++c)
          st4_grad<BF16>(a.dkv, (N + r) * ld + c * d + f, z4);
    }
  }
}

template <bool BF16, bool PARAMS, int MAXT, bool MULTI>
static hipError_t launch_bwd_taps(const BwdArgs& a, dim3 grid, int threads, hipStream_t s) {
  switch (a.taps) {
#define ENGRAM_TAPS_CASE(K)                                                                 \
  case K:                                                                                   \
    hipLaunchKernelGGL((bwd_gate_conv_kernel<BF16, K, PARAMS, MAXT, MULTI>), grid,         \
                       dim3(threads), 0, s, a);                                             \
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

hipError_t launch_bwd_gate_conv(const BwdArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  // one lane per 4 features, whole waves: d is a multiple of 256
  if (a.d % 256 != 0 || a.d / 4 > 64 * kBwMaxWaves) return hipErrorInvalidValue;
  const int threads = a.d / 4;
  dim3 grid((unsigned)((a.T + kBwTokens - 1) / kBwTokens), (unsigned)a.B);
  const bool params = a.pacc || a.dh || a.pad_rows > 0;
  if (a.pad_rows < 0 || a.pad_rows > 64) return hipErrorInvalidValue;
  if (a.branches < 1 || a.branch < 0 || a.branch >= a.branches || a.dv_mode < kDvDirect ||
      a.dv_mode > kDvLast || (a.dv_mode != kDvDirect && !a.dv_acc) ||
      (a.dv_mode == kDvDirect && a.branches != 1))
    return hipErrorInvalidValue;
  const bool narrow = threads <= 768;
  const bool multi = a.dv_mode != kDvDirect;
  if (a.io_dtype == ENGRAM_BF16) {
    if (multi) {
      if (!params) return narrow ? launch_bwd_taps<true, false, 768, true>(a, grid, threads, s)
                                 : launch_bwd_taps<true, false, 1024, true>(a, grid, threads, s);
      return narrow ? launch_bwd_taps<true, true, 768, true>(a, grid, threads, s)
                    : launch_bwd_taps<true, true, 1024, true>(a, grid, threads, s);
    }
    if (!params) return narrow ? launch_bwd_taps<true, false, 768, false>(a, grid, threads, s)
                               : launch_bwd_taps<true, false, 1024, false>(a, grid, threads, s);
    return narrow ? launch_bwd_taps<true, true, 768, false>(a, grid, threads, s)
                  : launch_bwd_taps<true, true, 1024, false>(a, grid, threads, s);
  }
  if (multi) {
    if (!params) return narrow ? launch_bwd_taps<false, false, 768, true>(a, grid, threads, s)
                               : launch_bwd_taps<false, false, 1024, true>(a, grid, threads, s);
    return narrow ? launch_bwd_taps<false, true, 768, true>(a, grid, threads, s)
                  : launch_bwd_taps<false, true, 1024, true>(a, grid, threads, s);
  }
  if (!params) return narrow ? launch_bwd_taps<false, false, 768, false>(a, grid, threads, s)
                             : launch_bwd_taps<false, false, 1024, false>(a, grid, threads, s);
  return narrow ? launch_bwd_taps<false, true, 768, false>(a, grid, threads, s)
                : launch_bwd_taps<false, true, 1024, false>(a, grid, threads, s);
}

int64_t bwd_blocks(int64_t B, int64_t T) { return B * ((T + kBwTokens - 1) / kBwTokens); }

// ------------------------------------------------------------- fp16 range
// The de and dW contractions take [dk_t | dv_t] in fp16, whose range (normal
// numbers from 2^-14 to 65504) the gradients of a loss can leave at either
// end.  Each token's row is stored times s_t = 2^E_t, chosen from an upper
// bound b_t of |dk_t|, |dv_t| so that b_t s_t < 2^14, and the factor is
// taken out again where it is exact (the de epilogue, e_t / s_t in bf16).
// The bound follows the chain rule of bwd_gate_conv_kernel, with
// m_u = max |G_u|, M_t = max_{t <= u <= t+taps-1} m_u, W = max_c sum_i |w[c][i]|
// and |dz| <= 1.1 |G| (SiLU' lies in (-0.1, 1.1)):
//   |dvt_t|   <= (1 + 1.1 W) M_t
//   |dv_t|    <= sum over branches of alpha_t (1 + 1.1 W) M_t
//   |dalpha_t| <= ||dvt_t||_2 ||v_t||_2 <= sqrt(d) (1 + 1.1 W) M_t ||v_t||_2
//   |ds_t|    = alpha (1 - alpha) |dalpha_t|
//   |dk_t|    <= |ds_t| rk (Gamma + rk rq |P| / d), Gamma = max_c |g_q g_k|,
// using |h| <= ||h||_2 <= sqrt(d) / rq and |k| <= sqrt(d) / rk.
__device__ inline float pow2_scale_for(float bound) {
  if (!(bound > 0.f) || !(bound <= 3.0e38f)) return 1.f;
  // bound < 2^e with e = (biased exponent) - 126 (normal bound); subnormal: e = -125
  const int ex = (int)((__float_as_uint(bound) >> 23) & 0xFFu);
  const int e = ex > 0 ? ex - 126 : -125;
  int E = 14 - e;
  E = E < -96 ? -96 : (E > 96 ? 96 : E);
  return __uint_as_float((uint32_t)(127 + E) << 23);
}

__device__ inline float wave_max_all(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum_all(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

constexpr int kScTok = 64;  // tokens of a sequence per workgroup
__global__ __launch_bounds__(256) void bwd_scale_kernel(BwdScaleArgs a) {
  constexpr int kMaxHalo = 7;
  __shared__ float mx[ENGRAM_MAX_BRANCHES][kScTok + kMaxHalo];
  __shared__ float vn2[kScTok];
  __shared__ float red[4][1 + ENGRAM_MAX_BRANCHES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = blockIdx.y, t0 = (int64_t)blockIdx.x * kScTok, T = a.T;
  const int d = a.d, taps = a.taps, NH = taps - 1, M = a.branches;
  const int64_t N = a.B * T, row0 = b * T;
  // W and Gamma_m over all features
  float wl = 0.f, gl[ENGRAM_MAX_BRANCHES];
  for (int m = 0; m < ENGRAM_MAX_BRANCHES; ++m) gl[m] = 0.f;
  for (int c = tid; c < d; c += 256) {
    float sw = 0.f;
    for (int i = 0; i < taps; ++i) sw += fabsf(a.conv_w[(int64_t)c * taps + i]);
    wl = fmaxf(wl, sw);
    for (int m = 0; m < M; ++m) {
      const float g = (a.gamma_q ? a.gamma_q[(int64_t)m * d + c] : 1.f) *
                      (a.gamma_k ? a.gamma_k[(int64_t)m * d + c] : 1.f);
      gl[m] = fmaxf(gl[m], fabsf(g));
    }
  }
  wl = wave_max_all(wl);
  for (int m = 0; m < M; ++m) gl[m] = wave_max_all(gl[m]);
  if (lane == 0) {
    red[wave][0] = wl;
    for (int m = 0; m < M; ++m) red[wave][1 + m] = gl[m];
  }
  // per-token maxima of |G| (with the halo after the block) and sums of v^2
  const int64_t tend = t0 + kScTok < T ? t0 + kScTok : T;
  const int64_t hend = t0 + kScTok + NH < T ? t0 + kScTok + NH : T;
  const int nu = (int)(hend - t0), nv = (int)(tend - t0);
  const int pieces = d / 8;  // 16-byte pieces of a bf16 row
  for (int it = wave; it < M * nu + nv; it += 4) {
    const bool is_g = it < M * nu;
    const int m = is_g ? it / nu : 0;
    const int u = is_g ? it - m * nu : it - M * nu;
    const uint8_t* row = is_g ? a.dy + ((int64_t)m * N + row0 + t0 + u) * d * 2
                              : a.v + (row0 + t0 + u) * d * 2;
    float acc = 0.f;
    for (int p = lane; p < pieces; p += 64) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(row + p * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = __uint_as_float(q[i] << 16), x1 = __uint_as_float(q[i] & 0xFFFF0000u);
        if (is_g)
          acc = fmaxf(acc, fmaxf(fabsf(x0), fabsf(x1)));
        else
          acc += x0 * x0 + x1 * x1;
      }
    }
    if (is_g) {
      acc = wave_max_all(acc);
      if (lane == 0) mx[m][u] = acc;
    } else {
      acc = wave_sum_all(acc);
      if (lane == 0) vn2[u] = acc;
    }
  }
  __syncthreads();
  if (tid >= nv) return;
  const float W = fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0]));
  const float wf = 1.f + 1.1f * W;
  const float sqd = sqrtf((float)d), inv_d = 1.f / (float)d;
  const float vn = sqrtf(vn2[tid]);
  float dvb = 0.f, dkb = 0.f;
  for (int m = 0; m < M; ++m) {
    float Mt = 0.f;
    for (int i = 0; i <= NH && tid + i < nu; ++i) Mt = fmaxf(Mt, mx[m][tid + i]);
    const float G = fmaxf(fmaxf(red[0][1 + m], red[1][1 + m]), fmaxf(red[2][1 + m], red[3][1 + m]));
    const floatx4 st = *reinterpret_cast<const floatx4*>(a.stats + ((int64_t)m * N + row0 + t0 + tid) * 4);
    const float al = st[0], rq = st[1], rk = st[2], P = st[3];
    dvb += al * wf * Mt;
    const float dsb = al * (1.f - al) * sqd * wf * Mt * vn;
    dkb = fmaxf(dkb, dsb * rk * (G + rk * rq * fabsf(P) * inv_d));
  }
  // 1.01: rounding in the kernels' fp32 sums stays far inside the 4x left to 65504
  a.scale[row0 + t0 + tid] = pow2_scale_for(1.01f * fmaxf(dvb, dkb));
}

hipError_t launch_bwd_scale(const BwdScaleArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  if (a.d % 8 != 0 || a.taps < 1 || a.taps > 8 || a.branches < 1 || a.branches > ENGRAM_MAX_BRANCHES)
    return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.T + kScTok - 1) / kScTok), (unsigned)a.B);
  hipLaunchKernelGGL(bwd_scale_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// rows of e divided by their token's scale (a power of two: exact in bf16)
__global__ __launch_bounds__(256) void scale_rows_kernel(const uint8_t* __restrict__ e,
                                                         const float* __restrict__ scale,
                                                         uint64_t pieces, int32_t row_pieces,
                                                         uint8_t* __restrict__ out) {
  const uint64_t c = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= pieces) return;
  const float inv = pow2_inverse(scale[c / (uint64_t)row_pieces]);
  u32x4 q = *(reinterpret_cast<const u32x4*>(e) + c);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    q[i] = pack_bf16x2(__uint_as_float(q[i] << 16) * inv, __uint_as_float(q[i] & 0xFFFF0000u) * inv);
  *(reinterpret_cast<u32x4*>(out) + c) = q;
}

hipError_t launch_scale_rows_bf16(const uint8_t* e, const float* scale, int64_t N, int32_t cols,
                                  uint8_t* out, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (cols % 8 != 0) return hipErrorInvalidValue;
  const uint64_t pieces = (uint64_t)N * (cols / 8);
  hipLaunchKernelGGL(scale_rows_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, e,
                     scale, pieces, cols / 8, out);
  return hipGetLastError();
}

// ------------------------------------------------------------- parameter sums
// dst[c][e] = sum of src rows c*64 .. c*64+63 (< rows) in column e, in order
__global__ __launch_bounds__(256) void colsum64_kernel(const float* __restrict__ src,
                                                       float* __restrict__ dst, int64_t rows,
                                                       int64_t cols) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int64_t r1 = r0 + 64 < rows ? r0 + 64 : rows;
  float acc = 0.f;
  for (int64_t r = r0; r < r1; ++r) acc += src[r * cols + e];
  dst[(int64_t)blockIdx.y * cols + e] = acc;
}

// sums [d][taps+1] -> dconv [d][taps], dgq = g_k S, dgk = g_q S
__global__ __launch_bounds__(256) void param_finish_kernel(const float* __restrict__ sums, int32_t d,
                                                           int32_t taps, const float* gamma_q,
                                                           const float* gamma_k, float* dconv,
                                                           float* dgq, float* dgk) {
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= d) return;
  const float* sf = sums + (int64_t)f * (taps + 1);
  if (dconv)
    for (int i = 0; i < taps; ++i) dconv[(int64_t)f * taps + i] = sf[i];
  const float S = sf[taps];
  if (dgq) dgq[f] = (gamma_k ? gamma_k[f] : 1.f) * S;
  if (dgk) dgk[f] = (gamma_q ? gamma_q[f] : 1.f) * S;
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

int64_t bwd_param_tmp_floats(int64_t nblk, int32_t d, int32_t taps) {
  const int64_t cols = (int64_t)d * (taps + 1);
  int64_t rows = nblk, total = 0;
  while (rows > 1) {
    rows = (rows + 63) / 64;
    total += rows * cols;
  }
  return total;
}

hipError_t launch_bwd_param_sums(const float* pacc, float* tmp, int64_t nblk, int32_t d,
                                 int32_t taps, const float* gamma_q, const float* gamma_k,
                                 float* dconv, float* dgq, float* dgk, hipStream_t s) {
  if (nblk <= 0) return hipErrorInvalidValue;
  const int64_t cols = (int64_t)d * (taps + 1);
  // passes of 64-row sums, each into a fresh region of tmp, until one row is left
  const float* src = pacc;
  float* dst = tmp;
  int64_t rows = nblk;
  while (rows > 1) {
    const int64_t groups = (rows + 63) / 64;
    if (groups > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(colsum64_kernel, dim3((unsigned)((cols + 255) / 256), (unsigned)groups),
                       dim3(256), 0, s, src, dst, rows, cols);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    src = dst;
    dst += groups * cols;
    rows = groups;
  }
  hipLaunchKernelGGL(param_finish_kernel, dim3((unsigned)((d + 255) / 256)), dim3(256), 0, s, src,
                     d, taps, gamma_q, gamma_k, dconv, dgq, dgk);
  return hipGetLastError();
}

// ------------------------------------------------------------- W transpose
// W_kv [rows = 2d][cols = d_mem] -> Wt [d_mem][2d]: fp16 from bf16 (exact for
// |w| >= 2^-14, the fp16 normal range) or fp32 from fp32.
template <bool BF16>
__global__ __launch_bounds__(256) void transpose_w_kernel(const uint8_t* __restrict__ w,
                                                          uint8_t* __restrict__ wt, int rows,
                                                          int cols) {
  __shared__ float tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  for (int i = threadIdx.y; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + threadIdx.x;
    float x = 0.f;
    if (r < rows && c < cols) {
      const int64_t e = (int64_t)r * cols + c;
      x = BF16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(w)[e])
               : reinterpret_cast<const float*>(w)[e];
    }
    tile[i][threadIdx.x] = x;
  }
  __syncthreads();
  for (int i = threadIdx.y; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + threadIdx.x;
    if (c < cols && r < rows) {
      const int64_t e = (int64_t)c * rows + r;
      if (BF16)
        reinterpret_cast<_Float16*>(wt)[e] = (_Float16)tile[threadIdx.x][i];
      else
        reinterpret_cast<float*>(wt)[e] = tile[threadIdx.x][i];
    }
  }
}

hipError_t launch_transpose_w(const uint8_t* w, uint8_t* wt, int32_t rows, int32_t cols,
                              int32_t io_dtype, hipStream_t s) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32), block(32, 8);
  if (io_dtype == ENGRAM_BF16)
    hipLaunchKernelGGL(transpose_w_kernel<true>, grid, block, 0, s, w, wt, rows, cols);
  else
    hipLaunchKernelGGL(transpose_w_kernel<false>, grid, block, 0, s, w, wt, rows, cols);
  return hipGetLastError();
}

}  // namespace engram
