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
// cb).  One workgroup owns R tokens and all d features of one sequence and
// walks u = t0-taps+1 .. t0+R+taps-2, keeping the last taps values of v, G,
// dz and the gated value in registers; each output token needs one
// workgroup-wide sum (dalpha).  dk and dv leave as fp16 (bf16 io) or fp32
// (fp32 io): the operands of the de GEMM.
#include "kernels.h"

namespace engram {

constexpr int kBwTokens = 32;

template <bool BF16>
__device__ inline void ld4(const uint8_t* base, int64_t elem, float* out) {
  if constexpr (BF16) {
    const u32x2 u = *reinterpret_cast<const u32x2*>(base + elem * 2);
    out[0] = __uint_as_float(u[0] << 16);
    out[1] = __uint_as_float(u[0] & 0xFFFF0000u);
    out[2] = __uint_as_float(u[1] << 16);
    out[3] = __uint_as_float(u[1] & 0xFFFF0000u);
  } else {
    const floatx4 f = *reinterpret_cast<const floatx4*>(base + elem * 4);
    out[0] = f[0];
    out[1] = f[1];
    out[2] = f[2];
    out[3] = f[3];
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

template <bool BF16, int TAPS>
__global__ __launch_bounds__(1024) void bwd_gate_conv_kernel(BwdArgs a) {
  constexpr int R = kBwTokens;
  constexpr int NH = TAPS - 1;
  __shared__ floatx4 st_s[R + 2 * NH + 1];
  __shared__ float red[16];
  const int64_t b = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * R;
  const int d = a.d;
  const int64_t T = a.T;
  const float inv_d = 1.0f / (float)d;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  for (int i = threadIdx.x; i < R + 2 * NH; i += blockDim.x) {
    const int64_t u = t0 - NH + i;
    st_s[i] = (u >= 0 && u < T) ? *reinterpret_cast<const floatx4*>(a.stats + (b * T + u) * 4)
                                : floatx4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();

  const int f = threadIdx.x * 4;
  const bool act = f < d;
  const int fc = act ? f : 0;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nwaves = (blockDim.x + 63) >> 6;
  float w[4][TAPS], gqk[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int i = 0; i < TAPS; ++i) w[c][i] = a.conv_w[(fc + c) * TAPS + i];
    gqk[c] = (a.gamma_q ? a.gamma_q[fc + c] : 1.f) * (a.gamma_k ? a.gamma_k[fc + c] : 1.f);
  }
  float vtw[NH > 0 ? NH : 1][4];  // gated value at u-1-i
  float vw[TAPS][4], Gw[TAPS][4], dzw[TAPS][4];  // at u-i
#pragma unroll
  for (int i = 0; i < TAPS; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      vw[i][c] = Gw[i][c] = dzw[i][c] = 0.f;
      if (i < NH) vtw[i][c] = 0.f;
    }
  const int64_t row0 = b * T;
  for (int64_t u = t0 - NH; u < t0 + R + NH; ++u) {
    const bool in = u >= 0 && u < T;
    float v[4] = {0.f, 0.f, 0.f, 0.f}, G[4] = {0.f, 0.f, 0.f, 0.f};
    if (in && act) {
      ld4<BF16>(a.v, (row0 + u) * d + fc, v);
      if (u >= t0) ld4<BF16>(a.dy, (row0 + u) * d + fc, G);
    }
    const float al = st_s[u - (t0 - NH)][0];
    float vt[4], dz[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) vt[c] = al * v[c];
    if (in && u >= t0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float z = w[c][0] * vt[c];
#pragma unroll
        for (int i = 1; i < TAPS; ++i) z += w[c][i] * vtw[i - 1][c];
        const float sg = 1.0f / (1.0f + expf(-z));
        dz[c] = G[c] * sg * (1.0f + z * (1.0f - sg));
      }
    }
#pragma unroll
    for (int i = TAPS - 1; i > 0; --i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        vw[i][c] = vw[i - 1][c];
        Gw[i][c] = Gw[i - 1][c];
        dzw[i][c] = dzw[i - 1][c];
      }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      vw[0][c] = v[c];
      Gw[0][c] = G[c];
      dzw[0][c] = dz[c];
    }
#pragma unroll
    for (int i = NH - 1; i > 0; --i)
#pragma unroll
      for (int c = 0; c < 4; ++c) vtw[i][c] = vtw[i - 1][c];
    if (NH > 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) vtw[0][c] = vt[c];
    }

    const int64_t t = u - NH;  // token whose dz_{t..t+NH} are now all known
    if (t < t0 || t >= T) continue;  // uniform over the workgroup
    float dvt[4];
    float pd = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float acc = Gw[NH][c];
#pragma unroll
      for (int i = 0; i < TAPS; ++i) acc += w[c][i] * dzw[NH - i][c];
      dvt[c] = acc;
      pd += acc * vw[NH][c];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) pd += __shfl_xor(pd, o);
    if (lane == 0) red[wave] = pd;
    __syncthreads();
    float dalpha = 0.f;
    for (int i = 0; i < nwaves; ++i) dalpha += red[i];
    __syncthreads();
    if (!act) continue;
    const floatx4 st = st_s[t - (t0 - NH)];
    const float alpha = st[0], rq = st[1], rk = st[2], P = st[3];
    const float ds = dalpha * alpha * (1.0f - alpha);
    const float ca = ds * rq * rk * inv_sqrt_d;
    const float cb = rk * rk * rk * ds * rq * P * inv_sqrt_d * inv_d;
    float hv[4], kv[4], dk[4], dv[4];
    ld4<BF16>(a.h, (row0 + t) * d + fc, hv);
    ld4<BF16>(a.k, (row0 + t) * d + fc, kv);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      dk[c] = ca * gqk[c] * hv[c] - cb * kv[c];
      dv[c] = alpha * dvt[c];
    }
    st4_grad<BF16>(a.dkv, (row0 + t) * 2 * d + fc, dk);
    st4_grad<BF16>(a.dkv, (row0 + t) * 2 * d + d + fc, dv);
  }
}

template <bool BF16>
static hipError_t launch_bwd_taps(const BwdArgs& a, dim3 grid, int threads, hipStream_t s) {
  switch (a.taps) {
#define ENGRAM_TAPS_CASE(K)                                                               \
  case K:                                                                                 \
    hipLaunchKernelGGL((bwd_gate_conv_kernel<BF16, K>), grid, dim3(threads), 0, s, a); \
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
  const int threads = (a.d / 4 + 63) / 64 * 64;
  if (threads > 1024) return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.T + kBwTokens - 1) / kBwTokens), (unsigned)a.B);
  return a.io_dtype == ENGRAM_BF16 ? launch_bwd_taps<true>(a, grid, threads, s)
                                   : launch_bwd_taps<false>(a, grid, threads, s);
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
