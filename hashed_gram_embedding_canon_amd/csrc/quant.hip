// E4M3 quantization for the FP8 projection ("DeepSeek AI II", section
// "DeepSeek Engram", multi-branch integration: the key and value
// projections fused into one dense FP8 matmul).  Each row (a weight row, or a
// token's concatenated memory vector e_t) gets its own scale s = max|x| / 448
// (1 for an all-zero row), and its values become the OCP E4M3 codes of x / s,
// rounded to nearest even.  The quotient is clamped to [-448, 448] first, so
// the largest magnitude maps to 448 whatever the rounding of s.
#include "kernels.h"

namespace engram {

// 8 values -> the E4M3 codes of x / s (2 words): a correctly rounded fp32
// division, then the hardware conversion (round to nearest even)
__device__ inline u32x2 to_e4m3x8(const float* x, float s) {
  u32x2 out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = fminf(fmaxf(x[4 * w + i] / s, -448.f), 448.f);
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
    out[w] = (uint32_t)word;
  }
  return out;
}

__device__ inline void widen8(const u32x4 u, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(u[i] << 16);
    x[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// the scale of a row whose largest magnitude is amax
__device__ inline float row_scale(float amax) { return amax > 0.f ? amax / 448.f : 1.f; }

// One wavefront per row of `cols` bf16 (or fp32) values; cols % 8 == 0.
template <bool BF16>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint8_t* __restrict__ src, int64_t rows,
                                                         int32_t cols, uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;  // whole wavefronts leave together
  const int chunks = cols / 8;
  auto load8 = [&](int c, float* x) {
    if constexpr (BF16) {
      widen8(*reinterpret_cast<const u32x4*>(src + (r * cols + c * 8) * 2), x);
    } else {
      const floatx4* p = reinterpret_cast<const floatx4*>(src + (r * cols + c * 8) * 4);
      const floatx4 a = p[0], b = p[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = a[i];
        x[4 + i] = b[i];
      }
    }
  };
  float amax = 0.f;
  for (int c = lane; c < chunks; c += 64) {
    float x[8];
    load8(c, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  }
  const float s = row_scale(wave_max(amax));
  if (lane == 0) scales[r] = s;
  for (int c = lane; c < chunks; c += 64) {
    float x[8];
    load8(c, x);
    *reinterpret_cast<u32x2*>(codes + r * cols + c * 8) = to_e4m3x8(x, s);
  }
}

// Row gather with quantization: one wavefront per token n gathers its J rows
// (bf16, 16-byte pieces), takes the scale of the whole e_n and writes e_n's
// codes [d_mem] and se[n].  A lane holds pieces lane, lane + 64, ...
constexpr int kQuantMaxPieces = kQuantMaxDmem / (64 * 8);  // bf16 16-byte pieces per lane
__global__ __launch_bounds__(256) void gather_quant_kernel(const int32_t* __restrict__ idx, int64_t N,
                                                           GatherArgs g, int32_t d_mem,
                                                           uint8_t* __restrict__ e8,
                                                           float* __restrict__ se) {
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  const int P = d_mem / 8;        // bf16 pieces of e_n
  const int PR = g.row_chunks;    // pieces per table row
  const int64_t row_bytes = (int64_t)PR * 16;
  u32x4 raw[kQuantMaxPieces];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kQuantMaxPieces; ++i) {
    const int p = lane + 64 * i;
    if (p < P) {
      const int j = p / PR, c = p - j * PR;
      raw[i] = *reinterpret_cast<const u32x4*>(g.base[j] + (int64_t)idx[n * g.J + j] * row_bytes + c * 16);
      float x[8];
      widen8(raw[i], x);
#pragma unroll
      for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
    }
  }
  const float s = row_scale(wave_max(amax));
  if (lane == 0) se[n] = s;
#pragma unroll
  for (int i = 0; i < kQuantMaxPieces; ++i) {
    const int p = lane + 64 * i;
    if (p < P) {
      float x[8];
      widen8(raw[i], x);
      *reinterpret_cast<u32x2*>(e8 + n * d_mem + p * 8) = to_e4m3x8(x, s);
    }
  }
}

hipError_t launch_quant_rows(const uint8_t* src, int32_t io_dtype, int64_t rows, int32_t cols,
                             uint8_t* codes, float* scales, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (cols % 8 != 0 || cols <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (io_dtype == ENGRAM_BF16)
    hipLaunchKernelGGL(quant_rows_kernel<true>, grid, dim3(256), 0, s, src, rows, cols, codes, scales);
  else
    hipLaunchKernelGGL(quant_rows_kernel<false>, grid, dim3(256), 0, s, src, rows, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_gather_quant(const int32_t* idx, int64_t N, const GatherArgs& g, int32_t d_mem,
                               uint8_t* e8, float* se, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (d_mem % 8 != 0 || d_mem / 8 > 64 * kQuantMaxPieces) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_quant_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, idx, N, g,
                     d_mem, e8, se);
  return hipGetLastError();
}

}  // namespace engram
