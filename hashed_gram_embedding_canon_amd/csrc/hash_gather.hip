// Canonicalisation + multi-head hashing, and the row gather that builds e_t.
//
// Hashing ("DeepSeek AI II", section "DeepSeek Engram": tokenizer
// compression, suffix N-grams, multi-head hashing into prime-sized tables):
// one lane per token; the canonical ids of the previous positions come from
// neighbouring lanes of the same wavefront (cross-lane shift), so each token
// id and its canonical-map entry are read once per wave.
//
// Gather ("DeepSeek AI II", section "DeepSeek Engram": all retrieved
// embeddings are concatenated into e_t): one block column per table, 16-byte
// lanes walking each row, so a table row is read as whole contiguous
// 16-byte pieces and e is written in order.
#include "kernels.h"

namespace engram {

__global__ __launch_bounds__(256) void hash_kernel(const int32_t* __restrict__ tokens,
                                                   const int32_t* __restrict__ canon, int64_t N,
                                                   int32_t T, int32_t* __restrict__ idx,
                                                   HashArgs a) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = n < N;
  const int64_t nc = live ? n : N - 1;  // dead lanes still take part in the shifts
  const int t = (int)(nc % T);
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t c0 = (uint32_t)canon[tokens[nc]];
  uint32_t c[ENGRAM_MAX_ORDERS];
  c[0] = c0;
#pragma unroll
  for (int i = 1; i < ENGRAM_MAX_ORDERS; ++i) {
    if (i < a.max_order) {
      const uint32_t from_left = __shfl_up(c0, i);
      if (t - i < 0)
        c[i] = (uint32_t)a.pad_id;
      else if (lane < i)
        c[i] = (uint32_t)canon[tokens[nc - i]];
      else
        c[i] = from_left;
    } else {
      c[i] = 0;
    }
  }
  if (!live) return;
  int32_t* out = idx + n * a.J;
  int j = 0;
  for (int o = 0; o < a.num_orders; ++o) {
    const int order = a.orders[o];
    for (int k = 0; k < a.heads; ++k, ++j) out[j] = (int32_t)hash_one(a, j, order, c);
  }
}

hipError_t launch_hash(const int32_t* tokens, const int32_t* canon, int64_t N, int32_t T,
                       int32_t* idx, const HashArgs& args, hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int64_t blocks = (N + 255) / 256;
  hipLaunchKernelGGL(hash_kernel, dim3((unsigned)blocks), dim3(256), 0, s, tokens, canon, N, T,
                     idx, args);
  return hipGetLastError();
}

// grid.y = table j (uniform per block); x walks (token, 16-byte piece) pairs.
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ idx,
                                                     uint8_t* __restrict__ e, int64_t N,
                                                     GatherArgs g) {
  const int j = blockIdx.y;
  const int rc = g.row_chunks;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= N * rc) return;
  const int64_t n = c / rc;
  const int part = (int)(c - n * rc);
  const int64_t row = idx[n * g.J + j];
  const uint4* src = reinterpret_cast<const uint4*>(g.base[j] + row * rc * 16) + part;
  uint4* dst = reinterpret_cast<uint4*>(e + (n * g.J + j) * rc * 16) + part;
  *dst = *src;
}

hipError_t launch_gather(const int32_t* idx, uint8_t* e, int64_t N, const GatherArgs& g,
                         hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int64_t blocks = (N * g.row_chunks + 255) / 256;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks, g.J), dim3(256), 0, s, idx, e, N, g);
  return hipGetLastError();
}

}  // namespace engram
