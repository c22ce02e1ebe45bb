// Canonicalisation + multi-head hashing, and the row gather that builds e_t.
//
// Hashing ("DeepSeek AI II", section "DeepSeek Engram": tokenizer
// compression, suffix N-grams, multi-head hashing into prime-sized tables):
// one lane per token; the canonical ids of the previous positions come from
// neighbouring lanes of the same wavefront (cross-lane shift), so each token
// id and its canonical-map entry are read once per wave.
//
// Gather ("DeepSeek AI II", section "DeepSeek Engram": all retrieved
// embeddings are concatenated into e_t): e is numbered in 16-byte pieces and
// each lane copies pieces of it, so table rows are read as whole contiguous
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
  const uint32_t c0 = canon_of(canon, tokens[nc], a, live);
  uint32_t c[ENGRAM_MAX_ORDERS];
  c[0] = c0;
#pragma unroll
  for (int i = 1; i < ENGRAM_MAX_ORDERS; ++i) {
    if (i < a.max_order) {
      const uint32_t from_left = __shfl_up(c0, i);
      if (t - i < 0)
        c[i] = (uint32_t)a.pad_id;
      else if (lane < i)
        c[i] = canon_of(canon, tokens[nc - i], a, false);
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

// Piece c of e (16 bytes) is piece c % rc of row idx[c / rc] of table
// (c / rc) % J: e is written front to back and idx read in order.  Each
// thread moves kGatherPer pieces, kGatherPer * 256 apart, with all its row
// loads in flight together.  32-bit piece numbers (the host checks the size).
#ifndef ENGRAM_GATHER_PER
#define ENGRAM_GATHER_PER 4
#endif
#ifndef ENGRAM_GATHER_NT
#define ENGRAM_GATHER_NT 0
#endif
constexpr int kGatherPer = ENGRAM_GATHER_PER;
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ idx,
                                                     uint8_t* __restrict__ e, uint32_t pieces,
                                                     GatherArgs g) {
  __shared__ const uint8_t* base_s[ENGRAM_MAX_TABLES];
  if (threadIdx.x < (unsigned)g.J) base_s[threadIdx.x] = g.base[threadIdx.x];
  __syncthreads();
  const uint32_t rc = (uint32_t)g.row_chunks;
  const uint32_t J = (uint32_t)g.J;
  const uint32_t c0 = blockIdx.x * (256u * kGatherPer) + threadIdx.x;
  u32x4 v[kGatherPer];
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u) {
    const uint32_t c = c0 + u * 256u;
    if (c < pieces) {
      const uint32_t nj = c / rc;  // token * J + table
      const uint32_t part = c - nj * rc;
      const uint32_t j = nj % J;
      const int64_t row = idx[nj];
      v[u] = *(reinterpret_cast<const u32x4*>(base_s[j] + row * rc * 16) + part);
    }
  }
  if (g.row_scale) {  // bf16 rows of token n divided by row_scale[n] (a power of two: exact)
#pragma unroll
    for (int u = 0; u < kGatherPer; ++u) {
      const uint32_t c = c0 + u * 256u;
      if (c < pieces) {
        const float inv = pow2_inverse(g.row_scale[c / rc / J]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[u][i] = pack_bf16x2(__uint_as_float(v[u][i] << 16) * inv,
                                __uint_as_float(v[u][i] & 0xFFFF0000u) * inv);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u) {
    const uint32_t c = c0 + u * 256u;
    if (c < pieces) *(reinterpret_cast<u32x4*>(e) + c) = v[u];
  }
}

// Hash and gather in one kernel, for the forward that gathers e into memory:
// a block first hashes the tokens its pieces of e belong to (their canonical
// ids, with the N-gram context before them, staged in LDS), then copies its
// pieces as gather_kernel does, reading the row indices from LDS.  The
// indices of a token are written out (when asked) by the block that holds
// its first piece.  One kernel boundary fewer than hash + gather; the hashes
// of a token whose pieces straddle two blocks are computed twice.
constexpr int kHgPieces = 256 * kGatherPer;      // pieces of e per block
constexpr int kHgMaxTok = kHgPieces / 32 + 1;   // tokens a block touches (>= 32 pieces a token)
__global__ __launch_bounds__(256) void hash_gather_kernel(const int32_t* __restrict__ tokens,
                                                          const int32_t* __restrict__ canon,
                                                          int32_t T, uint32_t pieces, GatherArgs g,
                                                          HashArgs a, uint8_t* __restrict__ e,
                                                          int32_t* __restrict__ idx_out) {
  __shared__ const uint8_t* base_s[ENGRAM_MAX_TABLES];
  __shared__ uint32_t c_s[kHgMaxTok + ENGRAM_MAX_ORDERS - 1];
  __shared__ int32_t idx_s[kHgMaxTok * ENGRAM_MAX_TABLES];
  const uint32_t rc = (uint32_t)g.row_chunks;
  const uint32_t J = (uint32_t)g.J;
  const uint32_t tp = rc * J;  // pieces per token
  const uint32_t c_begin = blockIdx.x * (uint32_t)kHgPieces;
  const uint32_t c_end = c_begin + kHgPieces < pieces ? c_begin + kHgPieces : pieces;
  const int64_t n0 = c_begin / tp;
  const int ntok = (int)((c_end - 1) / tp - n0) + 1;
  const int H = a.max_order - 1;  // context tokens before n0
  if (threadIdx.x < J) base_s[threadIdx.x] = g.base[threadIdx.x];
  for (int i = threadIdx.x; i < ntok + H; i += 256) {
    const int64_t n = n0 - H + i;
    // the block holding a token's first piece owns it (counts a bad id)
    const bool own = i >= H && (uint64_t)n * tp >= c_begin;
    c_s[i] = n >= 0 ? canon_of(canon, tokens[n], a, own) : 0u;  // n < 0 is never read (pad instead)
  }
  __syncthreads();
  for (int q = threadIdx.x; q < ntok * (int)J; q += 256) {
    const int k = q / (int)J, j = q - k * (int)J;  // token n0 + k, table j
    const int64_t n = n0 + k;
    const int t = (int)(n % T);
    uint32_t c[ENGRAM_MAX_ORDERS];
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDERS; ++i)
      c[i] = i < a.max_order ? (t - i < 0 ? (uint32_t)a.pad_id : c_s[k + H - i]) : 0u;
    const int32_t r = (int32_t)hash_one(a, j, a.orders[j / a.heads], c);
    idx_s[q] = r;
    if (idx_out && (uint64_t)n * tp >= c_begin) idx_out[n * J + j] = r;
  }
  __syncthreads();
  const uint32_t c0 = c_begin + threadIdx.x;
  u32x4 v[kGatherPer];
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u) {
    const uint32_t c = c0 + u * 256u;
    if (c < c_end) {
      const uint32_t nj = c / rc;  // token * J + table
      const uint32_t part = c - nj * rc;
      const uint32_t j = nj % J;
      const int64_t row = idx_s[nj - (uint32_t)n0 * J];
      v[u] = *(reinterpret_cast<const u32x4*>(base_s[j] + row * rc * 16) + part);
    }
  }
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u) {
    const uint32_t c = c0 + u * 256u;
    if (c < c_end) {
      u32x4* p = reinterpret_cast<u32x4*>(e) + c;
      if constexpr (ENGRAM_GATHER_NT != 0)
        __builtin_nontemporal_store(v[u], p);
      else
        *p = v[u];
    }
  }
}

hipError_t launch_hash_gather(const int32_t* tokens, const int32_t* canon, int64_t N, int32_t T,
                              const HashArgs& a, const GatherArgs& g, uint8_t* e, int32_t* idx_out,
                              hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int64_t tp = (int64_t)g.J * g.row_chunks;
  const int64_t pieces = N * tp;
  if (tp < 32 || pieces >= (int64_t(1) << 32) - kHgPieces) return hipErrorInvalidValue;
  const int64_t blocks = (pieces + kHgPieces - 1) / kHgPieces;
  hipLaunchKernelGGL(hash_gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, tokens, canon, T,
                     (uint32_t)pieces, g, a, e, idx_out);
  return hipGetLastError();
}

// Hash + gather with the repeats of a tile served from LDS: a block owns
// kDdTok consecutive tokens.  It hashes their J indices into LDS, marks each
// (table, row) pair's first occurrence in the tile as its leader, reads only
// the leaders' rows from the tables into LDS, and writes every token's pieces
// of e from there.  N-grams recur in text, often within a few tokens, so a
// tile can hold the same (table, row) more than once; each such row then
// costs one read instead of several.
#ifndef ENGRAM_DEDUP_TOKENS
#define ENGRAM_DEDUP_TOKENS 16
#endif
constexpr int kDdTok = ENGRAM_DEDUP_TOKENS;
constexpr int kDdPer = 8;  // leader-row loads in flight per thread
__global__ __launch_bounds__(256) void dedup_gather_kernel(const int32_t* __restrict__ tokens,
                                                           const int32_t* __restrict__ canon,
                                                           int64_t N, int32_t T, GatherArgs g,
                                                           HashArgs a, uint8_t* __restrict__ e,
                                                           int32_t* __restrict__ idx_out) {
  extern __shared__ __attribute__((aligned(16))) u32x4 rows_s[];  // [kDdTok * J][rc]
  __shared__ const uint8_t* base_s[ENGRAM_MAX_TABLES];
  __shared__ uint32_t c_s[kDdTok + ENGRAM_MAX_ORDERS - 1];
  __shared__ int32_t key_s[kDdTok * ENGRAM_MAX_TABLES];
  __shared__ int16_t lead_s[kDdTok * ENGRAM_MAX_TABLES];
  __shared__ int16_t list_s[kDdTok * ENGRAM_MAX_TABLES];
  __shared__ int nlead_s;
  const int tid = threadIdx.x;
  const int J = g.J, rc = g.row_chunks;
  const int64_t n0 = (int64_t)blockIdx.x * kDdTok;
  const int ntok = N - n0 < kDdTok ? (int)(N - n0) : kDdTok;
  const int H = a.max_order - 1;
  if (tid < J) base_s[tid] = g.base[tid];
  if (tid == 0) nlead_s = 0;
  for (int i = tid; i < ntok + H; i += 256) {
    const int64_t n = n0 - H + i;
    c_s[i] = n >= 0 ? canon_of(canon, tokens[n], a, i >= H) : 0u;  // n < 0 is never read
  }
  __syncthreads();
  const int np = ntok * J;  // pairs (token k, table j), q = k * J + j
  for (int q = tid; q < np; q += 256) {
    const int k = q / J, j = q - k * J;
    const int64_t n = n0 + k;
    const int t = (int)(n % T);
    uint32_t c[ENGRAM_MAX_ORDERS];
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDERS; ++i)
      c[i] = i < a.max_order ? (t - i < 0 ? (uint32_t)a.pad_id : c_s[k + H - i]) : 0u;
    const int32_t r = (int32_t)hash_one(a, j, a.orders[j / a.heads], c);
    key_s[q] = r;
    if (idx_out) idx_out[n * J + j] = r;
  }
  __syncthreads();
  // leader of pair (k, j): the first token of the tile with the same row of table j
  for (int q = tid; q < np; q += 256) {
    const int k = q / J, j = q - k * J;
    const int32_t key = key_s[q];
    int kl = k;
    for (int k2 = 0; k2 < k; ++k2)
      if (key_s[k2 * J + j] == key) {
        kl = k2;
        break;
      }
    lead_s[q] = (int16_t)(kl * J + j);
    if (kl == k) list_s[atomicAdd(&nlead_s, 1)] = (int16_t)q;
  }
  __syncthreads();
  // the leaders' rows into LDS, kDdPer loads in flight per thread
  const int nl = nlead_s;
  for (int c0 = tid; c0 < nl * rc; c0 += 256 * kDdPer) {
    u32x4 v[kDdPer];
    int dst[kDdPer];
#pragma unroll
    for (int u = 0; u < kDdPer; ++u) {
      const int c = c0 + u * 256;
      dst[u] = -1;
      if (c < nl * rc) {
        const int li = c / rc, part = c - li * rc;
        const int q = list_s[li];
        const int j = q % J;
        v[u] = *(reinterpret_cast<const u32x4*>(base_s[j] + (int64_t)key_s[q] * rc * 16) + part);
        dst[u] = q * rc + part;
      }
    }
#pragma unroll
    for (int u = 0; u < kDdPer; ++u)
      if (dst[u] >= 0) rows_s[dst[u]] = v[u];
  }
  __syncthreads();
  // every pair's pieces of e from its leader's row
  u32x4* eo = reinterpret_cast<u32x4*>(e) + (uint64_t)n0 * J * rc;
  for (int c = tid; c < np * rc; c += 256) {
    const int q = c / rc, part = c - q * rc;
    eo[c] = rows_s[lead_s[q] * rc + part];
  }
}

hipError_t launch_dedup_gather(const int32_t* tokens, const int32_t* canon, int64_t N, int32_t T,
                               const HashArgs& a, const GatherArgs& g, uint8_t* e, int32_t* idx_out,
                               hipStream_t s) {
  if (N == 0) return hipSuccess;
  const size_t lds = dedup_gather_lds_bytes(g.J, g.row_chunks);
  if (lds == 0) return hipErrorInvalidValue;
  const int64_t blocks = (N + kDdTok - 1) / kDdTok;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const hipError_t at = hipFuncSetAttribute((const void*)dedup_gather_kernel,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (at != hipSuccess) return at;
  hipLaunchKernelGGL(dedup_gather_kernel, dim3((unsigned)blocks), dim3(256), lds, s, tokens, canon,
                     N, T, g, a, e, idx_out);
  return hipGetLastError();
}

size_t dedup_gather_lds_bytes(int32_t J, int32_t row_chunks) {
  const size_t b = (size_t)kDdTok * J * row_chunks * 16;
  return b <= (size_t(64) << 10) ? b : 0;  // the rest of the 160 KB is the block's own arrays
}

hipError_t launch_gather(const int32_t* idx, uint8_t* e, int64_t N, const GatherArgs& g,
                         hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int64_t pieces = N * g.J * g.row_chunks;
  if (pieces >= (int64_t(1) << 32) - 256 * kGatherPer) return hipErrorInvalidValue;
  const int64_t blocks = (pieces + 256 * kGatherPer - 1) / (256 * kGatherPer);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, idx, e,
                     (uint32_t)pieces, g);
  return hipGetLastError();
}

}  // namespace engram
