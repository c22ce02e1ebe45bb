// Table-sharded row exchange, the per-GPU device steps ("DeepSeek AI II",
// system-efficiency part: in training the tables are sharded over GPUs and
// each step exchanges the requested rows, and then their gradients, with
// All-to-All).  Rows of table j are owned in contiguous ranges: GPU g holds
// rows [g S_j, (g+1) S_j) with S_j = ceil(M_j / G), and a request names its
// row by (table, row - g S_j).
//
// Sender: distinct (table, row) keys of its tokens (sorted table-major, from
// the sort of the table-gradient path), grouped by owner: owner g's block
// holds its keys table by table in ascending row order.  Replies come back in
// the same order, so the forward reads token n's row j at the key's position
// in the send order (the compact-mode forward, unchanged).
// Owner: gathers the requested rows of its shard in request order, and adds
// the gradient rows it receives into its shard's dense gradient, one sender
// block after the other (a fixed order; rows are distinct within a block, so
// no atomics).
#include "kernels.h"

namespace engram {

constexpr int kShardMaxG = 64;

// first[j*G + g] = index of the first key of (table j, owner g) in the sorted
// keys; first[J*G] = count.  dest_base[g*J + j] = position in the send order
// of that key; send_counts[g] = keys for owner g.  One thread per (j, g)
// searches its boundary; thread 0 then lays out the blocks.
__global__ __launch_bounds__(1024) void owner_bounds_kernel(const uint64_t* __restrict__ keys,
                                                            const uint32_t* __restrict__ count_u32,
                                                            const int64_t* __restrict__ count_i64,
                                                            int32_t J, int32_t G, ShardRows sr,
                                                            int64_t* __restrict__ first,
                                                            int64_t* __restrict__ dest_base,
                                                            int64_t* __restrict__ send_counts) {
  const int64_t count = count_u32 ? (int64_t)count_u32[0] : count_i64[0];
  for (int t = threadIdx.x; t < J * G; t += blockDim.x) {
    const int j = t / G, g = t % G;
    // smallest index whose key is >= (j, g * S_j)
    const uint64_t target = ((uint64_t)j << 32) | (uint64_t)((int64_t)g * sr.rows[j]);
    int64_t lo = 0, hi = count;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (keys[mid] < target) lo = mid + 1; else hi = mid;
    }
    first[t] = lo;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    first[J * G] = count;
    int64_t pos = 0;
    for (int g = 0; g < G; ++g) {
      const int64_t b0 = pos;
      for (int j = 0; j < J; ++j) {
        const int64_t n = first[j * G + g + 1] - first[j * G + g];
        dest_base[g * J + j] = pos;
        pos += n;
      }
      send_counts[g] = pos - b0;
    }
  }
}

// For each key s < count: its send position, the request id (j << 27) |
// local row, and (with rows) its 16-byte pieces of the gradient row.
__global__ __launch_bounds__(256) void shard_pack_kernel(const uint64_t* __restrict__ keys,
                                                         const uint32_t* __restrict__ count_u32,
                                                         const int64_t* __restrict__ count_i64,
                                                         int32_t J, int32_t G, ShardRows sr,
                                                         const int64_t* __restrict__ first,
                                                         const int64_t* __restrict__ dest_base,
                                                         uint32_t* __restrict__ send_ids,
                                                         int32_t* __restrict__ send_pos,
                                                         const floatx4* __restrict__ rows,
                                                         floatx4* __restrict__ send_rows,
                                                         int32_t pieces, int64_t capacity) {
  const int64_t count = count_u32 ? (int64_t)count_u32[0] : count_i64[0];
  const int per = rows ? pieces : 1;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < capacity * per;
       e += (int64_t)gridDim.x * 256) {
    const int64_t s = e / per;
    const int c = (int)(e - s * per);
    if (s >= count) break;  // e only grows
    const uint64_t key = keys[s];
    const int j = (int)(key >> 32);
    const int64_t row = (int64_t)(uint32_t)key;
    const int g = (int)(row / sr.rows[j]);
    const int64_t pos = dest_base[g * J + j] + (s - first[j * G + g]);
    if (c == 0) {
      send_ids[pos] = ((uint32_t)j << 27) | (uint32_t)(row - (int64_t)g * sr.rows[j]);
      if (send_pos) send_pos[s] = (int32_t)pos;
    }
    if (rows) send_rows[pos * pieces + c] = rows[s * pieces + c];
  }
}

// inverse[i] = send_pos[inverse[i]]
__global__ __launch_bounds__(256) void remap_kernel(int32_t* __restrict__ inverse,
                                                    const int32_t* __restrict__ send_pos, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) inverse[i] = send_pos[inverse[i]];
}

// rows_out[i] = shard table j's local row, for request id (j << 27) | row
__global__ __launch_bounds__(256) void serve_kernel(ShardTables st, const uint32_t* __restrict__ ids,
                                                    int64_t n, u32x4* __restrict__ rows_out,
                                                    int32_t pieces) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n * pieces;
       e += (int64_t)gridDim.x * 256) {
    const int64_t i = e / pieces;
    const int c = (int)(e - i * pieces);
    const uint32_t id = ids[i];
    const u32x4* src = reinterpret_cast<const u32x4*>(st.base[id >> 27]);
    rows_out[e] = src[(int64_t)(id & 0x7FFFFFFu) * pieces + c];
  }
}

// grads_j[local row] += the received row, for one sender's block
__global__ __launch_bounds__(256) void grad_add_kernel(ShardGrads sg, const uint32_t* __restrict__ ids,
                                                       const floatx4* __restrict__ rows, int64_t n,
                                                       int32_t pieces) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n * pieces;
       e += (int64_t)gridDim.x * 256) {
    const int64_t i = e / pieces;
    const int c = (int)(e - i * pieces);
    const uint32_t id = ids[i];
    floatx4* dst = reinterpret_cast<floatx4*>(sg.base[id >> 27]) + (int64_t)(id & 0x7FFFFFFu) * pieces + c;
    *dst += rows[e];
  }
}

static unsigned grid_for(int64_t work) {
  const int64_t b = (work + 255) / 256;
  return (unsigned)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

hipError_t launch_shard_pack(const ShardPackArgs& a, hipStream_t s) {
  if (a.G < 1 || a.G > kShardMaxG || a.J * a.G > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(owner_bounds_kernel, dim3(1), dim3(1024), 0, s, a.keys, a.count_u32, a.count_i64,
                     a.J, a.G, a.shard_rows, a.first, a.dest_base, a.send_counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.capacity == 0) return e;
  const int per = a.rows ? a.pieces : 1;
  hipLaunchKernelGGL(shard_pack_kernel, dim3(grid_for(a.capacity * per)), dim3(256), 0, s, a.keys,
                     a.count_u32, a.count_i64, a.J, a.G, a.shard_rows, a.first, a.dest_base,
                     a.send_ids, a.send_pos, reinterpret_cast<const floatx4*>(a.rows),
                     reinterpret_cast<floatx4*>(a.send_rows), a.pieces, a.capacity);
  e = hipGetLastError();
  if (e != hipSuccess || !a.inverse || a.n_inverse == 0) return e;
  hipLaunchKernelGGL(remap_kernel, dim3((unsigned)((a.n_inverse + 255) / 256)), dim3(256), 0, s,
                     a.inverse, a.send_pos, a.n_inverse);
  return hipGetLastError();
}

hipError_t launch_shard_serve(const ShardTables& st, const uint32_t* ids, int64_t n, uint8_t* rows_out,
                              int32_t row_bytes, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int pieces = row_bytes / 16;
  hipLaunchKernelGGL(serve_kernel, dim3(grid_for(n * pieces)), dim3(256), 0, s, st, ids, n,
                     reinterpret_cast<u32x4*>(rows_out), pieces);
  return hipGetLastError();
}

hipError_t launch_shard_grad_add(const ShardGrads& sg, const uint32_t* ids, const float* rows,
                                 int64_t n, int32_t dim, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int pieces = dim / 4;
  hipLaunchKernelGGL(grad_add_kernel, dim3(grid_for(n * pieces)), dim3(256), 0, s, sg, ids,
                     reinterpret_cast<const floatx4*>(rows), n, pieces);
  return hipGetLastError();
}

}  // namespace engram
