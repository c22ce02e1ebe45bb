// Table-gradient scatter: dE_j[r] = sum_{t: idx_j(t) = r} de_t[j*D:(j+1)*D]
// ("DeepSeek AI II", system-efficiency part: the gradients of the gathered
// rows are sent back to the rows they came from).
//
// Deterministic path: per table, a stable LSD radix sort of the row ids
// (8-bit digits, token ids as payload, so equal rows keep token order),
// segment heads -> one segment per distinct (table, row), then a segmented
// fp32 reduction in sorted order: a group of D/4 lanes sums each segment,
// Zipf-heavy rows (long segments) included, with two accumulators in a fixed
// order.
// Comparison path: every token adds its slice with fp32 atomics (summation
// order varies run to run).
#include "kernels.h"

namespace engram {

constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;  // keys per block

static inline int64_t sort_blocks(int64_t N) { return (N + kSortTile - 1) / kSortTile; }

static inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

size_t sort_workspace_bytes(int64_t N, int32_t J) {
  const size_t nj = (size_t)N * J;
  const size_t nb = (size_t)sort_blocks(N);
  return 4 * align_up(nj * 4) + align_up((size_t)J * 256 * nb * 4) + align_up((size_t)J * nb * 4) +
         align_up(nj * 4) + align_up(nj * 8) + align_up(4);
}

void carve_sort(uint8_t* base, int64_t N, int32_t J, SortBufs* b) {
  const size_t nj = (size_t)N * J;
  const size_t nb = (size_t)sort_blocks(N);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = base + off;
    off += align_up(bytes);
    return p;
  };
  b->keys[0] = (uint32_t*)take(nj * 4);
  b->keys[1] = (uint32_t*)take(nj * 4);
  b->vals[0] = (uint32_t*)take(nj * 4);
  b->vals[1] = (uint32_t*)take(nj * 4);
  b->hist = (uint32_t*)take((size_t)J * 256 * nb * 4);
  b->seg_count = (uint32_t*)take((size_t)J * nb * 4);
  b->seg_start = (uint32_t*)take(nj * 4);
  b->seg_key = (uint64_t*)take(nj * 8);
  b->total = (uint32_t*)take(4);
}

// keys[j][n] = idx[n][j], vals[j][n] = n
__global__ __launch_bounds__(256) void sort_init_kernel(const int32_t* __restrict__ idx,
                                                        uint32_t* __restrict__ keys,
                                                        uint32_t* __restrict__ vals, int64_t N,
                                                        int J) {
  const int j = blockIdx.y;
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  keys[j * N + n] = (uint32_t)idx[n * J + j];
  vals[j * N + n] = (uint32_t)n;
}

// hist[j][digit][blk] for one 8-bit digit
__global__ __launch_bounds__(kSortThreads) void sort_hist_kernel(const uint32_t* __restrict__ keys,
                                                                 uint32_t* __restrict__ hist,
                                                                 int64_t N, int shift, int nb) {
  __shared__ uint32_t cnt[256];
  const int j = blockIdx.y;
  const int blk = blockIdx.x;
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const uint32_t* k = keys + j * N;
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t p = (int64_t)blk * kSortTile + r * kSortThreads + threadIdx.x;
    if (p < N) atomicAdd(&cnt[(k[p] >> shift) & 255u], 1u);
  }
  __syncthreads();
  hist[((int64_t)j * 256 + threadIdx.x) * nb + blk] = cnt[threadIdx.x];
}

// exclusive scan of hist[j][*][*] in (digit, block) order; thread = digit
__global__ __launch_bounds__(256) void sort_scan_kernel(uint32_t* __restrict__ hist, int nb) {
  __shared__ uint32_t sums[256];
  const int j = blockIdx.x;
  uint32_t* h = hist + ((int64_t)j * 256 + threadIdx.x) * nb;
  uint32_t s = 0;
  for (int i = 0; i < nb; ++i) s += h[i];
  sums[threadIdx.x] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over 256 digit totals
  for (int o = 1; o < 256; o <<= 1) {
    const uint32_t x = threadIdx.x >= o ? sums[threadIdx.x - o] : 0u;
    __syncthreads();
    sums[threadIdx.x] += x;
    __syncthreads();
  }
  uint32_t run = sums[threadIdx.x] - s;  // exclusive
  for (int i = 0; i < nb; ++i) {
    const uint32_t c = h[i];
    h[i] = run;
    run += c;
  }
}

// Stable scatter by digit.  Keys of a block are taken in rounds of 256
// (round-major, then thread order = input order); inside a round the rank of
// a key among equal digits comes from wave ballots and per-wave digit counts.
__global__ __launch_bounds__(kSortThreads) void sort_scatter_kernel(
    const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin, uint32_t* __restrict__ kout,
    uint32_t* __restrict__ vout, const uint32_t* __restrict__ hist, int64_t N, int shift, int nb) {
  constexpr int NW = kSortThreads / 64;
  __shared__ uint32_t running[256];
  __shared__ uint32_t wcount[NW][256];
  const int j = blockIdx.y;
  const int blk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  running[threadIdx.x] = hist[((int64_t)j * 256 + threadIdx.x) * nb + blk];
#pragma unroll
  for (int w = 0; w < NW; ++w) wcount[w][threadIdx.x] = 0;
  __syncthreads();
  const uint32_t* ki = kin + j * N;
  const uint32_t* vi = vin + j * N;
  uint32_t* ko = kout + j * N;
  uint32_t* vo = vout + j * N;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t p = (int64_t)blk * kSortTile + r * kSortThreads + threadIdx.x;
    const bool valid = p < N;
    const uint32_t key = valid ? ki[p] : 0u;
    const uint32_t val = valid ? vi[p] : 0u;
    const uint32_t dg = (key >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t bal = __ballot((dg >> bit) & 1u);
      peers &= ((dg >> bit) & 1u) ? bal : ~bal;
    }
    const uint32_t rank = (uint32_t)__popcll(peers & lt_mask);
    if (valid && rank == 0) wcount[wave][dg] = (uint32_t)__popcll(peers);
    __syncthreads();
    if (valid) {
      uint32_t base = running[dg];
      for (int w = 0; w < wave; ++w) base += wcount[w][dg];
      ko[base + rank] = key;
      vo[base + rank] = val;
    }
    __syncthreads();
    uint32_t add = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      add += wcount[w][threadIdx.x];
      wcount[w][threadIdx.x] = 0;
    }
    running[threadIdx.x] += add;
    __syncthreads();
  }
}

// number of segment heads per block of sorted keys
__global__ __launch_bounds__(256) void seg_count_kernel(const uint32_t* __restrict__ keys,
                                                        uint32_t* __restrict__ seg_count,
                                                        int64_t N, int nb) {
  __shared__ uint32_t tot;
  const int j = blockIdx.y;
  const int blk = blockIdx.x;
  if (threadIdx.x == 0) tot = 0;
  __syncthreads();
  const uint32_t* k = keys + j * N;
  uint32_t c = 0;
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t p = (int64_t)blk * kSortTile + r * 256 + threadIdx.x;
    if (p < N && (p == 0 || k[p] != k[p - 1])) ++c;
  }
  atomicAdd(&tot, c);
  __syncthreads();
  if (threadIdx.x == 0) seg_count[j * nb + blk] = tot;
}

// exclusive scan over all (table, block) head counts in order; total -> total[0]
__global__ __launch_bounds__(1024) void seg_scan_kernel(uint32_t* __restrict__ seg_count, int n,
                                                        uint32_t* __restrict__ total,
                                                        int64_t* __restrict__ count_out) {
  __shared__ uint32_t sums[1024];
  const int per = (n + 1023) / 1024;
  const int beg = threadIdx.x * per;
  uint32_t s = 0;
  for (int i = 0; i < per && beg + i < n; ++i) s += seg_count[beg + i];
  sums[threadIdx.x] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const uint32_t x = threadIdx.x >= o ? sums[threadIdx.x - o] : 0u;
    __syncthreads();
    sums[threadIdx.x] += x;
    __syncthreads();
  }
  uint32_t run = sums[threadIdx.x] - s;
  for (int i = 0; i < per && beg + i < n; ++i) {
    const uint32_t c = seg_count[beg + i];
    seg_count[beg + i] = run;
    run += c;
  }
  if (threadIdx.x == 1023) {
    total[0] = sums[1023];
    if (count_out) count_out[0] = (int64_t)sums[1023];
  }
}

// seg_start / seg_key of every head, in sorted order
__global__ __launch_bounds__(256) void seg_write_kernel(const uint32_t* __restrict__ keys,
                                                        const uint32_t* __restrict__ seg_count,
                                                        uint32_t* __restrict__ seg_start,
                                                        uint64_t* __restrict__ seg_key, int64_t N,
                                                        int nb) {
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t base_s;
  const int j = blockIdx.y;
  const int blk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (threadIdx.x == 0) base_s = seg_count[j * nb + blk];
  __syncthreads();
  const uint32_t* k = keys + j * N;
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t p = (int64_t)blk * kSortTile + r * 256 + threadIdx.x;
    const bool head = p < N && (p == 0 || k[p] != k[p - 1]);
    const uint64_t bal = __ballot(head);
    if (lane == 0) wsum[wave] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t base = base_s;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    if (head) {
      const uint32_t s = base + (uint32_t)__popcll(bal & lt_mask);
      seg_start[s] = (uint32_t)(j * N + p);
      seg_key[s] = ((uint64_t)j << 32) | k[p];
    }
    __syncthreads();
    if (threadIdx.x == 0) base_s += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
}

// inverse[n][j] = index of (j, idx[n][j]) among all segment heads: the
// position of token n's row in the distinct keys seg_key.  The segment of
// sorted position p is the number of heads at or before p, minus one.
__global__ __launch_bounds__(256) void seg_inverse_kernel(const uint32_t* __restrict__ keys,
                                                          const uint32_t* __restrict__ vals,
                                                          const uint32_t* __restrict__ seg_count,
                                                          int32_t* __restrict__ inverse, int64_t N,
                                                          int nb, int J) {
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t base_s;
  const int j = blockIdx.y;
  const int blk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint64_t le_mask = ~0ull >> (63 - lane);
  if (threadIdx.x == 0) base_s = seg_count[j * nb + blk];
  __syncthreads();
  const uint32_t* k = keys + j * N;
  const uint32_t* v = vals + j * N;
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t p = (int64_t)blk * kSortTile + r * 256 + threadIdx.x;
    const bool head = p < N && (p == 0 || k[p] != k[p - 1]);
    const uint64_t bal = __ballot(head);
    if (lane == 0) wsum[wave] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t base = base_s;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    if (p < N) inverse[(int64_t)v[p] * J + j] = (int32_t)(base + (uint32_t)__popcll(bal & le_mask) - 1);
    __syncthreads();
    if (threadIdx.x == 0) base_s += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
}

// Segmented reduce.  A wave holds S = 64 / (D/4) lane groups of D/4 lanes
// (one 16-byte column piece per lane); each group sums whole segments in a
// grid-stride walk and writes their rows.  Most segments have one element,
// so the cost is the chain segment start -> token -> de row; a group runs two
// segments side by side (two independent chains) and sums each segment's
// elements in sorted order with two accumulators (a fixed order).
constexpr int kSegBlocksMax = 4096;
template <int MODE>
__global__ __launch_bounds__(256) void seg_reduce_kernel(ScatterArgs a, const uint32_t* __restrict__ vals,
                                                         const uint32_t* __restrict__ seg_start,
                                                         const uint64_t* __restrict__ seg_key,
                                                         const uint32_t* __restrict__ total) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int D4 = a.D / 4;               // <= 64 (D <= 256)
  const int S = 64 / D4;
  const int grp = lane / D4;
  const int col = lane - grp * D4;
  if (grp >= S) return;
  const int64_t U = total[0];
  const int64_t NJ = a.N * a.J;
  const int64_t dm = (int64_t)a.J * a.D;
  const int64_t stride = (int64_t)gridDim.x * 4 * S;
  auto bounds = [&](int64_t seg, int64_t& beg, int64_t& end, uint64_t& key) {
    beg = seg_start[seg];
    end = (seg + 1 < U) ? (int64_t)seg_start[seg + 1] : NJ;
    key = seg_key[seg];
  };
  auto row_src = [&](uint64_t key) -> const float* {
    return a.de + (int64_t)(key >> 32) * a.D + col * 4;
  };
  // the rest of a segment after its first element
  auto tail = [&](const float* src, int64_t p, int64_t end, floatx4 acc0) -> floatx4 {
    floatx4 acc1 = floatx4{0.f, 0.f, 0.f, 0.f};
    for (; p + 1 < end; p += 2) {
      const int64_t t0 = vals[p], t1 = vals[p + 1];
      acc0 += *reinterpret_cast<const floatx4*>(src + t0 * dm);
      acc1 += *reinterpret_cast<const floatx4*>(src + t1 * dm);
    }
    if (p < end) acc0 += *reinterpret_cast<const floatx4*>(src + (int64_t)vals[p] * dm);
    return acc0 + acc1;
  };
  auto emit = [&](int64_t seg, uint64_t key, floatx4 acc) {
    const int j = (int)(key >> 32);
    const int64_t row = (int64_t)(key & 0xFFFFFFFFu);
    if (MODE == ENGRAM_GRAD_SORTED_SPARSE) {
      *reinterpret_cast<floatx4*>(a.rows_out + seg * a.D + col * 4) = acc;
      if (col == 0) a.keys_out[seg] = (int64_t)key;
    } else {
      floatx4* dst = reinterpret_cast<floatx4*>(a.dense[j] + row * a.D + col * 4);
      *dst = *dst + acc;
    }
  };
  for (int64_t sa = ((int64_t)blockIdx.x * 4 + wave) * S + grp; sa < U; sa += 2 * stride) {
    const int64_t sb = sa + stride;
    const bool hb = sb < U;
    int64_t ba, ea, bb = 0, eb = 0;
    uint64_t ka, kb = 0;
    bounds(sa, ba, ea, ka);
    if (hb) bounds(sb, bb, eb, kb);
    const float* srca = row_src(ka);
    const float* srcb = row_src(kb);
    const int64_t ta = vals[ba];
    const int64_t tb = hb ? (int64_t)vals[bb] : 0;
    floatx4 xa = *reinterpret_cast<const floatx4*>(srca + ta * dm);
    floatx4 xb = hb ? *reinterpret_cast<const floatx4*>(srcb + tb * dm) : floatx4{};
    if (ea - ba > 1) xa = tail(srca, ba + 1, ea, xa);
    emit(sa, ka, xa);
    if (hb) {
      if (eb - bb > 1) xb = tail(srcb, bb + 1, eb, xb);
      emit(sb, kb, xb);
    }
  }
}

hipError_t launch_sorted_scatter(const ScatterArgs& a, const SortBufs& b, int32_t mode,
                                 hipStream_t s) {
  const int64_t N = a.N;
  const int J = a.J;
  if (N == 0) {  // no keys: the scan of zero counts writes count 0 (no memset node)
    hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(1024), 0, s, b.seg_count, 0, b.total,
                       mode == ENGRAM_GRAD_SORTED_SPARSE ? a.count_out : nullptr);
    return hipGetLastError();
  }
  const int nb = (int)sort_blocks(N);
  hipLaunchKernelGGL(sort_init_kernel, dim3((unsigned)((N + 255) / 256), J), dim3(256), 0, s, a.idx,
                     b.keys[0], b.vals[0], N, J);
  int cur = 0;
  const int passes = (a.key_bits + 7) / 8;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * 8;
    hipLaunchKernelGGL(sort_hist_kernel, dim3(nb, J), dim3(kSortThreads), 0, s, b.keys[cur], b.hist,
                       N, shift, nb);
    hipLaunchKernelGGL(sort_scan_kernel, dim3(J), dim3(256), 0, s, b.hist, nb);
    hipLaunchKernelGGL(sort_scatter_kernel, dim3(nb, J), dim3(kSortThreads), 0, s, b.keys[cur],
                       b.vals[cur], b.keys[cur ^ 1], b.vals[cur ^ 1], b.hist, N, shift, nb);
    cur ^= 1;
  }
  hipLaunchKernelGGL(seg_count_kernel, dim3(nb, J), dim3(256), 0, s, b.keys[cur], b.seg_count, N, nb);
  hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(1024), 0, s, b.seg_count, nb * J, b.total,
                     mode == ENGRAM_GRAD_SORTED_SPARSE ? a.count_out : nullptr);
  hipLaunchKernelGGL(seg_write_kernel, dim3(nb, J), dim3(256), 0, s, b.keys[cur], b.seg_count,
                     b.seg_start, b.seg_key, N, nb);
  // grid-stride over at most N*J segments, S per wave
  const int64_t max_segs = N * J;
  const int S = 64 / (a.D / 4);
  const int64_t want = (max_segs + 4 * S - 1) / (4 * S);
  const unsigned blocks = (unsigned)(want < kSegBlocksMax ? want : kSegBlocksMax);
  if (mode == ENGRAM_GRAD_SORTED_SPARSE)
    hipLaunchKernelGGL(seg_reduce_kernel<ENGRAM_GRAD_SORTED_SPARSE>, dim3(blocks), dim3(256), 0, s, a,
                       b.vals[cur], b.seg_start, b.seg_key, b.total);
  else
    hipLaunchKernelGGL(seg_reduce_kernel<ENGRAM_GRAD_SORTED_DENSE>, dim3(blocks), dim3(256), 0, s, a,
                       b.vals[cur], b.seg_start, b.seg_key, b.total);
  return hipGetLastError();
}

hipError_t launch_dedup(const int32_t* idx, int64_t N, int32_t J, int32_t key_bits,
                        const SortBufs& b, int32_t* inverse, hipStream_t s) {
  if (N == 0) {  // zero heads: total 0
    hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(1024), 0, s, b.seg_count, 0, b.total, nullptr);
    return hipGetLastError();
  }
  const int nb = (int)sort_blocks(N);
  hipLaunchKernelGGL(sort_init_kernel, dim3((unsigned)((N + 255) / 256), J), dim3(256), 0, s, idx,
                     b.keys[0], b.vals[0], N, J);
  int cur = 0;
  const int passes = (key_bits + 7) / 8;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * 8;
    hipLaunchKernelGGL(sort_hist_kernel, dim3(nb, J), dim3(kSortThreads), 0, s, b.keys[cur], b.hist,
                       N, shift, nb);
    hipLaunchKernelGGL(sort_scan_kernel, dim3(J), dim3(256), 0, s, b.hist, nb);
    hipLaunchKernelGGL(sort_scatter_kernel, dim3(nb, J), dim3(kSortThreads), 0, s, b.keys[cur],
                       b.vals[cur], b.keys[cur ^ 1], b.vals[cur ^ 1], b.hist, N, shift, nb);
    cur ^= 1;
  }
  hipLaunchKernelGGL(seg_count_kernel, dim3(nb, J), dim3(256), 0, s, b.keys[cur], b.seg_count, N, nb);
  hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(1024), 0, s, b.seg_count, nb * J, b.total, nullptr);
  hipLaunchKernelGGL(seg_write_kernel, dim3(nb, J), dim3(256), 0, s, b.keys[cur], b.seg_count,
                     b.seg_start, b.seg_key, N, nb);
  hipLaunchKernelGGL(seg_inverse_kernel, dim3(nb, J), dim3(256), 0, s, b.keys[cur], b.vals[cur],
                     b.seg_count, inverse, N, nb, J);
  return hipGetLastError();
}

// grid.y = table; x walks (token, float4 column)
__global__ __launch_bounds__(256) void atomic_scatter_kernel(ScatterArgs a) {
  const int j = blockIdx.y;
  const int D4 = a.D / 4;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= a.N * D4) return;
  const int64_t n = c / D4;
  const int c4 = (int)(c - n * D4);
  const int64_t row = a.idx[n * a.J + j];
  const floatx4 v =
      *reinterpret_cast<const floatx4*>(a.de + n * (int64_t)a.J * a.D + (int64_t)j * a.D + c4 * 4);
  float* dst = a.dense[j] + row * a.D + c4 * 4;
  unsafeAtomicAdd(dst + 0, v[0]);
  unsafeAtomicAdd(dst + 1, v[1]);
  unsafeAtomicAdd(dst + 2, v[2]);
  unsafeAtomicAdd(dst + 3, v[3]);
}

hipError_t launch_atomic_scatter(const ScatterArgs& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  const int64_t total = a.N * (a.D / 4);
  hipLaunchKernelGGL(atomic_scatter_kernel, dim3((unsigned)((total + 255) / 256), a.J), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace engram
