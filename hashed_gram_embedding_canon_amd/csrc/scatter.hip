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

// bit 1: the segmented reduce reads the per-token gradient rows with
// non-temporal loads (each is read once); bit 2: it writes the sparse rows
// with non-temporal stores
#ifndef ENGRAM_SCATTER_NT
#define ENGRAM_SCATTER_NT 1
#endif
#ifndef ENGRAM_RED_SEGS
#define ENGRAM_RED_SEGS 256
#endif
// 1: the groups of the whole grid take the short segments in a grid-stride
// walk (all of them in one window of the output at a time); 0: each block
// takes the segments of its own range
#ifndef ENGRAM_RED_GRID_STRIDE
#define ENGRAM_RED_GRID_STRIDE 1
#endif
// segments per group and batch
#ifndef ENGRAM_RED_BATCH
#define ENGRAM_RED_BATCH 4
#endif
// 1: the next batch's bounds, keys and tokens load behind the current rows
#ifndef ENGRAM_RED_PREFETCH
#define ENGRAM_RED_PREFETCH 1
#endif

namespace engram {

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / 64;
#ifndef ENGRAM_SORT_ITEMS
#define ENGRAM_SORT_ITEMS 16
#endif
constexpr int kSortItems = ENGRAM_SORT_ITEMS;  // keys per thread
constexpr int kSortTile = kSortThreads * kSortItems;  // keys per block
constexpr int kWaveRange = 64 * kSortItems;            // keys per wave
// Up to this many blocks per table, each scatter block derives its digit
// offsets from the per-block histograms itself (one cache line per digit);
// beyond it a separate scan kernel writes them.
constexpr int kFusedScanBlocks = 64;

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

// Position of item r of a lane inside table j's key array: a block takes
// kSortTile consecutive keys, each of its waves kWaveRange of them, one
// coalesced row of 64 per item.  Key order inside a block is (wave, item,
// lane), which is input order.
__device__ __forceinline__ int64_t tile_pos(int blk, int wave, int r, int lane) {
  return (int64_t)blk * kSortTile + wave * kWaveRange + r * 64 + lane;
}

// Key and token of position p of table j.  The first pass reads the row ids
// straight from idx [N][J] (the token is the position); later passes read the
// previous pass's output.
template <bool FIRST>
__device__ __forceinline__ void load_pair(const int32_t* __restrict__ idx,
                                          const uint32_t* __restrict__ kin,
                                          const uint32_t* __restrict__ vin, int64_t N, int J, int j,
                                          int64_t p, uint32_t& key, uint32_t& val) {
  if (p >= N) {
    key = 0u;
    val = 0u;
  } else if (FIRST) {
    key = (uint32_t)idx[p * J + j];
    val = (uint32_t)p;
  } else {
    key = kin[j * N + p];
    val = vin[j * N + p];
  }
}

// hist[j][digit][blk] for one 8-bit digit
template <bool FIRST>
__global__ __launch_bounds__(kSortThreads) void sort_hist_kernel(const int32_t* __restrict__ idx,
                                                                 const uint32_t* __restrict__ keys,
                                                                 uint32_t* __restrict__ hist,
                                                                 int64_t N, int J, int shift, int nb) {
  __shared__ uint32_t cnt[256];
  const int j = blockIdx.y;
  const int blk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  uint32_t key[kSortItems];
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    uint32_t v;
    load_pair<FIRST>(idx, keys, keys, N, J, j, tile_pos(blk, wave, r, lane), key[r], v);
  }
  cnt[threadIdx.x] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSortItems; ++r)
    if (tile_pos(blk, wave, r, lane) < N) atomicAdd(&cnt[(key[r] >> shift) & 255u], 1u);
  __syncthreads();
  hist[((int64_t)j * 256 + threadIdx.x) * nb + blk] = cnt[threadIdx.x];
}

// Exclusive scan of hist[j][*][*] in (digit, block) order, thread = digit;
// used when a table has more than kFusedScanBlocks blocks.
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

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Stable scatter by one 8-bit digit.  All keys of the block are loaded
// first.  Each wave ranks its own kWaveRange keys in order with ballots and a
// per-wave digit count in LDS (no block barrier between items).  The block
// then orders its keys by digit in LDS (digit start in the block + counts of
// the waves before + rank) and writes them out in that order, so that each
// digit's keys form one run of consecutive output positions starting at the
// digit's block base (this block's share of the table-wide exclusive scan).
template <bool FIRST, bool FUSED>
__global__ __launch_bounds__(kSortThreads) void sort_scatter_kernel(
    const int32_t* __restrict__ idx, const uint32_t* __restrict__ kin,
    const uint32_t* __restrict__ vin, uint32_t* __restrict__ kout, uint32_t* __restrict__ vout,
    const uint32_t* __restrict__ hist, int64_t N, int J, int shift, int nb) {
  __shared__ uint32_t wcount[kSortWaves][256];
  __shared__ uint32_t wtot[kSortWaves], wtot2[kSortWaves];
  __shared__ uint32_t dstart[256], dshift[256];
  __shared__ uint32_t ks[kSortTile], vs[kSortTile];
  const int j = blockIdx.y;
  const int blk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  uint32_t key[kSortItems], val[kSortItems];
#pragma unroll
  for (int r = 0; r < kSortItems; ++r)
    load_pair<FIRST>(idx, kin, vin, N, J, j, tile_pos(blk, wave, r, lane), key[r], val[r]);
  // this block's output offset of digit threadIdx.x
  uint32_t base;
  if (FUSED) {
    const uint32_t* h = hist + ((int64_t)j * 256 + threadIdx.x) * nb;
    uint32_t pre = 0, tot = 0;
    for (int b0 = 0; b0 < nb; b0 += 16) {  // 16 loads in flight at a time
      uint32_t c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) c[u] = b0 + u < nb ? h[b0 + u] : 0u;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        tot += c[u];
        pre += b0 + u < blk ? c[u] : 0u;
      }
    }
    uint32_t incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t wb = 0;
    for (int w = 0; w < wave; ++w) wb += wtot[w];
    base = wb + incl - tot + pre;
  } else {
    base = hist[((int64_t)j * 256 + threadIdx.x) * nb + blk];
  }
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) wcount[w][threadIdx.x] = 0;
  __syncthreads();
  const uint64_t lt = lanes_below(lane);
  uint32_t rank[kSortItems];
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const bool valid = tile_pos(blk, wave, r, lane) < N;
    const uint32_t dg = (key[r] >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t bal = __ballot((dg >> bit) & 1u);
      peers &= ((dg >> bit) & 1u) ? bal : ~bal;
    }
    const uint32_t below = (uint32_t)__popcll(peers & lt);
    // One wave's LDS accesses complete in issue order: every peer reads the
    // count before its first peer writes the new one.
    const uint32_t before = wcount[wave][dg];
    rank[r] = before + below;
    __builtin_amdgcn_wave_barrier();
    if (valid && below == 0) wcount[wave][dg] = before + (uint32_t)__popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // Digit d of this block: its keys' offsets among themselves (per wave), the
  // start of its run in the block's digit order, and the shift from there to
  // its output position.
  {
    uint32_t cnt = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) {
      const uint32_t c = wcount[w][threadIdx.x];
      wcount[w][threadIdx.x] = cnt;
      cnt += c;
    }
    uint32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wtot2[wave] = incl;
    __syncthreads();
    uint32_t loc = incl - cnt;
    for (int w = 0; w < wave; ++w) loc += wtot2[w];
    dstart[threadIdx.x] = loc;
    dshift[threadIdx.x] = base - loc;  // mod 2^32
  }
  __syncthreads();
  // the block's keys in digit order in LDS, then written out in that order:
  // each digit's keys go to consecutive output positions
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    if (tile_pos(blk, wave, r, lane) < N) {
      const uint32_t dg = (key[r] >> shift) & 255u;
      const uint32_t lp = dstart[dg] + wcount[wave][dg] + rank[r];
      ks[lp] = key[r];
      vs[lp] = val[r];
    }
  }
  __syncthreads();
  const int64_t left = N - (int64_t)blk * kSortTile;
  const int nvalid = left < kSortTile ? (int)left : kSortTile;
  uint32_t* ko = kout + j * N;
  uint32_t* vo = vout + j * N;
  for (int i = threadIdx.x; i < nvalid; i += kSortThreads) {
    const uint32_t k = ks[i];
    const uint32_t pos = dshift[(k >> shift) & 255u] + (uint32_t)i;
    ko[pos] = k;
    vo[pos] = vs[i];
  }
}

// Heads of segments: the first key of a table and every key that differs
// from the one before it.

// number of segment heads per block of sorted keys
__global__ __launch_bounds__(256) void seg_count_kernel(const uint32_t* __restrict__ keys,
                                                        uint32_t* __restrict__ seg_count,
                                                        int64_t N, int nb) {
  __shared__ uint32_t tot;
  const int j = blockIdx.y;
  const int blk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x == 0) tot = 0;
  const uint32_t* k = keys + j * N;
  uint32_t kv[kSortItems], pv[kSortItems];  // all loads in flight together
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t p = tile_pos(blk, wave, r, lane);
    kv[r] = p < N ? k[p] : 0u;
    pv[r] = p > 0 && p < N ? k[p - 1] : ~kv[r];
  }
  uint32_t c = 0;
#pragma unroll
  for (int r = 0; r < kSortItems; ++r)
    c += (uint32_t)__popcll(__ballot(tile_pos(blk, wave, r, lane) < N && kv[r] != pv[r]));
  __syncthreads();
  if (lane == 0) atomicAdd(&tot, c);
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

// Keys and head flags of a wave's positions, and the number of heads before
// the wave's first position (block's scanned count plus the heads of the
// waves before it).
__device__ __forceinline__ uint32_t seg_wave_base(const uint32_t* __restrict__ k,
                                                  const uint32_t* __restrict__ seg_count,
                                                  int64_t N, int nb, uint32_t (&kv)[kSortItems],
                                                  uint64_t (&bal)[kSortItems], uint32_t* wtot) {
  const int j = blockIdx.y;
  const int blk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  bool h[kSortItems];
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t p = tile_pos(blk, wave, r, lane);
    kv[r] = p < N ? k[p] : 0u;
    h[r] = p < N && (p == 0 || kv[r] != k[p - 1]);
  }
  uint32_t c = 0;
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    bal[r] = __ballot(h[r]);
    c += (uint32_t)__popcll(bal[r]);
  }
  if (lane == 0) wtot[wave] = c;
  __syncthreads();
  uint32_t base = seg_count[j * nb + blk];
  for (int w = 0; w < wave; ++w) base += wtot[w];
  return base;
}

// seg_start / seg_key of every head, in sorted order, and (when seg_tok is
// given) the token of its first element
__global__ __launch_bounds__(256) void seg_write_kernel(const uint32_t* __restrict__ keys,
                                                        const uint32_t* __restrict__ vals,
                                                        const uint32_t* __restrict__ seg_count,
                                                        uint32_t* __restrict__ seg_start,
                                                        uint64_t* __restrict__ seg_key,
                                                        uint32_t* __restrict__ seg_tok, int64_t N,
                                                        int nb) {
  __shared__ uint32_t wtot[kSortWaves];
  const int j = blockIdx.y;
  const int blk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint32_t* k = keys + j * N;
  uint32_t tv[kSortItems];
  if (seg_tok) {
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
      const int64_t p = tile_pos(blk, wave, r, lane);
      tv[r] = p < N ? vals[j * N + p] : 0u;
    }
  }
  uint32_t kv[kSortItems];
  uint64_t bal[kSortItems];
  uint32_t base = seg_wave_base(k, seg_count, N, nb, kv, bal, wtot);
  const uint64_t lt = lanes_below(lane);
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t p = tile_pos(blk, wave, r, lane);
    if ((bal[r] >> lane) & 1ull) {
      const uint32_t s = base + (uint32_t)__popcll(bal[r] & lt);
      seg_start[s] = (uint32_t)(j * N + p);
      seg_key[s] = ((uint64_t)j << 32) | kv[r];
      if (seg_tok) seg_tok[s] = tv[r];
    }
    base += (uint32_t)__popcll(bal[r]);
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
  __shared__ uint32_t wtot[kSortWaves];
  const int j = blockIdx.y;
  const int blk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint32_t* k = keys + j * N;
  const uint32_t* v = vals + j * N;
  uint32_t tv[kSortItems];
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t p = tile_pos(blk, wave, r, lane);
    tv[r] = p < N ? v[p] : 0u;
  }
  uint32_t kv[kSortItems];
  uint64_t bal[kSortItems];
  uint32_t base = seg_wave_base(k, seg_count, N, nb, kv, bal, wtot);
  const uint64_t le = ~0ull >> (63 - lane);
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t p = tile_pos(blk, wave, r, lane);
    if (p < N) inverse[(int64_t)tv[r] * J + j] = (int32_t)(base + (uint32_t)__popcll(bal[r] & le) - 1);
    base += (uint32_t)__popcll(bal[r]);
  }
}

// Segmented reduce.  Block b owns segments [b*kSegsPerBlock, ...).  A wave
// holds S = 64 / (D/4) lane groups of D/4 lanes (one 16-byte column piece per
// lane), a block G = 4*S groups.  A Zipf-heavy row can have hundreds of
// elements: segments of kLongSeg or more are summed first, by the whole
// block, group g taking elements g, g+G, ... in order, and the G partial
// sums are then added in group order.  Nearly every other segment has one
// element; a group takes kRedBatch consecutive segments at a time, with the
// first rows of all of them in flight together and the bounds, keys and
// first tokens of its next batch loading behind them, and sums the rest of a
// segment's elements in sorted order.  Both orders depend only on D, so
// results repeat run to run.
constexpr int kSegsPerBlock = ENGRAM_RED_SEGS;
constexpr int kLongSeg = 32;
constexpr int kRedBatch = ENGRAM_RED_BATCH;

__device__ __forceinline__ floatx4 load_row_piece(const float* p) {
#if (ENGRAM_SCATTER_NT & 1) != 0
  return __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
#else
  return *reinterpret_cast<const floatx4*>(p);
#endif
}

template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void seg_reduce_kernel(ScatterArgs a, const uint32_t* __restrict__ vals,
                                                         const uint32_t* __restrict__ seg_start,
                                                         const uint64_t* __restrict__ seg_key,
                                                         const uint32_t* __restrict__ seg_tok,
                                                         const uint32_t* __restrict__ total) {
  constexpr int kScan = (kSegsPerBlock + 255) / 256;
  __shared__ floatx4 part[256];  // G * D/4 = 4 * S * D/4 <= 256
  __shared__ uint32_t lst[kSegsPerBlock];
  __shared__ uint32_t nl;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int D4 = a.D / 4;  // <= 64 (D <= 256)
  const int S = 64 / D4;
  const int G = 4 * S;
  const int grp = lane / D4;
  const int col = lane - grp * D4;
  const bool act = grp < S;
  const int gi = wave * S + grp;
  const uint32_t U = total[0];
  const uint32_t s0 = blockIdx.x * (uint32_t)kSegsPerBlock;
#if !ENGRAM_RED_GRID_STRIDE
  if (s0 >= U) return;  // block-uniform
#endif
  const uint32_t s1 = min(s0 + (uint32_t)kSegsPerBlock, U);
  const uint32_t NJ = (uint32_t)(a.N * a.J);
  const int64_t dm = (int64_t)a.J * a.D;
  auto start_of = [&](uint32_t s) -> uint32_t { return s < U ? seg_start[s] : NJ; };
  auto row = [&](uint64_t key, uint32_t t) -> floatx4 {
    return load_row_piece(a.de + (int64_t)t * dm + (int64_t)(key >> 32) * a.D + col * 4);
  };
  auto emit = [&](uint32_t seg, uint64_t key, floatx4 acc) {
    const int j = (int)(key >> 32);
    const int64_t r = (int64_t)(key & 0xFFFFFFFFu);
    if (MODE == ENGRAM_GRAD_SORTED_SPARSE) {
      floatx4* p = reinterpret_cast<floatx4*>(a.rows_out + (int64_t)seg * a.D + col * 4);
      if constexpr ((ENGRAM_SCATTER_NT & 2) != 0)
        __builtin_nontemporal_store(acc, p);
      else
        *p = acc;
      if (col == 0) a.keys_out[seg] = (int64_t)key;
    } else {
      floatx4* dst = reinterpret_cast<floatx4*>(a.dense[j] + r * a.D + col * 4);
      *dst = *dst + acc;
    }
  };
  const floatx4 zero = floatx4{0.f, 0.f, 0.f, 0.f};

  // long segments of the block's range, whole block
  if (threadIdx.x == 0) nl = 0;
  __syncthreads();
  {
    uint32_t len[kScan];
#pragma unroll
    for (int c = 0; c < kScan; ++c) {
      const uint32_t s = s0 + c * 256 + threadIdx.x;
      len[c] = s < s1 && c * 256 + (int)threadIdx.x < kSegsPerBlock ? start_of(s + 1) - seg_start[s] : 0u;
    }
#pragma unroll
    for (int c = 0; c < kScan; ++c)
      if (len[c] >= (uint32_t)kLongSeg) lst[atomicAdd(&nl, 1u)] = s0 + c * 256 + threadIdx.x;
  }
  __syncthreads();
  const uint32_t n_long = nl;
  for (uint32_t i = 0; i < n_long; ++i) {
    const uint32_t sl = lst[i];
    const uint32_t beg = seg_start[sl];
    const uint32_t end = start_of(sl + 1);
    const uint64_t key = seg_key[sl];
    if (act) {
      floatx4 acc = zero;
      for (uint32_t p = beg + gi; p < end; p += (uint32_t)(G * kRedBatch)) {
        uint32_t t[kRedBatch];
#pragma unroll
        for (int u = 0; u < kRedBatch; ++u) {
          const uint32_t q = p + (uint32_t)(u * G);
          t[u] = q < end ? vals[q] : 0u;
        }
        floatx4 x[kRedBatch];
#pragma unroll
        for (int u = 0; u < kRedBatch; ++u)
          x[u] = p + (uint32_t)(u * G) < end ? row(key, t[u]) : zero;
#pragma unroll
        for (int u = 0; u < kRedBatch; ++u) acc += x[u];
      }
      part[gi * D4 + col] = acc;
    }
    __syncthreads();
    if (threadIdx.x < D4) {  // wave 0, group 0: col == threadIdx.x
      floatx4 sum = part[threadIdx.x];
      for (int g = 1; g < G; ++g) sum += part[g * D4 + threadIdx.x];
      emit(sl, key, sum);
    }
    __syncthreads();
  }

  // the other segments, kRedBatch consecutive ones per group
  if (!act) return;
#if ENGRAM_RED_GRID_STRIDE
  const uint32_t b_end = U;
  const uint32_t b_first = (blockIdx.x * (uint32_t)G + (uint32_t)gi) * kRedBatch;
  const uint32_t b_step = gridDim.x * (uint32_t)G * kRedBatch;
#else
  const uint32_t b_end = s1;
  const uint32_t b_first = s0 + (uint32_t)(gi * kRedBatch);
  const uint32_t b_step = (uint32_t)(G * kRedBatch);
#endif
  uint32_t st[kRedBatch + 1];
  uint64_t key[kRedBatch];
  uint32_t tok[kRedBatch];
  auto load_meta = [&](uint32_t sb) {
#pragma unroll
    for (int u = 0; u <= kRedBatch; ++u) st[u] = start_of(sb + u);
#pragma unroll
    for (int u = 0; u < kRedBatch; ++u) {
      const bool in = sb + u < b_end;
      key[u] = in ? seg_key[sb + u] : 0ull;
      tok[u] = in ? seg_tok[sb + u] : 0u;
    }
  };
  uint32_t sb = b_first;
  if (sb < b_end) load_meta(sb);
  for (; sb < b_end; sb += b_step) {
    bool ok[kRedBatch];
    floatx4 x[kRedBatch];
    uint32_t cst[kRedBatch + 1];
    uint64_t ckey[kRedBatch];
#pragma unroll
    for (int u = 0; u < kRedBatch; ++u) {
      ok[u] = sb + u < b_end && st[u + 1] - st[u] < (uint32_t)kLongSeg;
      x[u] = ok[u] ? row(key[u], tok[u]) : zero;
    }
#pragma unroll
    for (int u = 0; u <= kRedBatch; ++u) cst[u] = st[u];
#pragma unroll
    for (int u = 0; u < kRedBatch; ++u) ckey[u] = key[u];
    const uint32_t next = sb + b_step;
#if ENGRAM_RED_PREFETCH
    if (next < b_end) load_meta(next);
#endif
#pragma unroll
    for (int u = 0; u < kRedBatch; ++u) {
      if (!ok[u]) continue;
      for (uint32_t p = cst[u] + 1; p < cst[u + 1]; p += 4) {
        uint32_t tt[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) tt[v] = p + v < cst[u + 1] ? vals[p + v] : 0u;
        floatx4 y[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) y[v] = p + v < cst[u + 1] ? row(ckey[u], tt[v]) : zero;
#pragma unroll
        for (int v = 0; v < 4; ++v) x[u] += y[v];
      }
      emit(sb + u, ckey[u], x[u]);
    }
#if !ENGRAM_RED_PREFETCH
    if (next < b_end) load_meta(next);
#endif
  }
}

// Stable sort of every table's (row id, token) pairs by row id: one digit
// pass per 8 bits of the largest row id, the first reading idx itself.
// Returns the ping-pong buffer that holds the result.
static int sort_pairs(const int32_t* idx, int64_t N, int J, int key_bits, const SortBufs& b,
                      hipStream_t s) {
  const int nb = (int)sort_blocks(N);
  const bool fused = nb <= kFusedScanBlocks;
  const int passes = key_bits > 8 ? (key_bits + 7) / 8 : 1;
  const dim3 grid(nb, J);
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * 8;
    const int in = (pass - 1) & 1, out = pass & 1;
    if (pass == 0)
      hipLaunchKernelGGL(sort_hist_kernel<true>, grid, dim3(kSortThreads), 0, s, idx, nullptr, b.hist,
                         N, J, shift, nb);
    else
      hipLaunchKernelGGL(sort_hist_kernel<false>, grid, dim3(kSortThreads), 0, s, idx, b.keys[in],
                         b.hist, N, J, shift, nb);
    if (!fused) hipLaunchKernelGGL(sort_scan_kernel, dim3(J), dim3(256), 0, s, b.hist, nb);
    const uint32_t* kin = pass ? b.keys[in] : nullptr;
    const uint32_t* vin = pass ? b.vals[in] : nullptr;
    if (pass == 0 && fused)
      hipLaunchKernelGGL((sort_scatter_kernel<true, true>), grid, dim3(kSortThreads), 0, s, idx, kin,
                         vin, b.keys[out], b.vals[out], b.hist, N, J, shift, nb);
    else if (pass == 0)
      hipLaunchKernelGGL((sort_scatter_kernel<true, false>), grid, dim3(kSortThreads), 0, s, idx, kin,
                         vin, b.keys[out], b.vals[out], b.hist, N, J, shift, nb);
    else if (fused)
      hipLaunchKernelGGL((sort_scatter_kernel<false, true>), grid, dim3(kSortThreads), 0, s, idx, kin,
                         vin, b.keys[out], b.vals[out], b.hist, N, J, shift, nb);
    else
      hipLaunchKernelGGL((sort_scatter_kernel<false, false>), grid, dim3(kSortThreads), 0, s, idx,
                         kin, vin, b.keys[out], b.vals[out], b.hist, N, J, shift, nb);
  }
  return (passes - 1) & 1;
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
  const int cur = sort_pairs(a.idx, N, J, a.key_bits, b, s);
  hipLaunchKernelGGL(seg_count_kernel, dim3(nb, J), dim3(256), 0, s, b.keys[cur], b.seg_count, N, nb);
  hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(1024), 0, s, b.seg_count, nb * J, b.total,
                     mode == ENGRAM_GRAD_SORTED_SPARSE ? a.count_out : nullptr);
  // the first token of every segment goes to the spare ping-pong buffer
  uint32_t* seg_tok = b.vals[cur ^ 1];
  hipLaunchKernelGGL(seg_write_kernel, dim3(nb, J), dim3(256), 0, s, b.keys[cur], b.vals[cur],
                     b.seg_count, b.seg_start, b.seg_key, seg_tok, N, nb);
  // at most N*J segments; blocks past the actual count return at once
  const int64_t max_segs = N * J;
  const unsigned blocks = (unsigned)((max_segs + kSegsPerBlock - 1) / kSegsPerBlock);
  if (mode == ENGRAM_GRAD_SORTED_SPARSE)
    hipLaunchKernelGGL(seg_reduce_kernel<ENGRAM_GRAD_SORTED_SPARSE>, dim3(blocks), dim3(256), 0, s, a,
                       b.vals[cur], b.seg_start, b.seg_key, seg_tok, b.total);
  else
    hipLaunchKernelGGL(seg_reduce_kernel<ENGRAM_GRAD_SORTED_DENSE>, dim3(blocks), dim3(256), 0, s, a,
                       b.vals[cur], b.seg_start, b.seg_key, seg_tok, b.total);
  return hipGetLastError();
}

hipError_t launch_dedup(const int32_t* idx, int64_t N, int32_t J, int32_t key_bits,
                        const SortBufs& b, int32_t* inverse, hipStream_t s) {
  if (N == 0) {  // zero heads: total 0
    hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(1024), 0, s, b.seg_count, 0, b.total, nullptr);
    return hipGetLastError();
  }
  const int nb = (int)sort_blocks(N);
  const int cur = sort_pairs(idx, N, J, key_bits, b, s);
  hipLaunchKernelGGL(seg_count_kernel, dim3(nb, J), dim3(256), 0, s, b.keys[cur], b.seg_count, N, nb);
  hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(1024), 0, s, b.seg_count, nb * J, b.total, nullptr);
  hipLaunchKernelGGL(seg_write_kernel, dim3(nb, J), dim3(256), 0, s, b.keys[cur], b.vals[cur],
                     b.seg_count, b.seg_start, b.seg_key, nullptr, N, nb);
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
