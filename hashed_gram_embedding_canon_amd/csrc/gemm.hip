// Key/value projections ("DeepSeek AI II", section "DeepSeek Engram": the
// retrieved memory e_t is the shared input of the key and value
// projections W_K, W_V) and the backward contraction de = W_K^T dk + W_V^T dv,
// on CDNA4 matrix cores.
//
// Formulation: C^T[f][m] = sum_k A[f][k] B[m][k] with A = the weight rows
// (output features f, K contiguous) and B = the token rows (K contiguous).
// Features are the MFMA row dimension and tokens the column dimension, so
// each lane of a 32x32 accumulator block owns one token and 16 of its
// features.  That makes the gate's per-token reductions (sum k^2,
// sum g_q g_k h k, sum h^2) plain in-register sums in the epilogue: the key
// goes to HBM only when the caller saves it, and h is read exactly once, here.
//
// Row gather fused into the B operand: with GATHER, the 16-byte pieces of a
// token row of B are read straight from the embedding tables through the
// tile's row indices (kept in LDS), so the concatenated memory vector e_t is
// never written to or read back from HBM.
//
// Tiling: 256 features x 256 tokens per workgroup of 4 wavefronts, each
// owning a 128 x 128 block (16 accumulators of 32x32).  K advances 128 bytes
// per stage through two LDS buffers (or 64 bytes through four) filled by
// direct-to-LDS 16-byte global loads (no staging registers); the 16-byte
// pieces of a row are XOR-swizzled (Stage::swz) so that the ds_read_b128 of
// 32-row fragments hit distinct banks.  Matrix cores:
// v_mfma_f32_32x32x16_bf16 / _f16, v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// scales for E4M3; fp32 inputs use four v_mfma_f32_32x32x2f32 per 16-byte
// fragment.  The grid is persistent (one workgroup per CU).  Workgroup ids
// reach the 8 XCDs round-robin; the id -> tile map keeps the f-tiles of a
// small group of token tiles on one XCD so they share rows and weight slabs
// in its L2.  In the bf16 projection a workgroup loads the first K stage of
// its next tile while it finishes the current one, and every tile's first K
// step writes its accumulators (zero C operand), so tiles follow each other
// without a load wait or zeroing writes.
#include <algorithm>
#include <type_traits>

#include "kernels.h"
#include "mfma_ring.h"

namespace engram {

// 4 consecutive values of an io tensor (bf16 or fp32) as floats.
__device__ inline floatx4 load4(const uint8_t* base, int64_t i, int io) {
  if (io == ENGRAM_BF16) {
    const u32x2 u = *reinterpret_cast<const u32x2*>(base + i * 2);
    return floatx4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                   __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
  }
  return *reinterpret_cast<const floatx4*>(base + i * 4);
}

__device__ inline void store4(uint8_t* base, int64_t i, int io, float a, float b, float c, float d) {
  if (io == ENGRAM_BF16) {
    u32x2 u;
    u.x = pack_bf16x2(a, b);
    u.y = pack_bf16x2(c, d);
    *reinterpret_cast<u32x2*>(base + i * 2) = u;
  } else {
    *reinterpret_cast<floatx4*>(base + i * 4) = floatx4{a, b, c, d};
  }
}

constexpr int kBF = kGemmBF;  // features per tile
constexpr int kBT = 256;      // tokens per tile
constexpr int kNT = 256;      // threads (4 waves)
constexpr int kGatherMaxJ = 16;
constexpr int kRedFloats = 2 * 2 * 4 * 32 * 3;  // [2 wf][2 wt][4 blocks][32 tokens][3 sums]

// Stage shapes: SB bytes of K per row and stage.  64-byte stages use a
// 4-deep ring (loads 3 stages ahead), 128-byte stages a 2-deep ring; both
// fill 128 KB of LDS.  16-byte pieces of a row are XOR-swizzled so that the
// fragment reads of 32 consecutive rows hit distinct banks for both 8- and
// 16-lane LDS phases (found by exhaustive search over XOR maps of the row
// bits 0..3).
template <int SB>
struct Stage {
  static constexpr int kStages = SB == 64 ? 4 : 2;
  static constexpr int kOperandBytes = 256 * SB;   // one operand, one stage
  static constexpr int kPieces = SB / 16;          // 16-byte pieces per row
  static constexpr int kRowsPerLoad = 1024 / SB;   // rows one wave-wide load fills
  static constexpr int kLoadsPerOperand = SB / 16; // per wave and stage
  static constexpr int kKSteps = SB / 32;          // 16-element (bf16) MFMA steps
  __device__ static int swz(int r) {
    if constexpr (SB == 64)
      return ((r >> 1) ^ (r >> 3)) & 3;
    else
      return (r & 7) ^ ((r >> 3) & 1);
  }
};

#ifndef ENGRAM_GEMM_SPREAD
#define ENGRAM_GEMM_SPREAD 1
#endif
// Spread the next stage's load instructions between MFMA groups (1) or issue
// them in one burst at the start of a stage (0).
constexpr bool kSpreadLoads = ENGRAM_GEMM_SPREAD != 0;
#ifndef ENGRAM_GEMM_LOAD_GROUPS
#define ENGRAM_GEMM_LOAD_GROUPS 10
#endif
// Spread over the first this many MFMA groups of a stage (the later groups
// issue no loads), so the last load of the next stage has the rest of the
// stage to land before the wait at its end.  Of the 16 groups of a 128-byte
// stage, the first 10 measured best at the 27B shape: 1.540 ms per
// projection against 1.630 ms with one load after every group (8 and 12:
// 1.549 and 1.543 ms; 6: 1.575 ms).
constexpr int kLoadGroups = ENGRAM_GEMM_LOAD_GROUPS;
#ifndef ENGRAM_GEMM_EARLY_BARRIER
#define ENGRAM_GEMM_EARLY_BARRIER 1
#endif
#ifndef ENGRAM_GEMM_LATE
#define ENGRAM_GEMM_LATE 6
#endif
#ifndef ENGRAM_GEMM_EARLY_PER
#define ENGRAM_GEMM_EARLY_PER 2
#endif
#ifndef ENGRAM_GEMM_H1_LATE
#define ENGRAM_GEMM_H1_LATE 0
#endif
#ifndef ENGRAM_GEMM_V_NT
#define ENGRAM_GEMM_V_NT 0
#endif
// Row stores of a value tile's epilogue unrolled this far (all 16 LDS reads
// of a pass in flight): 1.485 ms per projection against 1.494 ms with 4.
#ifndef ENGRAM_GEMM_VSTORE_UNROLL
#define ENGRAM_GEMM_VSTORE_UNROLL 16
#endif
constexpr int kVStoreUnroll = ENGRAM_GEMM_VSTORE_UNROLL;
#ifndef ENGRAM_GEMM_PREFETCH_TILE
#define ENGRAM_GEMM_PREFETCH_TILE 1
#endif
// key tiles: 0 = no early stage-0 load, 1 = before token blocks 2 and 3 are
// summed, 2 = between blocks 2 and 3
// Each K stage of the bf16 projection also fetches the workgroup's eighth of
// its B tile's rows three stages ahead into L2 (into LDS scratch that nothing
// reads), so the tiles that meet a token tile first do not wait for HBM at
// every stage.
#ifndef ENGRAM_GEMM_PREFETCH_E
#define ENGRAM_GEMM_PREFETCH_E 1
#endif
// The same in the de contraction (five f-tiles share a token tile: two loads
// per wave and stage, 64 rows per workgroup).
#ifndef ENGRAM_GEMM_PREFETCH_E_DE
#define ENGRAM_GEMM_PREFETCH_E_DE 1
#endif
// The de contraction can load its next tile's stage 0 early too (in the load
// slots of its last two stages; its epilogue stores from the accumulators):
// its prologue drops from 3.3-5K to 1.4K cycles, yet the kernel time stays
// the same (1.4261 against 1.4271 ms), so it is off.
#ifndef ENGRAM_GEMM_PREFETCH_TILE_DE
#define ENGRAM_GEMM_PREFETCH_TILE_DE 0
#endif
#ifndef ENGRAM_GEMM_PREFETCH_KEY
#define ENGRAM_GEMM_PREFETCH_KEY 1
#endif
// Load stage 0 of a workgroup's next tile while this one finishes (bf16
// key/value projection): value tiles in the load slots of their last K stage,
// key tiles once the first half of their gate sums has freed that buffer.

#ifdef ENGRAM_GEMM_TRACE
// Measurement build only: shader-clock stamps of workgroups 0..31 (wave 0),
// per tile: start, K loop done, epilogue done, first stage landed, epilogue
// midpoint, epilogue stores issued, set-up done, first-stage wait done, key
// tiles' first h part landed; per stage of their second tile.
constexpr int kTrWG = 32, kTrTiles = 48, kTrStages = 96, kTrPer = 9;
__device__ uint64_t g_gemm_trace[kTrWG * kTrTiles * kTrPer + kTrWG * kTrStages + 2];
#define ENGRAM_TRACE_TILE(which)                                                          \
  do {                                                                                    \
    if (threadIdx.x == 0 && blockIdx.x < kTrWG && it_ < kTrTiles)                         \
      g_gemm_trace[(blockIdx.x * kTrTiles + it_) * kTrPer + (which)] =                    \
          __builtin_readcyclecounter();                                                   \
  } while (0)
#define ENGRAM_TRACE_STAGE(k)                                                             \
  do {                                                                                    \
    if (threadIdx.x == 0 && blockIdx.x < kTrWG && it_ == 1 && (k) < kTrStages)           \
      g_gemm_trace[kTrWG * kTrTiles * kTrPer + blockIdx.x * kTrStages + (k)] =           \
          __builtin_readcyclecounter();                                                   \
  } while (0)
// per wave (lane 0), workgroups 0..7, second tile: stamp w of stage k
constexpr int kTr2WG = 8, kTr2Stages = 24;
__device__ uint64_t g_gemm_trace2[kTr2WG * kTr2Stages * 4 * 3];
#define ENGRAM_TRACE_W(k, w)                                                               \
  do {                                                                                     \
    if ((threadIdx.x & 63) == 0 && blockIdx.x < kTr2WG && it_ == 1 && (k) < kTr2Stages)   \
      g_gemm_trace2[((blockIdx.x * kTr2Stages + (k)) * 4 + (threadIdx.x >> 6)) * 3 + (w)] = \
          __builtin_readcyclecounter();                                                    \
  } while (0)
#else
#define ENGRAM_TRACE_TILE(which) \
  do {                           \
  } while (0)
#define ENGRAM_TRACE_STAGE(k) \
  do {                        \
  } while (0)
#define ENGRAM_TRACE_W(k, w) \
  do {                       \
  } while (0)
#endif
// what the load slots of a K stage carry
constexpr int kSlotNext = 0, kSlotNone = 1, kSlotH = 2;  // kSlotH + X: part X of h
// the last two K stages with the next-tile prefetch: h part 0 (key tiles),
// the next tile's stage 0 (value tiles), chosen per tile without branches
constexpr int kSlotTail = -1;
template <int X>
using SlotHPart = std::integral_constant<int, kSlotH + X>;

template <int GT, int EPI, bool GATHER, int SB>
__global__ __launch_bounds__(kNT) void gemm_kernel(GemmArgs g) {
  using S = Stage<SB>;
  constexpr int NS = S::kStages;
  constexpr int ES = (GT == GEMM_F32) ? 4 : (GT == GEMM_FP8 ? 1 : 2);
  constexpr int FB = 4, TB = 4;  // 32-blocks per wave along f and tokens
  constexpr int kTS = S::kOperandBytes;
  // One LDS object per stage (A then B): the compiler tracks the direct-to-LDS
  // writes of each object separately, so reading stage k does not make it
  // wait for the loads still in flight into the other stages.  The epilogue
  // reuses them.
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * kTS];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[2 * kTS];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[NS > 2 ? 2 * kTS : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[NS > 2 ? 2 * kTS : 16];
  // row indices of the tile (fused gather), later the gate reduction buffer
  __shared__ __attribute__((aligned(16))) int32_t sIdx[GATHER ? kBT * kGatherMaxJ : kRedFloats + kBF];
  int32_t* const sIdxOrRed = sIdx;
  __shared__ const uint8_t* sTab[GATHER ? kGatherMaxJ : 1];
  // E4M3: the dequantization scales of the tile's 256 A rows (features)
  __shared__ __attribute__((aligned(16))) float sScaleA[GT == GEMM_FP8 ? kBF : 1];

  // ---- workgroup id -> (token tile, feature tile), XCD-grouped.  XCD list x
  // holds the token tiles x, x+8, ... in groups of group_m; its slots run
  // over a group's f-tiles, each f-tile over the group's token tiles, so the
  // f-tiles of a group share rows and weight slabs in one XCD's L2.  A grid
  // of fewer workgroups than slots makes each workgroup of list x
  // (workgroups x, x+8, ...) loop over slots s, s + gridDim/8, ...
  // (persistent: no per-tile dispatch gap).
  const int xcd = blockIdx.x & 7;
  const int slot_step = gridDim.x >> 3;
  const int tiles_f = g.F / kBF;
  const int64_t tiles_m = (g.M + kBT - 1) / kBT;
  const int tx = xcd < tiles_m ? (int)((tiles_m - 1 - xcd) / 8 + 1) : 0;  // token tiles of list x
  const int nslots = tx * tiles_f;
  auto tile_of = [&](int sl, int64_t& tm_o, int& f0_o) __attribute__((always_inline)) {
    const int gm = g.group_m;
    const int per_group = gm * tiles_f;
    const int grp = sl / per_group;
    const int in_g = sl - grp * per_group;
    const int full = tx / gm;                          // groups of group_m token tiles
    const int gsz = grp < full ? gm : tx - full * gm;  // token tiles in this group
    const int tf = in_g / gsz;
    const int tm_local = in_g - tf * gsz;
    const int64_t tm_fwd = (int64_t)(grp * gm + tm_local) * 8 + xcd;  // < tiles_m
    // token tiles walked last to first when asked (the newest rows of B first)
    tm_o = g.reverse_m ? tiles_m - 1 - tm_fwd : tm_fwd;
    f0_o = tf * kBF;
  };
  constexpr bool kPrefetchTile =
      ENGRAM_GEMM_PREFETCH_TILE && ENGRAM_GEMM_EARLY_BARRIER && S::kStages == 2 && !GATHER &&
      ((GT == GEMM_BF16 && EPI == EPI_KV) ||
       (ENGRAM_GEMM_PREFETCH_TILE_DE && GT == GEMM_F16 && EPI == EPI_STORE_F32));
  // how this tile's stage 0 was loaded: 0 by its own prologue; else by the
  // previous tile, followed there by 1: exactly 32 row stores per wave (a
  // whole value tile), 2: an unknown number of stores, 3: 64 stores per wave
  // (a whole tile of the de contraction)
  int pf_kind = 0;
  // this tile's coordinates, found by the previous iteration (the mapping
  // costs three integer divisions)
  int64_t tm_c = 0;
  int f0_c = 0;
  if ((int)(blockIdx.x >> 3) < nslots) tile_of(blockIdx.x >> 3, tm_c, f0_c);
  for (int slot = blockIdx.x >> 3; slot < nslots; slot += slot_step) {
  [[maybe_unused]] const int it_ = (slot - (int)(blockIdx.x >> 3)) / slot_step;
  ENGRAM_TRACE_TILE(0);
  const int64_t tm = tm_c;
  const int f0 = f0_c;
  const int64_t m0 = tm * kBT;
  // the next tile of this workgroup; with kPrefetchTile its stage 0 is loaded
  // early when it is a whole token tile (its B rows need no clamping)
  int64_t tmn = 0;
  int f0n = 0;
  const bool has_next = slot + slot_step < nslots;
  if (has_next) tile_of(slot + slot_step, tmn, f0n);
  const bool pf_next = kPrefetchTile && has_next && (tmn + 1) * kBT <= g.M;
  // EPI_KV output features: the keys of `branches` branches (d each), then v.
  // A feature tile lies inside one branch key or inside v (d % 256 == 0);
  // fk is its first feature there.  h, gamma, k and the partial sums of a
  // branch sit branch-major ([branch][M][d], [branch][d], [branch][M][d/256][3]).
  const int nbr = g.branches > 0 ? g.branches : 1;
  const bool key_tile = EPI == EPI_KV && f0 < nbr * g.d;
  const int br = key_tile ? f0 / g.d : 0;
  const int fk = EPI != EPI_KV ? 0 : (key_tile ? f0 - br * g.d : f0 - nbr * g.d);
  constexpr int HSZ = GT == GEMM_F32 ? 4 : 2;  // bytes per element of h, k, v
  const int64_t bstride = g.M * (int64_t)g.d;   // elements from one branch to the next
  const uint8_t* const hB = EPI == EPI_KV ? g.h + br * bstride * HSZ : nullptr;
  const float* const gqB = g.gamma_q ? g.gamma_q + br * g.d : nullptr;
  const float* const gkB = g.gamma_k ? g.gamma_k + br * g.d : nullptr;
  float* const partB = EPI == EPI_KV ? g.partials + br * g.M * (g.d / kBF) * 3 : nullptr;
  uint8_t* const koutB = g.k_out ? g.k_out + br * bstride * HSZ : nullptr;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wf = wave & 1;
  const int wt = wave >> 1;
  const int64_t row_bytes = (int64_t)g.K * ES;
  const int nk = (int)(row_bytes / SB);

  static_assert(kBT == kNT, "one thread per token of the tile");
  if constexpr (GATHER) {
    // thread r stages the J row indices of token m0 + r
    const int J = g.J;
    int64_t m = m0 + tid;
    m = m < g.M ? m : g.M - 1;
    const int32_t* src = g.idx + m * J;
    if ((J & 3) == 0) {
      for (int j = 0; j < J; j += 4)
        *reinterpret_cast<u32x4*>(sIdx + tid * kGatherMaxJ + j) = *reinterpret_cast<const u32x4*>(src + j);
    } else {
      for (int j = 0; j < J; ++j) sIdx[tid * kGatherMaxJ + j] = src[j];
    }
    if (tid < J) sTab[tid] = g.tables[tid];
    __syncthreads();
  }

  // ---- per-lane load descriptors: wave-wide load i of this wave fills rows
  //      ch*kRowsPerLoad .. (ch = wave + 4i); lane -> row ch*kRowsPerLoad +
  //      lane/kPieces, physical 16-byte slot lane % kPieces
  constexpr int NL = S::kLoadsPerOperand;
  // byte offsets of piece i inside the tile's rows (A: rows f0.., B: rows m0..)
  uint32_t voffA[NL], voffB[NL];
  int gj[NL], gw[NL], grow[NL];  // GATHER: table, element offset and local row of the piece at stage 0
  // B rows past the last token repeat it (32-bit offsets: a tile's rows span
  // less than 2^31 bytes, gemm_supported)
  const int last_row = (int)std::min<int64_t>(g.M - 1 - m0, kBT - 1);
  const int rb32 = (int)row_bytes;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int ch = wave + 4 * i;
    const int row = ch * S::kRowsPerLoad + lane / S::kPieces;
    const int c = (lane % S::kPieces) ^ S::swz(row);
    voffA[i] = (uint32_t)(row * rb32 + c * 16);
    voffB[i] = (uint32_t)(std::min(row, last_row) * rb32 + c * 16);
    if constexpr (GATHER) {
      const int e0 = c * 16 / ES;
      gj[i] = e0 / g.D;
      gw[i] = e0 - gj[i] * g.D;
      grow[i] = row;
    } else {
      gj[i] = gw[i] = grow[i] = 0;
    }
  }
  const uint8_t* const tileA = g.A + (int64_t)f0 * row_bytes;
  const uint8_t* const tileB = GATHER ? nullptr : g.B + m0 * row_bytes;
  const uint8_t* const nextA = kPrefetchTile ? g.A + (int64_t)f0n * row_bytes : nullptr;
  const uint8_t* const nextB = kPrefetchTile ? g.B + tmn * kBT * row_bytes : nullptr;
  // B rows fetched ahead: share q = (f-tile mod 8 / kPfEL) of the tile's
  // rows, kPfEL loads of 8 rows per wave (the f-tiles that share a token tile
  // in one pass of the XCD take distinct shares); 16-byte piece lane % 8 of a
  // 128-byte stage
  constexpr bool kPfE =
      ENGRAM_GEMM_PREFETCH_E && SB == 128 && !GATHER &&
      (kPrefetchTile || (ENGRAM_GEMM_PREFETCH_E_DE && EPI == EPI_STORE_F32 && GT == GEMM_F16 &&
                         ENGRAM_GEMM_EARLY_BARRIER && S::kStages == 2));
  constexpr int kPfEL = EPI == EPI_KV ? 1 : 2;
  uint32_t pfe_voff[kPfEL];
#pragma unroll
  for (int l = 0; l < kPfEL; ++l) {
    const int q = (f0 / kBF) % (8 / kPfEL);
    const int row = std::min(q * 32 * kPfEL + l * 32 + wave * 8 + (lane >> 3), last_row);
    pfe_voff[l] = kPfE ? (uint32_t)(row * rb32 + (lane & 7) * 16) : 0u;
  }
  constexpr int kStageElems = SB / ES;
  const int64_t dbytes = (int64_t)g.D * ES;

  // GATHER: (gj, gw) = table and element of piece i at the next stage to
  // issue, (nrow, nbase) = its row index and table base, read from LDS one
  // stage ahead so the loads never wait on those LDS reads.  issue() must be
  // called for kt = 0, 1, 2, ... in order.
  int32_t nrow[NL];
  const uint8_t* nbase[NL];
  if constexpr (GATHER) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      nrow[i] = sIdx[grow[i] * kGatherMaxJ + gj[i]];
      nbase[i] = sTab[gj[i]];
    }
  }
  // ---- bf16 epilogue staging: 256 token rows of 512 bytes (the tile's 256
  // features) in the stage buffers, part X = buffer X.  Token t = 128w +
  // 64u + r (w: wave half, u: which 64 of it) lives in part u (two buffers,
  // row 64w + r) or part 2u + w (four buffers, row r), so the first two
  // token blocks of every wave (u = 0) sit in the first half of the parts.
  constexpr bool kBf16Epi = EPI == EPI_KV && (GT == GEMM_BF16 || GT == GEMM_FP8);
  auto part_base = [&](int X) __attribute__((always_inline)) -> uint8_t* {
    return X == 0 ? st0 : (X == 1 ? st1 : (X == 2 ? st2 : st3));
  };
  auto trow = [&](int t) __attribute__((always_inline)) -> uint8_t* {
    const int w = t >> 7, u = (t >> 6) & 1, r = t & 63;
    if constexpr (NS == 4)
      return part_base(2 * u + w) + r * 512;
    else
      return part_base(u) + (w * 64 + r) * 512;
  };
  // Key tiles load h part by part into buffers as the ring frees them: with
  // two buffers part 0 in the load slots of the last K stage, with four
  // parts 0, 1, 2 in those of the last three; the last part goes out after
  // the loop and lands while the first two token blocks are summed.  Row pair
  // p of part X covers tokens t0, t0+1 (h_t0); lane l takes token t0 + l/32
  // (rows past M repeat the last one) and lands its 16-byte piece
  // (l%32) ^ (t%32) at slot l%32 of the row.  A part is 2*NL row pairs per
  // wave, one per load slot.
  constexpr bool kHOverlap = kBf16Epi;
  const bool hov = kHOverlap && key_tile;
  auto h_t0 = [&](int X, int p) __attribute__((always_inline)) {
    if constexpr (NS == 4)  // 32 pairs: part X = 2u + w
      return ((X & 1) << 7) | ((X >> 1) << 6) | (p << 1);
    else                    // 64 pairs: part X = u
      return ((p >> 5) << 7) | (X << 6) | ((p & 31) << 1);
  };
  auto h_voff = [&](int X, int p) __attribute__((always_inline)) -> uint32_t {
    const int t = h_t0(X, p) + (lane >> 5);
    const int c16 = (lane & 31) ^ (t & 31);
    const int64_t tc = m0 + t < g.M ? t : g.M - 1 - m0;
    return (uint32_t)((tc * g.d + c16 * 8) * 2);
  };
  const void* const hbase = kBf16Epi ? uniform_ptr(hB + (m0 * g.d + fk) * 2) : nullptr;

  // Load slot j of a stage (j = 2i + op): piece i of operand A (op 0) or B
  // (op 1) into the stage buffer at LDS address la (A) / la + kTS (B).
  // bA / bB: uniform_ptr(tileA / tileB + kt * SB), the stage's row bases.
  auto issue_one = [&](const void* bA, const void* bB, uint32_t la, int j)
                       __attribute__((always_inline)) {
    const int i = j >> 1, op = j & 1;
    const uint32_t m0v = la + (uint32_t)((wave + 4 * i) * 1024) + (op ? kTS : 0);
    if (op == 0) {
      load_lds16_s(voffA[i], bA, m0v);
    } else if constexpr (GATHER) {
      load_lds16(nbase[i] + (int64_t)nrow[i] * dbytes + (int64_t)gw[i] * ES, m0v);
      // advance to the next stage: D >= kStageElems, so at most one table boundary
      gw[i] += kStageElems;
      const bool wrap = gw[i] >= g.D;
      gw[i] = wrap ? gw[i] - g.D : gw[i];
      gj[i] = wrap ? gj[i] + 1 : gj[i];
      const int jn = gj[i] < g.J ? gj[i] : g.J - 1;  // past the last stage: any valid entry
      nrow[i] = sIdx[grow[i] * kGatherMaxJ + jn];
      nbase[i] = sTab[jn];
    } else {
      load_lds16_s(voffB[i], bB, m0v);
    }
  };
  // Load slot j of the next tile's stage 0 into buffer 0.  That tile is
  // whole, so its B rows are unclamped and take A's offsets.
  auto issue_tile0 = [&](const void* bA, const void* bB, int j) __attribute__((always_inline)) {
    const int i = j >> 1, op = j & 1;
    const uint32_t m0v = lds_addr(st0) + (uint32_t)((wave + 4 * i) * 1024) + (op ? kTS : 0);
    load_lds16_s(voffA[i], op ? bB : bA, m0v);
  };
  // Load slot j of the tail: the next tile's stage 0 (value tiles with a
  // whole next tile) or else h row pair (2*NL)*wave + j of part 0 (key
  // tiles), a repeated read of h's first 16 bytes into the same rows (other
  // value tiles); all of them land in buffer 0.  Selected per tile, no branch.
  const bool tail_tile0 = kPrefetchTile && !hov && pf_next;
  auto issue_tail = [&](int j) __attribute__((always_inline)) {
    const int i = j >> 1, op = j & 1;
    const int p = 2 * NL * wave + j;
    const uint32_t hv = hov ? h_voff(0, p) : 0u;
    const uint32_t m0t = lds_addr(st0) + (uint32_t)((wave + 4 * i) * 1024) + (op ? kTS : 0);
    if constexpr (kBf16Epi) {
      const uint32_t voff = tail_tile0 ? voffA[i] : hv;
      const void* base = tail_tile0 ? (op ? nextB : nextA) : hbase;
      load_lds16_s(voff, base, tail_tile0 ? m0t : lds_addr(trow(h_t0(0, p))));
    } else {
      // no h here: without a next tile, stage 0 of this one again (valid rows)
      const uint32_t voff = tail_tile0 ? voffA[i] : (op ? voffB[i] : voffA[i]);
      const void* base = tail_tile0 ? (op ? nextB : nextA) : (op ? tileB : tileA);
      load_lds16_s(voff, base, m0t);
    }
  };
  // h row pair (2*NL)*wave + j of part X (load slot j); value tiles (hov
  // false) read the first 16 bytes of the h tile in every lane instead
  auto issue_h = [&](int X, int j) __attribute__((always_inline)) {
    const int p = 2 * NL * wave + j;
    load_lds16_s(hov ? h_voff(X, p) : 0u, hbase, lds_addr(trow(h_t0(X, p))));
  };
  auto stage_base = [&](const uint8_t* tile, int kt) __attribute__((always_inline)) -> const void* {
    return uniform_ptr(tile + (int64_t)kt * SB);
  };
  // all 2*NL load slots of stage kt
  auto issue = [&](int kt, uint32_t la) __attribute__((always_inline)) {
    const void* bA = stage_base(tileA, kt);
    const void* bB = GATHER ? nullptr : stage_base(tileB, kt);
#pragma unroll
    for (int j = 0; j < 2 * NL; ++j) issue_one(bA, bB, la, j);
  };

  floatx16 acc[FB][TB];
#pragma unroll
  for (int a = 0; a < FB; ++a)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[a][b] = floatx16{};

  const int l32 = lane & 31;
  const int lhalf = lane >> 5;
  const int swl = S::swz(l32);  // fragment rows are blk*32 + l32; the swizzle reads bits 0..4 only

  // A fragment is 16 bytes of a row (32-byte K steps), or for E4M3 32 bytes
  // (64-element K steps: pieces 4 ss + 2 lhalf and the next one).
  using Frag = std::conditional_t<GT == GEMM_FP8, u32x8, u32x4>;
  auto piece = [&](const uint8_t* row, int ss, int k) __attribute__((always_inline)) {
    constexpr int PPS = GT == GEMM_FP8 ? 4 : 2;  // pieces per K step
    constexpr int PPL = PPS / 2;                 // pieces per lane half
    return *reinterpret_cast<const u32x4*>(row + (((ss * PPS + lhalf * PPL + k) ^ swl) * 16));
  };
  auto read_frag = [&](const uint8_t* row, int ss) __attribute__((always_inline)) {
    if constexpr (GT == GEMM_FP8) {
      const u32x4 lo = piece(row, ss, 0), hi = piece(row, ss, 1);
      return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return piece(row, ss, 0);
    }
  };
  auto frag_one = [&](const uint8_t* sa, const uint8_t* sb, int ss, int blk, Frag& af, Frag& bf)
                      __attribute__((always_inline)) {
    af = read_frag(sa + ((wf * FB + blk) * 32 + l32) * SB, ss);
    bf = read_frag(sb + ((wt * TB + blk) * 32 + l32) * SB, ss);
  };
  auto frag = [&](const uint8_t* sa, const uint8_t* sb, int ss, Frag* af, Frag* bf)
                  __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < FB; ++a) af[a] = read_frag(sa + ((wf * FB + a) * 32 + l32) * SB, ss);
#pragma unroll
    for (int b = 0; b < TB; ++b) bf[b] = read_frag(sb + ((wt * TB + b) * 32 + l32) * SB, ss);
  };
  // kKSteps 16-element K steps per stage, each FB groups of TB MFMAs (one
  // feature block against the TB token blocks).  The fragments of step s+1
  // are read from LDS during step s, and the 2*NL load instructions of a
  // later stage (nxt >= 0) are spread one per group (or in one burst before
  // the first step): with one wave per SIMD a wave stalled on a full
  // vector-memory queue issues no MFMA, so the loads go out in small pieces
  // between MFMA groups.
  // hfill: this is the last stage of a key tile; its load slots bring in the
  // st0 half of h instead.
  // One K stage from (sa, sb).  kSlots (compile-time, so the unrolled body
  // has no branches) says what its load slots carry: kSlotNext = stage kl into
  // the buffer at nla, kSlotH + X = part X of h, kSlotNone = nothing.
  auto compute = [&](const uint8_t* sa, const uint8_t* sb, int kl, uint32_t nla, auto kSlots)
                     __attribute__((always_inline)) {
    constexpr int SLOTS = decltype(kSlots)::value;
    constexpr int KS = GT == GEMM_FP8 ? SB / 64 : S::kKSteps;
    constexpr int NG = KS * FB;           // MFMA groups per stage
    constexpr int NI = 2 * NL;            // load slots per stage
    constexpr int MPER = GT == GEMM_F32 ? 4 : 1;  // MFMA instructions per fragment pair
    static_assert(FB == TB, "one A and one B fragment of the next step per group");
    static_assert(SLOTS < kSlotH || kHOverlap, "h parts only in the bf16 key/value epilogue");
    Frag af[2][FB], bf[2][TB];
    if constexpr (!kSpreadLoads && SLOTS == kSlotNext) issue(kl, nla);
    if constexpr (!kSpreadLoads && SLOTS >= kSlotH) {
#pragma unroll
      for (int j = 0; j < NI; ++j) issue_h(SLOTS - kSlotH, j);
    }
    const void* bA = SLOTS == kSlotNext ? stage_base(tileA, kl) : nullptr;
    const void* bB = SLOTS == kSlotNext && !GATHER ? stage_base(tileB, kl) : nullptr;
    frag(sa, sb, 0, af[0], bf[0]);
#pragma unroll
    for (int ss = 0; ss < KS; ++ss) {
      const int cur = ss & 1, nx = (ss + 1) & 1;
#pragma unroll
      for (int a = 0; a < FB; ++a) {
#pragma unroll
        for (int b = 0; b < TB; ++b) Mma<GT>::run(af[cur][a], bf[cur][b], acc[a][b]);
        if (ss + 1 < KS) {
          frag_one(sa, sb, ss + 1, a, af[nx][a], bf[nx][a]);
          // the group's LDS reads (2, or 4 for E4M3) between its TB MFMAs
          constexpr int NR = GT == GEMM_FP8 ? 4 : 2;
#pragma unroll
          for (int i = 0; i < NR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, TB * MPER / NR, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, TB * MPER, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kSpreadLoads && SLOTS != kSlotNone) {
          // load j goes out after group (j * LG) / NI
          constexpr int LG = kLoadGroups < NG ? kLoadGroups : NG;
          const int gi = ss * FB + a;
#pragma unroll
          for (int j = (gi * NI + LG - 1) / LG; gi < LG && j < ((gi + 1) * NI + LG - 1) / LG; ++j) {
            if constexpr (SLOTS == kSlotNext)
              issue_one(bA, bB, nla, j);
            else
              issue_h(SLOTS - kSlotH, j);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using SlotNext = std::integral_constant<int, kSlotNext>;
  using SlotNone = std::integral_constant<int, kSlotNone>;

  // ---- early-barrier schedule (two 128-byte stages, bf16 / fp16 operands).
  // Stage k's barrier sits after the first group of its last K step instead
  // of before its first: by then every wave has read all of stage k's
  // fragments (their reads ended with the step before), so stage k's buffer
  // is free, and stage k+1's data has landed.  The rest of stage k then
  // reads stage k+1's step-0 fragments while its last MFMAs run (the MFMAs of
  // a stage start without an LDS wait) and issues the first kLate loads of
  // stage k+2 into the freed buffer; stage k+1 issues the other loads of
  // stage k+2 in its first groups.  Buffer k % 2 holds stage k, and after the
  // last stage the virtual stages nk, nk+1 are the two parts of the h tile
  // (value tiles and the de contraction: placeholders or nothing).
  constexpr bool kEarlyBarrier =
      ENGRAM_GEMM_EARLY_BARRIER && NS == 2 && (GT == GEMM_BF16 || GT == GEMM_F16) && !GATHER;
  constexpr int kLate = ENGRAM_GEMM_LATE;  // slots issued after the barrier two stages ahead
  constexpr int kBarGroup = 12;  // the barrier follows this group (first of step 3)
  Frag af2[2][FB], bf2[2][TB];   // fragments carried across stages
  auto slot_issue = [&](auto kSlots, const void* bA, const void* bB, uint32_t la, int j)
                        __attribute__((always_inline)) {
    constexpr int SL = decltype(kSlots)::value;
    if constexpr (SL == kSlotNext)
      issue_one(bA, bB, la, j);
    else if constexpr (SL == kSlotTail)
      issue_tail(j);
    else if constexpr (SL >= kSlotH)
      issue_h(SL - kSlotH, j);
  };
  // sa, sb: this stage; na, nb: the next one (step-0 fragments, with kNext);
  // kEarlyS: slots kLate.. of the stage after this one (ekl at ela) in
  // groups 0..4; kLateS: slots 0..kLate-1 (all with kLateAll) of the stage
  // two ahead (lkl at lla) after the barrier.
  auto compute2 = [&](const uint8_t* sa, const uint8_t* sb, const uint8_t* na, const uint8_t* nb,
                      auto kEarlyS, int ekl, uint32_t ela, auto kLateS, int lkl, uint32_t lla,
                      auto kNext, auto kLateAll, [[maybe_unused]] int kid, auto kZero, auto kPfES)
                      __attribute__((always_inline)) {
    constexpr bool ZERO = decltype(kZero)::value;  // stage 0: step 0 starts the accumulators
    // kPfEL B fetch-ahead loads from group kPfEGroup on: the stage's own
    // loads have all gone out by then, so its barrier leaves just those in
    // flight
    constexpr bool PFE = decltype(kPfES)::value;
    constexpr int kPfEGroup = 8;  // the kPfEL loads follow groups 8, 9, ...
    constexpr int ESL = decltype(kEarlyS)::value;
    constexpr int LSL = decltype(kLateS)::value;
    constexpr bool NEXT = decltype(kNext)::value;
    constexpr int NI = 2 * NL;
    constexpr int KS = S::kKSteps;
    constexpr int NLATE = decltype(kLateAll)::value ? NI : kLate;
    constexpr int NAFTER = KS * FB - 1 - kBarGroup;  // groups after the barrier
    static_assert(KS == 4 && FB == 4 && NI == 16 && NAFTER == 3, "early-barrier stage shape");
    // every early slot goes out before the barrier that waits for it
    static_assert(kLate + ENGRAM_GEMM_EARLY_PER * (kBarGroup + 1) >= NI, "early loads after the barrier");
    const void* ebA = ESL == kSlotNext ? stage_base(tileA, ekl) : nullptr;
    const void* ebB = ESL == kSlotNext ? stage_base(tileB, ekl) : nullptr;
    const void* lbA = LSL == kSlotNext ? stage_base(tileA, lkl) : nullptr;
    const void* lbB = LSL == kSlotNext ? stage_base(tileB, lkl) : nullptr;
#pragma unroll
    for (int ss = 0; ss < KS; ++ss) {
      const int cur = ss & 1, nx = (ss + 1) & 1;
#pragma unroll
      for (int a = 0; a < FB; ++a) {
        const int gi = ss * FB + a;
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          if constexpr (ZERO) {
            if (ss == 0)
              Mma<GT>::run0(af2[cur][a], bf2[cur][b], acc[a][b]);
            else
              Mma<GT>::run(af2[cur][a], bf2[cur][b], acc[a][b]);
          } else {
            Mma<GT>::run(af2[cur][a], bf2[cur][b], acc[a][b]);
          }
        }
        if (ss + 1 < KS) {
          frag_one(sa, sb, ss + 1, a, af2[nx][a], bf2[nx][a]);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, TB / 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        } else if (NEXT && gi > kBarGroup) {
          // next stage's step 0: pairs 0 and 1 in group 13, 2 and 3 in 14 and 15
          if (gi == kBarGroup + 1) {
            frag_one(na, nb, 0, 0, af2[nx][0], bf2[nx][0]);
            frag_one(na, nb, 0, 1, af2[nx][1], bf2[nx][1]);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, TB - 1, 0);
          } else {
            const int pr = gi - kBarGroup;
            frag_one(na, nb, 0, pr, af2[nx][pr], bf2[nx][pr]);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, TB - 1, 0);
          }
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, TB, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ESL != kSlotNone) {
          constexpr int EP = ENGRAM_GEMM_EARLY_PER;  // early slots per group
#pragma unroll
          for (int j = kLate + EP * gi; j < kLate + EP * (gi + 1) && j < NI; ++j)
            slot_issue(kEarlyS, ebA, ebB, ela, j);
        }
        if constexpr (LSL != kSlotNone) {
          if (gi > kBarGroup) {
            const int g3 = gi - kBarGroup - 1;
#pragma unroll
            for (int j = g3 * NLATE / NAFTER; j < (g3 + 1) * NLATE / NAFTER; ++j)
              slot_issue(kLateS, lbA, lbB, lla, j);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PFE) {
          static_assert(kLate + ENGRAM_GEMM_EARLY_PER * kPfEGroup >= NI &&
                            kPfEGroup + kPfEL <= kBarGroup,
                        "the fetch-ahead loads follow every early slot");
          if (gi >= kPfEGroup && gi < kPfEGroup + kPfEL) {
            const int ks = kid + 3 < nk ? kid + 3 : nk - 1;
            load_lds16_s(pfe_voff[gi - kPfEGroup], stage_base(tileB, ks),
                         lds_addr(sIdx) + (uint32_t)wave * 1024u);
          }
        }
        if (gi == kBarGroup) {
          // this wave's loads of the next stage and its reads of this one are
          // done (a fetch-ahead load of this stage may still be in flight);
          // then every wave's are
          ENGRAM_TRACE_W(kid, 0);
          if constexpr (NEXT && PFE)
            ENGRAM_WAIT_VM_LDS(kPfEL);
          else if constexpr (NEXT)
            ENGRAM_WAIT_VM_LDS(0);
          else
            ENGRAM_WAIT_VM_LDS(63);
          ENGRAM_TRACE_W(kid, 1);
          ENGRAM_BARRIER();
          ENGRAM_TRACE_W(kid, 2);
        }
      }
    }
  };

  // ---- ring: stage k lives in buffer k % NS; loads run NS-1 stages ahead.
  // Each wave issues 2*NL loads per stage, so "stage k landed" is
  // vmcnt <= 2*NL * (stages issued after k).  nk is a multiple of NS
  // (gemm_supported); the final stages are peeled so that the loop body
  // always loads.
  uint8_t* const sA0 = st0;
  uint8_t* const sB0 = st0 + kTS;
  uint8_t* const sA1 = st1;
  uint8_t* const sB1 = st1 + kTS;
  const uint32_t l0 = lds_addr(st0), l1 = lds_addr(st1);
  if constexpr (kEarlyBarrier) {
    using True_ = std::true_type;
    using False_ = std::false_type;
    ENGRAM_TRACE_TILE(6);
    if (pf_kind == 0) issue(0, l0);
    {
      const void* bA = stage_base(tileA, 1);
      const void* bB = stage_base(tileB, 1);
#pragma unroll
      for (int j = 0; j < kLate; ++j) issue_one(bA, bB, l1, j);
    }
    // this wave's stage-0 loads landed (counted from the newest operation:
    // the previous tile's 32 row stores, when known, may still be in flight)
    if (pf_kind == 1)
      ENGRAM_WAIT_VM(kLate + 32);
    else if (pf_kind == 3)
      ENGRAM_WAIT_VM(63);
    else
      ENGRAM_WAIT_VM(kLate);
    ENGRAM_TRACE_TILE(7);
    ENGRAM_BARRIER();
    ENGRAM_TRACE_TILE(3);
    frag(sA0, sB0, 0, af2[0], bf2[0]);
    // stages 0 and 1 peeled (nk >= 4 here): stage 0's first step writes the
    // accumulators instead of adding to zeroed ones
    using PfE = std::integral_constant<bool, kPfE>;
    compute2(sA0, sB0, sA1, sB1, SlotNext{}, 1, l1, SlotNext{}, 2, l0, True_{}, False_{}, 0, True_{}, PfE{});
    compute2(sA1, sB1, sA0, sB0, SlotNext{}, 2, l0, SlotNext{}, 3, l1, True_{}, False_{}, 1, False_{}, PfE{});
    int kt = 2;
    for (; kt + 2 < nk; kt += 2) {
      compute2(sA0, sB0, sA1, sB1, SlotNext{}, kt + 1, l1, SlotNext{}, kt + 2, l0, True_{}, False_{},
               kt, False_{}, PfE{});
      compute2(sA1, sB1, sA0, sB0, SlotNext{}, kt + 2, l0, SlotNext{}, kt + 3, l1, True_{}, False_{},
               kt + 1, False_{}, PfE{});
    }
    // part 0 of the h tile (placeholder reads in value tiles) as stage nk;
    // part 1 goes out after the loop, where a burst of loads holds up no MFMA
    using H0 = std::conditional_t<kHOverlap, SlotHPart<0>, SlotNone>;
#if ENGRAM_GEMM_H1_LATE
    using H1 = std::conditional_t<kHOverlap, SlotHPart<1>, SlotNone>;
#else
    using H1 = SlotNone;
#endif
    if constexpr (kPrefetchTile) {
      // key tiles load part 0 of h into buffer 0, value tiles the next
      // tile's stage 0 (one code path: a branch here made the compiler spill)
      using TL = std::integral_constant<int, kSlotTail>;
      compute2(sA0, sB0, sA1, sB1, SlotNext{}, kt + 1, l1, TL{}, 0, 0u, True_{}, False_{}, kt, False_{},
               False_{});
      compute2(sA1, sB1, sA1, sB1, TL{}, 0, 0u, H1{}, 0, 0u, False_{}, True_{}, kt + 1, False_{},
               False_{});
    } else {
      compute2(sA0, sB0, sA1, sB1, SlotNext{}, kt + 1, l1, H0{}, 0, 0u, True_{}, False_{}, kt, False_{},
               False_{});
      compute2(sA1, sB1, sA1, sB1, H0{}, 0, 0u, H1{}, 0, 0u, False_{}, True_{}, kt + 1, False_{},
               False_{});
    }
  } else if constexpr (NS == 4) {
    uint8_t* const sA2 = st2;
    uint8_t* const sB2 = st2 + kTS;
    uint8_t* const sA3 = st3;
    uint8_t* const sB3 = st3 + kTS;
    const uint32_t l2 = lds_addr(st2), l3 = lds_addr(st3);
    issue(0, l0);
    issue(1, l1);
    issue(2, l2);
#define ENGRAM_STEP(k, SA, SB_, LN, W, SLOT) \
  {                                          \
    ENGRAM_WAIT_VM(W);                       \
    ENGRAM_BARRIER();                        \
    compute(SA, SB_, (k) + 3, LN, SLOT{});   \
  }
    int kt = 0;
    for (; kt + 4 < nk; kt += 4) {
      ENGRAM_STEP(kt, sA0, sB0, l3, 4 * NL, SlotNext);
      ENGRAM_STEP(kt + 1, sA1, sB1, l0, 4 * NL, SlotNext);
      ENGRAM_STEP(kt + 2, sA2, sB2, l1, 4 * NL, SlotNext);
      ENGRAM_STEP(kt + 3, sA3, sB3, l2, 4 * NL, SlotNext);
    }
    ENGRAM_STEP(kt, sA0, sB0, l3, 4 * NL, SlotNext);
    if constexpr (kHOverlap) {
      // h parts 0, 1, 2 into the buffers of stages nk-4, nk-3, nk-2 as they
      // free up; they count like stage loads in the waits
      ENGRAM_STEP(kt + 1, sA1, sB1, l0, 4 * NL, SlotHPart<0>);
      ENGRAM_STEP(kt + 2, sA2, sB2, l1, 4 * NL, SlotHPart<1>);
      ENGRAM_STEP(kt + 3, sA3, sB3, l2, 4 * NL, SlotHPart<2>);
    } else {
      ENGRAM_STEP(kt + 1, sA1, sB1, l0, 4 * NL, SlotNone);
      ENGRAM_STEP(kt + 2, sA2, sB2, l1, 2 * NL, SlotNone);
      ENGRAM_STEP(kt + 3, sA3, sB3, l2, 0, SlotNone);
    }
#undef ENGRAM_STEP
  } else {
    issue(0, l0);
#define ENGRAM_STEP(k, SA, SB_, LN, SLOT) \
  {                                       \
    ENGRAM_TRACE_W(k, 0);                 \
    ENGRAM_WAIT_VM(0);                    \
    ENGRAM_TRACE_W(k, 1);                 \
    ENGRAM_BARRIER();                     \
    ENGRAM_TRACE_W(k, 2);                 \
    ENGRAM_TRACE_STAGE(k);                \
    compute(SA, SB_, (k) + 1, LN, SLOT{}); \
  }
    int kt = 0;
    for (; kt + 2 < nk; kt += 2) {
      ENGRAM_STEP(kt, sA0, sB0, l1, SlotNext);
      ENGRAM_STEP(kt + 1, sA1, sB1, l0, SlotNext);
    }
    ENGRAM_STEP(kt, sA0, sB0, l1, SlotNext);
    // one code path for the last stage: value tiles fill their h slots with a
    // repeated 16-byte read instead of branching around them
    using LastSlots = std::conditional_t<kHOverlap, SlotHPart<0>, SlotNone>;
    ENGRAM_STEP(kt + 1, sA1, sB1, l0, LastSlots);
#undef ENGRAM_STEP
  }
  ENGRAM_TRACE_TILE(1);
  // stage buffers are free from here on (the st0 half of h may be in flight)
  if (kPrefetchTile || hov) {
    // with the next tile's stage 0 (value tiles) or h part 0 (key tiles) in
    // flight into buffer 0: every wave has read the last stage in buffer 1.
    // Value tiles without a next tile to load read h placeholders into
    // buffer 0 instead; those land before the tile ends.
    if (kPrefetchTile && !hov && !pf_next) ENGRAM_WAIT_VM(0);
    ENGRAM_WAIT_VM_LDS(63);
    ENGRAM_BARRIER();
  } else {
    // A value tile's last stages issued placeholder h loads into the rows its
    // epilogue writes next; the compiler cannot see those asm loads, so
    // __syncthreads() alone would not wait for them.
    ENGRAM_WAIT_VM(0);
    __syncthreads();
  }

  // ---- epilogues.  acc[a][b][q*4+r] holds C^T[f][m] with
  //      f = f0 + (wf*FB + a)*32 + q*8 + lhalf*4 + r,  m = m0 + (wt*TB + b)*32 + l32
  if constexpr (kBf16Epi) {
    // bf16: the whole 256-token x 256-feature tile goes through LDS as bf16,
    // token rows of 512 bytes (64 rows per stage buffer), 16-byte pieces
    // XOR-swizzled by (token & 31).  h is brought in and v goes out as whole
    // rows (a wave moves two 512-byte rows per instruction).
    const int d = g.d;
    if (key_tile) {
      if (hov) {
        // the last part of h (the others went out in the last K stages)
        if constexpr (!kEarlyBarrier || !ENGRAM_GEMM_H1_LATE) {
#pragma unroll
          for (int j = 0; j < 2 * NL; ++j) issue_h(NS - 1, j);
        }
      } else {
        // whole h tile: instruction i of wave w fills rows t0, t0+1 (t0 = 2(32w+i))
#pragma unroll 4
        for (int i = 0; i < 32; ++i) {
          const int t0 = (wave * 32 + i) * 2;
          const int t = t0 + (lane >> 5);
          const int c16 = (lane & 31) ^ (t & 31);  // logical piece landing at slot lane&31
          int64_t m = m0 + t;
          m = m < g.M ? m : g.M - 1;
          load_lds16(hB + ((m * d + fk) + c16 * 8) * 2, lds_addr(trow(t0)));
        }
      }
      float* red = reinterpret_cast<float*>(sIdxOrRed);  // [2 wf][2 wt][TB][32][3]
      float* const sg = red + kRedFloats;                 // [256] gamma_q * gamma_k of the tile
      const bool has_gamma = g.gamma_q || g.gamma_k;
      if (has_gamma) {
        const int f = fk + tid;
        sg[tid] = (gqB ? gqB[f] : 1.f) * (gkB ? gkB[f] : 1.f);
      }
      if constexpr (GT == GEMM_FP8) sScaleA[tid] = g.scale_a[f0 + tid];
      if (hov) {
        // parts of the first two token blocks landed (at most the last 16
        // h loads, the parts of blocks 2 and 3, still in flight), gamma written
        static_assert(NS == 2 ? 2 * NL == 16 : 4 * NL == 16, "h part sizes");
        ENGRAM_WAIT_VM_LDS(16);
      } else {
        ENGRAM_WAIT_VM_LDS(0);
      }
      ENGRAM_BARRIER();
      ENGRAM_TRACE_TILE(8);
      // Per token (lane column), over this wave's 128 features: sum k^2,
      // sum g h k (g = gamma_q gamma_k), sum h^2.  Variants without gamma and
      // without the k store keep those branches out of the unrolled body.
      // Token blocks [B0, B1) of this wave.
      auto key_sums = [&](auto kGamma, auto kStoreK, auto kB0, auto kB1) __attribute__((always_inline)) {
        constexpr bool G = decltype(kGamma)::value;
        constexpr bool SK = decltype(kStoreK)::value;
#pragma unroll
        for (int b = decltype(kB0)::value; b < decltype(kB1)::value; ++b) {
          const int t = (wt * TB + b) * 32 + l32;
          const int64_t m = m0 + t;
          const uint8_t* hrow = trow(t);
          // E4M3: k = acc * scale_a[f] * scale_b[m]; the token's scale_b factors
          // out of the sums and is applied once per token
          const float sb = GT == GEMM_FP8 ? g.scale_b[m < g.M ? m : g.M - 1] : 1.f;
          u32x2 hr[FB * 4];
#pragma unroll
          for (int j = 0; j < FB * 4; ++j) {
            const int c16 = wf * FB * 4 + j;
            hr[j] = *reinterpret_cast<const u32x2*>(hrow + ((c16 ^ (t & 31)) << 4) + lhalf * 8);
          }
          float skk = 0.f, shk = 0.f, shh = 0.f;
#pragma unroll
          for (int a = 0; a < FB; ++a) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x2 h2 = hr[a * 4 + q];
              floatx4 hx = floatx4{__uint_as_float(h2[0] << 16), __uint_as_float(h2[0] & 0xFFFF0000u),
                                   __uint_as_float(h2[1] << 16), __uint_as_float(h2[1] & 0xFFFF0000u)};
              shh += hx[0] * hx[0];
              shh += hx[1] * hx[1];
              shh += hx[2] * hx[2];
              shh += hx[3] * hx[3];
              if constexpr (G) {
                const int fl = (wf * FB + a) * 32 + q * 8 + lhalf * 4;
                hx *= *reinterpret_cast<const floatx4*>(sg + fl);
              }
              float kv[4];
              floatx4 sa4 = floatx4{1.f, 1.f, 1.f, 1.f};
              if constexpr (GT == GEMM_FP8)
                sa4 = *reinterpret_cast<const floatx4*>(sScaleA + (wf * FB + a) * 32 + q * 8 + lhalf * 4);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                kv[r] = acc_read(acc[a][b][q * 4 + r]);
                if constexpr (GT == GEMM_FP8) kv[r] *= sa4[r];
                skk += kv[r] * kv[r];
                shk += hx[r] * kv[r];
              }
              if constexpr (SK) {
                if (m < g.M) {
                  const int f = fk + (wf * FB + a) * 32 + q * 8 + lhalf * 4;
                  *reinterpret_cast<u32x2*>(koutB + (m * d + f) * 2) =
                      u32x2{pack_bf16x2(kv[0] * sb, kv[1] * sb), pack_bf16x2(kv[2] * sb, kv[3] * sb)};
                }
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (GT == GEMM_FP8) {
            skk *= sb * sb;
            shk *= sb;
          }
          skk += __shfl_xor(skk, 32);
          shk += __shfl_xor(shk, 32);
          shh += __shfl_xor(shh, 32);
          if (lhalf == 0) {
            float* p = red + ((((wf * 2) + wt) * TB + b) * 32 + l32) * 3;
            p[0] = skk;
            p[1] = shk;
            p[2] = shh;
          }
        }
      };
      using T_ = std::true_type;
      using F_ = std::false_type;
      auto sums = [&](auto kB0, auto kB1) __attribute__((always_inline)) {
        if (has_gamma) {
          if (g.k_out) key_sums(T_{}, T_{}, kB0, kB1); else key_sums(T_{}, F_{}, kB0, kB1);
        } else {
          if (g.k_out) key_sums(F_{}, T_{}, kB0, kB1); else key_sums(F_{}, F_{}, kB0, kB1);
        }
      };
      using I0 = std::integral_constant<int, 0>;
      using I2 = std::integral_constant<int, 2>;
      using I4 = std::integral_constant<int, TB>;
      static_assert(TB == 4, "two token blocks per h half");
      if (hov) {
        sums(I0{}, I2{});       // blocks 0, 1: h rows in st0
        ENGRAM_TRACE_TILE(4);
        ENGRAM_WAIT_VM_LDS(0);  // own st1-half loads landed, own reads of st0 done
        ENGRAM_BARRIER();
        auto key_prefetch = [&]() __attribute__((always_inline)) {
          if (pf_next) {
            const void* bA = uniform_ptr(nextA);
            const void* bB = uniform_ptr(nextB);
#pragma unroll
            for (int j = 0; j < 2 * NL; ++j) issue_tile0(bA, bB, j);
          }
        };
        // buffer 0 is free: the next tile's stage 0 lands while blocks 2, 3
        // are summed
        if constexpr (kPrefetchTile && ENGRAM_GEMM_PREFETCH_KEY == 1) key_prefetch();
        if constexpr (kPrefetchTile && ENGRAM_GEMM_PREFETCH_KEY == 2) {
          using I3 = std::integral_constant<int, 3>;
          sums(I2{}, I3{});
          key_prefetch();
          sums(I3{}, I4{});
        } else {
          sums(I2{}, I4{});     // blocks 2, 3: h rows in st1
        }
        ENGRAM_TRACE_TILE(5);
      } else {
        sums(I0{}, I4{});
      }
      if constexpr (kPrefetchTile) {
        // a fence-free barrier: __syncthreads() would wait for those loads
        ENGRAM_WAIT_VM_LDS(63);
        ENGRAM_BARRIER();
      } else {
        __syncthreads();
      }
      {  // 2 wt x TB x 32 = 256 tokens, one per thread; add the two feature halves
        const int wt2 = tid >> 7, b = (tid >> 5) & 3, l = tid & 31;
        const int64_t m = m0 + (wt2 * TB + b) * 32 + l;
        if (m < g.M) {
          const float* p0 = red + (((0 + wt2) * TB + b) * 32 + l) * 3;
          const float* p1 = red + (((2 + wt2) * TB + b) * 32 + l) * 3;
          float* out = partB + (m * (d / kBF) + fk / kBF) * 3;
          out[0] = p0[0] + p1[0];
          out[1] = p0[1] + p1[1];
          out[2] = p0[2] + p1[2];
        }
      }
    } else if constexpr (kPrefetchTile) {
      // value tile, with buffer 0 taken by the next tile's stage 0: the
      // accumulators go to bf16 rows in buffer 1 in two passes of 128 tokens
      // (token blocks 2R, 2R+1 of every wave), each stored as whole rows.
      // Token t = 128w + 64R + r sits at row 64w + r.
      auto value_round = [&](auto kR) __attribute__((always_inline)) {
        constexpr int R = decltype(kR)::value;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const int b = 2 * R + bb;
          const int t = (wt * TB + b) * 32 + l32;
          uint8_t* row = st1 + ((t >> 7) * 64 + (t & 63)) * 512;
#pragma unroll
          for (int a = 0; a < FB; ++a) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c16 = (wf * FB + a) * 4 + q;
              float x[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) x[r] = acc_read(acc[a][b][q * 4 + r]);
              u32x2 u;
              u[0] = pack_bf16x2(x[0], x[1]);
              u[1] = pack_bf16x2(x[2], x[3]);
              *reinterpret_cast<u32x2*>(row + ((c16 ^ (t & 31)) << 4) + lhalf * 8) = u;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        ENGRAM_WAIT_VM_LDS(63);
        ENGRAM_BARRIER();
        if constexpr (R == 0) ENGRAM_TRACE_TILE(4);
        // 128 rows x 32 pieces of 16 bytes; a wave writes two rows per instruction
#pragma unroll kVStoreUnroll
        for (int i = 0; i < 16; ++i) {
          const int lr = (wave * 16 + i) * 2 + (lane >> 5);
          const int t = (lr >> 6) * 128 + 64 * R + (lr & 63);
          const int c16 = lane & 31;
          const int64_t m = m0 + t;
          if (m < g.M) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(st1 + lr * 512 + ((c16 ^ (t & 31)) << 4));
            u32x4* vp = reinterpret_cast<u32x4*>(g.v_out + (m * d + fk + c16 * 8) * 2);
            if constexpr (ENGRAM_GEMM_V_NT != 0)
              __builtin_nontemporal_store(x, vp);
            else
              *vp = x;
          }
        }
      };
      value_round(std::integral_constant<int, 0>{});
      // the second pass rewrites the rows every wave has just read
      ENGRAM_WAIT_VM_LDS(63);
      ENGRAM_BARRIER();
      value_round(std::integral_constant<int, 1>{});
      ENGRAM_TRACE_TILE(5);
    } else {
      // value tile: accumulators -> bf16 rows in LDS -> whole rows to v
      // (8-byte stores straight from the accumulators measured 3 % slower)
      if constexpr (GT == GEMM_FP8) {
        sScaleA[tid] = g.scale_a[f0 + tid];
        __syncthreads();
      }
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        const int t = (wt * TB + b) * 32 + l32;
        uint8_t* row = trow(t);
        float sb = 1.f;
        if constexpr (GT == GEMM_FP8) {
          const int64_t m = m0 + t;
          sb = g.scale_b[m < g.M ? m : g.M - 1];
        }
#pragma unroll
        for (int a = 0; a < FB; ++a) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c16 = (wf * FB + a) * 4 + q;
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = acc_read(acc[a][b][q * 4 + r]);
            if constexpr (GT == GEMM_FP8) {
              const floatx4 sa4 = *reinterpret_cast<const floatx4*>(sScaleA + (wf * FB + a) * 32 + q * 8 + lhalf * 4);
#pragma unroll
              for (int r = 0; r < 4; ++r) x[r] *= sa4[r] * sb;
            }
            u32x2 u;
            u[0] = pack_bf16x2(x[0], x[1]);
            u[1] = pack_bf16x2(x[2], x[3]);
            *reinterpret_cast<u32x2*>(row + ((c16 ^ (t & 31)) << 4) + lhalf * 8) = u;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();
      ENGRAM_TRACE_TILE(4);
      // 256 rows x 32 pieces of 16 bytes; a wave writes two rows per instruction
#pragma unroll 4
      for (int i = 0; i < 32; ++i) {
        const int t = (wave * 32 + i) * 2 + (lane >> 5);
        const int c16 = lane & 31;
        const int64_t m = m0 + t;
        if (m < g.M) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(trow(t) + ((c16 ^ (t & 31)) << 4));
          u32x4* vp = reinterpret_cast<u32x4*>(g.v_out + (m * d + fk + c16 * 8) * 2);
          if constexpr (ENGRAM_GEMM_V_NT != 0)
            __builtin_nontemporal_store(x, vp);
          else
            *vp = x;
        }
      }
      ENGRAM_TRACE_TILE(5);
    }
  } else if constexpr (EPI == EPI_KV) {
    // fp32 (small shapes): straight from the accumulators
    const int io = g.io_dtype;
    const int d = g.d;
    if (key_tile) {
      // Key tile: per-token partial sums of the gate straight from the
      // accumulators (each lane owns one token and 64 of this wave's 128
      // features), h of the next token block loaded while this one is summed.
      float* red = reinterpret_cast<float*>(st0);  // [2 wf][2 wt][TB][32][3]
      // raw h bits (2 words per 4 bf16, 4 per 4 fp32), widened at use
      constexpr int HW = (GT == GEMM_BF16) ? 2 : 4;
      typedef uint32_t hraw_t __attribute__((ext_vector_type(HW)));
      hraw_t hb[2][FB * 4];
      auto load_hb = [&](int b, hraw_t* dst) __attribute__((always_inline)) {
        int64_t m = m0 + (wt * TB + b) * 32 + l32;
        m = m < g.M ? m : g.M - 1;
#pragma unroll
        for (int a = 0; a < FB; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            // element (m, f) of h sits at byte (m*d + f) * element size, and the
            // element size is HW bytes (4 elements = HW words)
            dst[a * 4 + q] = *reinterpret_cast<const hraw_t*>(
                hB + (m * d + fk + (wf * FB + a) * 32 + q * 8 + lhalf * 4) * (int64_t)HW);
      };
      // bf16 h is prefetched one token block ahead; fp32 h (twice the
      // registers) is loaded per block
      constexpr bool kPrefetchH = GT == GEMM_BF16;
      if (kPrefetchH) load_hb(0, hb[0]);
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        if (kPrefetchH) {
          if (b + 1 < TB) load_hb(b + 1, hb[(b + 1) & 1]);
        } else {
          load_hb(b, hb[b & 1]);
        }
        const int64_t m = m0 + (wt * TB + b) * 32 + l32;
        const bool valid = m < g.M;
        float skk = 0.f, shk = 0.f, shh = 0.f;
#pragma unroll
        for (int a = 0; a < FB; ++a) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = fk + (wf * FB + a) * 32 + q * 8 + lhalf * 4;
            floatx4 gg = floatx4{1.f, 1.f, 1.f, 1.f};
            if (gqB) gg *= *reinterpret_cast<const floatx4*>(gqB + f);
            if (gkB) gg *= *reinterpret_cast<const floatx4*>(gkB + f);
            const hraw_t hr = hb[b & 1][a * 4 + q];
            floatx4 hx;
            if constexpr (GT == GEMM_BF16) {
              hx = floatx4{__uint_as_float(hr[0] << 16), __uint_as_float(hr[0] & 0xFFFF0000u),
                           __uint_as_float(hr[1] << 16), __uint_as_float(hr[1] & 0xFFFF0000u)};
            } else {
              hx = floatx4{__uint_as_float(hr[0]), __uint_as_float(hr[1]), __uint_as_float(hr[2]),
                           __uint_as_float(hr[3])};
            }
            float kv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              kv[r] = acc_read(acc[a][b][q * 4 + r]);
              skk += kv[r] * kv[r];
              shk += gg[r] * hx[r] * kv[r];
              shh += hx[r] * hx[r];
            }
            if (koutB && valid) store4(koutB, m * d + f, io, kv[0], kv[1], kv[2], kv[3]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        skk += __shfl_xor(skk, 32);
        shk += __shfl_xor(shk, 32);
        shh += __shfl_xor(shh, 32);
        if (lhalf == 0) {
          float* p = red + ((((wf * 2) + wt) * TB + b) * 32 + l32) * 3;
          p[0] = skk;
          p[1] = shk;
          p[2] = shh;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
      {  // 2 wt x TB x 32 = 256 tokens, one per thread; add the two feature halves
        const int wt2 = tid >> 7, b = (tid >> 5) & 3, l = tid & 31;
        const int64_t m = m0 + (wt2 * TB + b) * 32 + l;
        if (m < g.M) {
          const float* p0 = red + (((0 + wt2) * TB + b) * 32 + l) * 3;
          const float* p1 = red + (((2 + wt2) * TB + b) * 32 + l) * 3;
          float* out = partB + (m * (d / kBF) + fk / kBF) * 3;
          out[0] = p0[0] + p1[0];
          out[1] = p0[1] + p1[1];
          out[2] = p0[2] + p1[2];
        }
      }
    } else {
      // Value tile: stored straight from the accumulators (4 features per
      // lane per store; the pieces of a token row meet in L2)
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        const int64_t m = m0 + (wt * TB + b) * 32 + l32;
        if (m < g.M) {
#pragma unroll
          for (int a = 0; a < FB; ++a) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int f = fk + (wf * FB + a) * 32 + q * 8 + lhalf * 4;
              store4(g.v_out, m * d + f, io, acc_read(acc[a][b][q * 4]),
                     acc_read(acc[a][b][q * 4 + 1]), acc_read(acc[a][b][q * 4 + 2]),
                     acc_read(acc[a][b][q * 4 + 3]));
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  } else {
    // a column (token) scaled by a power of two in its operand row comes back
    // to scale here, exactly
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const int64_t m = m0 + (wt * TB + b) * 32 + l32;
      if (m < g.M) {
        const float inv = g.col_scale ? pow2_inverse(g.col_scale[m]) : 1.f;
#pragma unroll
        for (int a = 0; a < FB; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = f0 + (wf * FB + a) * 32 + q * 8 + lhalf * 4;
            *reinterpret_cast<floatx4*>(g.c_out + m * g.F + f) =
                floatx4{acc_read(acc[a][b][q * 4]) * inv, acc_read(acc[a][b][q * 4 + 1]) * inv,
                        acc_read(acc[a][b][q * 4 + 2]) * inv, acc_read(acc[a][b][q * 4 + 3]) * inv};
          }
      }
    }
  }
  // the next tile reuses LDS: every wave's LDS reads of this one are done
  // (its global stores may still be in flight)
  ENGRAM_WAIT_VM_LDS(63);
  ENGRAM_BARRIER();
  ENGRAM_TRACE_TILE(2);
  if constexpr (kPrefetchTile) {
    // a whole value tile issued exactly 32 row stores per wave after the
    // next tile's stage 0; a key or ragged tile an unknown number
    const bool whole = (tm + 1) * kBT <= g.M;
    pf_kind = !pf_next || (key_tile && ENGRAM_GEMM_PREFETCH_KEY == 0)
                  ? 0
                  : (!whole || key_tile ? 2 : (EPI == EPI_KV ? 1 : 3));
  }
  tm_c = tmn;
  f0_c = f0n;
  }  // slot loop
}

template <int GT, int EPI, bool GATHER>
static hipError_t launch_one(const GemmArgs& g0, hipStream_t s) {
  GemmArgs g = g0;
  const int64_t tiles_m = (g.M + kBT - 1) / kBT;
  const int tiles_f = g.F / kBF;
  const int64_t slots = (tiles_m + 7) / 8 * tiles_f;  // of the longest XCD list
  if (slots >= (int64_t(1) << 30)) return hipErrorInvalidValue;  // slot + step stays in int
  // persistent: one workgroup per CU (the LDS use allows no second one), 8 XCDs
  int64_t per_xcd = slots;
  if (g.persistent) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidValue;
    per_xcd = std::min<int64_t>(slots, std::max(1, cus / 8));
  }
  const int64_t blocks = 8 * per_xcd;
  // the two-buffer schedule of bf16/fp16 operands peels its first two
  // stages before its last two: a K of two stages takes the 64-byte ring
  if (g.stage_bytes == 128 && (GT == GEMM_BF16 || GT == GEMM_F16) && !GATHER &&
      (int64_t)g.K * 2 <= 2 * 128)
    g.stage_bytes = 64;
  if (g.stage_bytes == 128)
    hipLaunchKernelGGL((gemm_kernel<GT, EPI, GATHER, 128>), dim3((unsigned)blocks), dim3(kNT), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_kernel<GT, EPI, GATHER, 64>), dim3((unsigned)blocks), dim3(kNT), 0, s, g);
  return hipGetLastError();
}

#ifdef ENGRAM_GEMM_TRACE
extern "C" int engram_debug_gemm_trace(uint64_t* out, int n) {
  const int total = (int)(sizeof(g_gemm_trace) / sizeof(uint64_t));
  if (n > total) n = total;
  if (hipMemcpyFromSymbol(out, HIP_SYMBOL(g_gemm_trace), n * sizeof(uint64_t)) != hipSuccess) return -1;
  return n;
}
extern "C" int engram_debug_gemm_trace2(uint64_t* out, int n) {
  const int total = (int)(sizeof(g_gemm_trace2) / sizeof(uint64_t));
  if (n > total) n = total;
  if (hipMemcpyFromSymbol(out, HIP_SYMBOL(g_gemm_trace2), n * sizeof(uint64_t)) != hipSuccess) return -1;
  return n;
}
#endif

bool gemm_supported(GemmType type, const GemmArgs& g, bool gather) {
  const int es = type == GEMM_F32 ? 4 : (type == GEMM_FP8 ? 1 : 2);
  if (type == GEMM_FP8 && (gather || !g.scale_a || !g.scale_b)) return false;
  if (g.F % kBF != 0 || g.group_m < 1) return false;
  if (g.stage_bytes != 64 && g.stage_bytes != 128) return false;
  if (((int64_t)g.K * es) % 256 != 0) return false;  // whole ring turns for either stage shape
  // per-lane 32-bit byte offsets inside a 256-row tile
  if ((int64_t)g.K * es * kBT >= (int64_t(1) << 31)) return false;
  if (gather) {
    if (g.J < 1 || g.J > kGatherMaxJ || g.D * es < g.stage_bytes) return false;
    if (((int64_t)g.D * es) % 16 != 0) return false;
    if ((int64_t)g.J * g.D != g.K) return false;
  }
  return true;
}

hipError_t launch_gemm(GemmType type, GemmEpilogue epi, const GemmArgs& g, hipStream_t s) {
  if (g.M == 0) return hipSuccess;
  const bool gather = g.idx != nullptr;
  if (!gemm_supported(type, g, gather)) return hipErrorInvalidValue;
  if (epi == EPI_KV) {
    if (type == GEMM_BF16)
      return gather ? launch_one<GEMM_BF16, EPI_KV, true>(g, s)
                    : launch_one<GEMM_BF16, EPI_KV, false>(g, s);
    if (type == GEMM_F32)
      return gather ? launch_one<GEMM_F32, EPI_KV, true>(g, s)
                    : launch_one<GEMM_F32, EPI_KV, false>(g, s);
    if (type == GEMM_FP8 && !gather) return launch_one<GEMM_FP8, EPI_KV, false>(g, s);
  } else if (!gather) {
    if (type == GEMM_F16) return launch_one<GEMM_F16, EPI_STORE_F32, false>(g, s);
    if (type == GEMM_F32) return launch_one<GEMM_F32, EPI_STORE_F32, false>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace engram
