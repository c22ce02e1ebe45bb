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
// never goes to HBM, and h is read exactly once, here.
//
// Row gather fused into the B operand: with GATHER, the 16-byte pieces of a
// token row of B are read straight from the embedding tables through the
// tile's row indices (kept in LDS), so the concatenated memory vector e_t is
// never written to or read back from HBM.
//
// Tiling: 256 features x 256 tokens per workgroup of 4 wavefronts, each
// owning a 128 x 128 block (16 accumulators of 32x32).  K advances 64 bytes
// per stage through a 4-stage LDS ring filled by direct-to-LDS 16-byte global
// loads (no staging registers); rows are 64 bytes in LDS with the 16-byte
// pieces XOR-swizzled by sw(r) = ((r >> 1) ^ (r >> 3)) & 3 so that the
// ds_read_b128 of 32-row fragments hit distinct banks.  Matrix cores:
// v_mfma_f32_32x32x16_bf16 / _f16; fp32 inputs use four
// v_mfma_f32_32x32x2f32 per 16-byte fragment.  Workgroup ids reach the 8
// XCDs round-robin; the id -> tile map keeps the f-tiles of a small group of
// token tiles on one XCD so they share rows and weight slabs in its L2.
#include "kernels.h"

namespace engram {

template <int GT>
struct Mma;

template <>
struct Mma<GEMM_BF16> {
  __device__ static inline void run(const u32x4& a, const u32x4& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mma<GEMM_F16> {
  __device__ static inline void run(const u32x4& a, const u32x4& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                               __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
  }
};

// fp32: lanes 0-31 hold k = 0..3 of the 32-byte K slice, lanes 32-63 hold
// k = 4..7; step i multiplies the pair (i, 4+i), so four steps cover all 8.
template <>
struct Mma<GEMM_F32> {
  __device__ static inline void run(const u32x4& a, const u32x4& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

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
    u.x = (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
    u.y = (uint32_t)f32_to_bf16_bits(c) | ((uint32_t)f32_to_bf16_bits(d) << 16);
    *reinterpret_cast<u32x2*>(base + i * 2) = u;
  } else {
    *reinterpret_cast<floatx4*>(base + i * 4) = floatx4{a, b, c, d};
  }
}

// 16-byte direct-to-LDS global load: lane l's 16 bytes land at lds_dst + 16*l
// (lds_dst is wave-uniform and goes through M0).  Written as asm so that the
// compiler does not treat every later LDS read as aliasing the write and wait
// for all loads in flight; the ring below waits with explicit vmcnt counts.
// The instruction has no destination register, so nothing the compiler
// allocates can be overwritten while it is in flight.
__device__ inline void load_lds16(const void* src, void* lds_dst) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(m0v)
               : "memory");
}

// Workgroup barrier without a memory fence: LDS written by this wave's
// direct-to-LDS loads is complete once vmcnt says so (waited for explicitly
// before the barrier), and LDS reads of the previous stage were consumed by
// MFMAs before it.  __syncthreads() would also wait for every load in flight.
#define ENGRAM_BARRIER()                 \
  do {                                   \
    __builtin_amdgcn_sched_barrier(0);   \
    __builtin_amdgcn_s_barrier();        \
    __builtin_amdgcn_sched_barrier(0);   \
  } while (0)

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding)
#define ENGRAM_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(((n)&0xF) | ((((n) >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8))

constexpr int kBF = kGemmBF;  // features per tile
constexpr int kBT = 256;      // tokens per tile
constexpr int kNT = 256;      // threads (4 waves)
constexpr int kStageBytes = 64;
constexpr int kStages = 4;
constexpr int kTileStage = 256 * kStageBytes;  // one operand, one stage
constexpr int kGatherMaxJ = 16;

__device__ inline int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

template <int GT, int EPI, bool GATHER>
__global__ __launch_bounds__(kNT) void gemm_kernel(GemmArgs g) {
  constexpr int ES = (GT == GEMM_F32) ? 4 : 2;
  constexpr int FB = 4, TB = 4;  // 32-blocks per wave along f and tokens
  // One LDS object per stage (A then B): the compiler tracks the direct-to-LDS
  // writes of each object separately, so reading stage k does not make it
  // wait for the loads still in flight into the other stages.  The epilogue
  // reuses st0.
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * kTileStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[2 * kTileStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[2 * kTileStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[2 * kTileStage];
  uint8_t* const sA0 = st0;
  uint8_t* const sA1 = st1;
  uint8_t* const sA2 = st2;
  uint8_t* const sA3 = st3;
  uint8_t* const sB0 = st0 + kTileStage;
  uint8_t* const sB1 = st1 + kTileStage;
  uint8_t* const sB2 = st2 + kTileStage;
  uint8_t* const sB3 = st3 + kTileStage;
  __shared__ int32_t sIdx[GATHER ? kBT * kGatherMaxJ : 1];
  __shared__ const uint8_t* sTab[GATHER ? kGatherMaxJ : 1];

  // ---- workgroup id -> (token tile, feature tile), XCD-grouped
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int tiles_f = g.F / kBF;
  const int gm = g.group_m;
  const int per_group = gm * tiles_f;
  const int grp = slot / per_group;
  const int in_g = slot - grp * per_group;
  const int tf = in_g / gm;
  const int tm_local = in_g - tf * gm;
  const int64_t tm = (int64_t)(grp * gm + tm_local) * 8 + xcd;
  const int64_t tiles_m = (g.M + kBT - 1) / kBT;
  if (tm >= tiles_m) return;
  const int f0 = tf * kBF;
  const int64_t m0 = tm * kBT;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wf = wave & 1;
  const int wt = wave >> 1;
  const int64_t row_bytes = (int64_t)g.K * ES;
  const int nk = (int)(row_bytes / kStageBytes);

  if constexpr (GATHER) {
    const int J = g.J;
    for (int i = tid; i < kBT * J; i += kNT) {
      const int r = i / J, j = i - r * J;
      int64_t m = m0 + r;
      m = m < g.M ? m : g.M - 1;
      sIdx[r * kGatherMaxJ + j] = g.idx[m * J + j];
    }
    if (tid < J) sTab[tid] = g.tables[tid];
    __syncthreads();
  }

  // ---- per-lane load descriptors: piece i of this wave covers rows
  //      ch*16 + lane/4 (ch = wave + 4i), physical 16-byte slot lane&3
  const uint8_t* srcA[4];
  const uint8_t* srcB[4];
  int gj[4], gw[4], grow[4];  // GATHER: table, element offset and local row of the piece at stage 0
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = wave + 4 * i;
    const int row = ch * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    srcA[i] = g.A + (int64_t)(f0 + row) * row_bytes + c * 16;
    int64_t m = m0 + row;
    m = m < g.M ? m : g.M - 1;
    if constexpr (GATHER) {
      const int e0 = c * 16 / ES;
      gj[i] = e0 / g.D;
      gw[i] = e0 - gj[i] * g.D;
      grow[i] = row;
      srcB[i] = nullptr;
    } else {
      srcB[i] = g.B + m * row_bytes + c * 16;
      gj[i] = gw[i] = grow[i] = 0;
    }
  }
  constexpr int kStageElems = kStageBytes / ES;
  const int64_t dbytes = (int64_t)g.D * ES;

  // GATHER: (gj, gw) = table and element of piece i at the next stage to
  // issue, (nrow, nbase) = its row index and table base, read from LDS one
  // stage ahead so the loads never wait on those LDS reads.  issue() must be
  // called for kt = 0, 1, 2, ... in order.
  int32_t nrow[4];
  const uint8_t* nbase[4];
  if constexpr (GATHER) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nrow[i] = sIdx[grow[i] * kGatherMaxJ + gj[i]];
      nbase[i] = sTab[gj[i]];
    }
  }
  auto issue = [&](int kt, uint8_t* sa, uint8_t* sb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = wave + 4 * i;
      load_lds16(srcA[i] + (int64_t)kt * kStageBytes, sa + ch * 1024);
      if constexpr (GATHER) {
        load_lds16(nbase[i] + (int64_t)nrow[i] * dbytes + (int64_t)gw[i] * ES, sb + ch * 1024);
        // advance to the next stage: D >= kStageElems, so at most one table boundary
        gw[i] += kStageElems;
        const bool wrap = gw[i] >= g.D;
        gw[i] = wrap ? gw[i] - g.D : gw[i];
        gj[i] = wrap ? gj[i] + 1 : gj[i];
        const int jn = gj[i] < g.J ? gj[i] : g.J - 1;  // past the last stage: any valid entry
        nrow[i] = sIdx[grow[i] * kGatherMaxJ + jn];
        nbase[i] = sTab[jn];
      } else {
        load_lds16(srcB[i] + (int64_t)kt * kStageBytes, sb + ch * 1024);
      }
    }
  };

  floatx16 acc[FB][TB];
#pragma unroll
  for (int a = 0; a < FB; ++a)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[a][b] = floatx16{};

  const int l32 = lane & 31;
  const int lhalf = lane >> 5;
  const int swl = swz(l32);  // fragment rows are blk*32 + l32: one swizzle for every blk

  auto frag = [&](const uint8_t* sa, const uint8_t* sb, int ss, u32x4* af, u32x4* bf)
                  __attribute__((always_inline)) {
    const int phys = ((ss * 2 + lhalf) ^ swl) * 16;
#pragma unroll
    for (int a = 0; a < FB; ++a)
      af[a] = *reinterpret_cast<const u32x4*>(sa + ((wf * FB + a) * 32 + l32) * kStageBytes + phys);
#pragma unroll
    for (int b = 0; b < TB; ++b)
      bf[b] = *reinterpret_cast<const u32x4*>(sb + ((wt * TB + b) * 32 + l32) * kStageBytes + phys);
  };
  // two 16-element K steps per stage; the fragments of the second are read
  // from LDS while the 16 MFMAs of the first run
  auto compute = [&](const uint8_t* sa, const uint8_t* sb) __attribute__((always_inline)) {
    u32x4 af0[FB], bf0[TB], af1[FB], bf1[TB];
    frag(sa, sb, 0, af0, bf0);
    frag(sa, sb, 1, af1, bf1);
#pragma unroll
    for (int a = 0; a < FB; ++a)
#pragma unroll
      for (int b = 0; b < TB; ++b) Mma<GT>::run(af0[a], bf0[b], acc[a][b]);
#pragma unroll
    for (int a = 0; a < FB; ++a)
#pragma unroll
      for (int b = 0; b < TB; ++b) Mma<GT>::run(af1[a], bf1[b], acc[a][b]);
    // schedule: the 8 reads of the first K step, then its 16 MFMAs with the 8
    // reads of the second step slotted in between, then the second 16 MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16 * (GT == GEMM_F32 ? 4 : 1), 0);
  };

  // ---- 4-stage ring: stage k lives in buffer k % 4; loads run 3 stages ahead.
  // Each wave issues 8 loads per stage, so "stage k landed" is vmcnt <= 8 * (stages after k).
  if (0 < nk) issue(0, sA0, sB0);
  if (1 < nk) issue(1, sA1, sB1);
  if (2 < nk) issue(2, sA2, sB2);
#define ENGRAM_STEP(k, SA, SB, SAN, SBN)        \
  {                                             \
    const int left_ = nk - 1 - (k);             \
    if (left_ >= 2)                             \
      ENGRAM_WAIT_VM(16);                       \
    else if (left_ == 1)                        \
      ENGRAM_WAIT_VM(8);                        \
    else                                        \
      ENGRAM_WAIT_VM(0);                        \
    ENGRAM_BARRIER();                           \
    if ((k) + 3 < nk) issue((k) + 3, SAN, SBN); \
    compute(SA, SB);                            \
  }
  for (int kt = 0; kt < nk; kt += 4) {
    ENGRAM_STEP(kt, sA0, sB0, sA3, sB3);
    ENGRAM_STEP(kt + 1, sA1, sB1, sA0, sB0);
    ENGRAM_STEP(kt + 2, sA2, sB2, sA1, sB1);
    ENGRAM_STEP(kt + 3, sA3, sB3, sA2, sB2);
  }
#undef ENGRAM_STEP
  __syncthreads();  // stage buffers are free from here on

  // ---- epilogues.  acc[a][b][q*4+r] holds C^T[f][m] with
  //      f = f0 + (wf*FB + a)*32 + q*8 + lhalf*4 + r,  m = m0 + (wt*TB + b)*32 + l32
  if constexpr (EPI == EPI_KV) {
    // Through LDS, 32 tokens x 256 features (fp32, 1 KB per token row, the
    // 16-byte pieces XOR-swizzled by the row) at a time: the two waves owning
    // those tokens write their accumulators, then 32 lanes per token read 8
    // features each, so h is read and k / v are written as whole rows.
    const int io = g.io_dtype;
    const int d = g.d;
    const bool key_tile = f0 < d;
    const int tg = tid >> 5;         // token of this thread within a round of 8
    const int c0 = (tid & 31) * 2;   // its two 16-byte pieces (8 features)
    uint8_t* const stage = st0;
    floatx4 g4[2] = {floatx4{1.f, 1.f, 1.f, 1.f}, floatx4{1.f, 1.f, 1.f, 1.f}};
    if (key_tile) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        if (g.gamma_q) g4[h2] *= *reinterpret_cast<const floatx4*>(g.gamma_q + f0 + c0 * 4 + 4 * h2);
        if (g.gamma_k) g4[h2] *= *reinterpret_cast<const floatx4*>(g.gamma_k + f0 + c0 * 4 + 4 * h2);
      }
    }
    // h of this thread's 4 tokens in pass p (8 features each), loaded one pass ahead
    auto load_h = [&](int p, floatx4* hb) __attribute__((always_inline)) {
#pragma unroll
      for (int round = 0; round < 4; ++round) {
        int64_t m = m0 + p * 32 + round * 8 + tg;
        m = m < g.M ? m : g.M - 1;
        hb[2 * round] = load4(g.h, m * d + f0 + c0 * 4, io);
        hb[2 * round + 1] = load4(g.h, m * d + f0 + c0 * 4 + 4, io);
      }
    };
    floatx4 hcur[8], hnext[8];
    if (key_tile) load_h(0, hnext);
#pragma unroll
    for (int p = 0; p < 8; ++p) {  // tokens p*32 .. p*32+31 of the tile
      if (key_tile) {
#pragma unroll
        for (int i = 0; i < 8; ++i) hcur[i] = hnext[i];
        if (p + 1 < 8) load_h(p + 1, hnext);
      }
      if (wt == (p >> 2)) {
        const int b = p & 3;
#pragma unroll
        for (int a = 0; a < FB; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int piece = ((wf * FB + a) * 32 + q * 8 + lhalf * 4) >> 2;
            *reinterpret_cast<floatx4*>(stage + l32 * 1024 + ((piece ^ (l32 & 15)) << 4)) =
                floatx4{acc[a][b][q * 4], acc[a][b][q * 4 + 1], acc[a][b][q * 4 + 2],
                        acc[a][b][q * 4 + 3]};
          }
      }
      __syncthreads();
#pragma unroll
      for (int round = 0; round < 4; ++round) {
        const int tl = round * 8 + tg;
        const int64_t m = m0 + p * 32 + tl;
        const uint8_t* row = stage + tl * 1024;
        const floatx4 x0 = *reinterpret_cast<const floatx4*>(row + ((c0 ^ (tl & 15)) << 4));
        const floatx4 x1 = *reinterpret_cast<const floatx4*>(row + (((c0 + 1) ^ (tl & 15)) << 4));
        const bool valid = m < g.M;
        const int f = c0 * 4;  // feature offset inside the tile
        if (key_tile) {
          const floatx4 h0 = hcur[2 * round];
          const floatx4 h1 = hcur[2 * round + 1];
          float skk = 0.f, shk = 0.f, shh = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            skk += x0[r] * x0[r] + x1[r] * x1[r];
            shk += g4[0][r] * h0[r] * x0[r] + g4[1][r] * h1[r] * x1[r];
            shh += h0[r] * h0[r] + h1[r] * h1[r];
          }
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) {
            skk += __shfl_xor(skk, o);
            shk += __shfl_xor(shk, o);
            shh += __shfl_xor(shh, o);
          }
          if (valid) {
            if ((tid & 31) == 0) {
              float* out = g.partials + (m * (d / kBF) + tf) * 3;
              out[0] = skk;
              out[1] = shk;
              out[2] = shh;
            }
            if (g.k_out) {
              store4(g.k_out, m * d + f0 + f, io, x0[0], x0[1], x0[2], x0[3]);
              store4(g.k_out, m * d + f0 + f + 4, io, x1[0], x1[1], x1[2], x1[3]);
            }
          }
        } else if (valid) {
          store4(g.v_out, m * d + (f0 - d) + f, io, x0[0], x0[1], x0[2], x0[3]);
          store4(g.v_out, m * d + (f0 - d) + f + 4, io, x1[0], x1[1], x1[2], x1[3]);
        }
      }
      __syncthreads();
    }
  } else {
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const int64_t m = m0 + (wt * TB + b) * 32 + l32;
      if (m < g.M) {
#pragma unroll
        for (int a = 0; a < FB; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = f0 + (wf * FB + a) * 32 + q * 8 + lhalf * 4;
            *reinterpret_cast<floatx4*>(g.c_out + m * g.F + f) =
                floatx4{acc[a][b][q * 4], acc[a][b][q * 4 + 1], acc[a][b][q * 4 + 2],
                        acc[a][b][q * 4 + 3]};
          }
      }
    }
  }
}

template <int GT, int EPI, bool GATHER>
static hipError_t launch_one(const GemmArgs& g, hipStream_t s) {
  const int64_t tiles_m = (g.M + kBT - 1) / kBT;
  const int tiles_f = g.F / kBF;
  const int64_t tiles_m_x = (tiles_m + 7) / 8;
  const int64_t groups = (tiles_m_x + g.group_m - 1) / g.group_m;
  const int64_t blocks = 8 * groups * g.group_m * tiles_f;
  hipLaunchKernelGGL((gemm_kernel<GT, EPI, GATHER>), dim3((unsigned)blocks), dim3(kNT), 0, s, g);
  return hipGetLastError();
}

bool gemm_supported(GemmType type, const GemmArgs& g, bool gather) {
  const int es = type == GEMM_F32 ? 4 : 2;
  if (g.F % kBF != 0 || g.group_m < 1) return false;
  if (((int64_t)g.K * es) % (kStageBytes * kStages) != 0) return false;
  if (gather) {
    if (g.J < 1 || g.J > kGatherMaxJ || g.D * es < kStageBytes) return false;
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
  } else if (!gather) {
    if (type == GEMM_F16) return launch_one<GEMM_F16, EPI_STORE_F32, false>(g, s);
    if (type == GEMM_F32) return launch_one<GEMM_F32, EPI_STORE_F32, false>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace engram
