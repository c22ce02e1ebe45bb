// Weight gradients of the key and value projections ("DeepSeek AI II",
// section "DeepSeek Engram": k_t = W_K e_t and v_t = W_V e_t share the
// retrieved memory e_t), on CDNA4 matrix cores:
//   dW[i][j] = sum_t X[t][i] Y[t][j],   X = [dk_t | dv_t], Y = e_t.
// Both operands are token-major (a token's features are contiguous) and the
// contraction runs over tokens.  Stages of KS tokens go to LDS as they lie in
// memory (direct-to-LDS 16-byte loads of whole token rows), and the MFMA
// fragments, which hold 8 consecutive K values per lane, are read across the
// rows with the 16-bit transposing LDS read (ds_read_b64_tr_b16: in each
// group of 16 lanes, lane 4r+c supplies 4 values of row r and lane j receives
// column j of the 4 rows; two reads give a lane its 8 K values).  X arrives
// in fp16 (each token's row times a power of two that keeps it inside fp16's
// range) and is rounded to bf16 in registers; Y is e in bf16 with each row
// divided by the same power of two, so the product needs no other factor.
// fp32 operands (small shapes) read their 4 K values with 4 LDS reads.
//
// Tiles are 256 x 256 outputs per workgroup of 4 wavefronts (128 x 128 each,
// 16 accumulators of 32x32).  The token range is split into chunks so that
// the few output tiles fill the chip; each chunk writes its own fp32 slice
// and tn_reduce_kernel sums the slices in order (deterministic).
#include <algorithm>

#include "kernels.h"
#include "mfma_ring.h"

namespace engram {

// Stage shapes: KS tokens per stage in a ring of NS stages; both operands of
// all stages fill 128 KB of LDS.
#ifndef ENGRAM_TN_KS
#define ENGRAM_TN_KS 32
#endif
#ifndef ENGRAM_TN_NS
#define ENGRAM_TN_NS 4
#endif
template <int GT>
struct TnShape;
template <>
struct TnShape<GEMM_F16> {
  static constexpr int ES = 2;   // bytes per element in LDS (fp16 X, bf16 Y)
  static constexpr int KS = ENGRAM_TN_KS;  // tokens per stage
  static constexpr int NS = ENGRAM_TN_NS;  // stages in the ring
  static constexpr int KK = 16;  // tokens per MFMA step (8 per lane half)
};
template <>
struct TnShape<GEMM_F32> {
  static constexpr int ES = 4;
  static constexpr int KS = 16;
  static constexpr int NS = 4;
  static constexpr int KK = 8;   // 4 per lane half, four 32x32x2 MFMAs
};
static_assert(TnShape<GEMM_F16>::KS <= kTnPadTokens && kTnPadTokens % TnShape<GEMM_F16>::KS == 0, "");

// 16-byte piece p of LDS row r sits at piece p ^ tn_swz(r).  A transposing
// read covers 4 consecutive rows x 32 bytes per 16 lanes; XOR with 2(r & 3)
// spreads them over 8 distinct pieces (measured 2 % faster than 4(r & 3),
// which separates the 64-byte spans of a half wave instead).
#ifndef ENGRAM_TN_SWZ
#define ENGRAM_TN_SWZ 1
#endif
__device__ inline int tn_swz(int r) { return (r & 3) << ENGRAM_TN_SWZ; }

typedef __fp16 half4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) half4_t lds_half4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) float lds_f32;

__device__ inline u32x2 read_tr16(const lds_u8* base, uint32_t byte) {
  const half4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_half4*)(base + byte));
  return __builtin_bit_cast(u32x2, v);
}

// two fp16 (bits in a 32-bit word) -> two bf16, round to nearest even
__device__ inline uint32_t f16x2_to_bf16x2(uint32_t u) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 h = __builtin_bit_cast(h2, u);
  return pack_bf16x2((float)h[0], (float)h[1]);
}

template <int GT>
__global__ __launch_bounds__(256, 1) void gemm_tn_kernel(GemmTnArgs g) {
  using S = TnShape<GT>;
  constexpr int ES = S::ES, KS = S::KS, KK = S::KK, NS = S::NS;
  constexpr int RB = 256 * ES;              // bytes of a token row in LDS
  constexpr int kTnOperand = KS * RB;       // bytes of one operand in one stage
  constexpr int NL = kTnOperand / (256 * 16);  // loads per operand, thread and stage
  static_assert(NS * 2 * kTnOperand == 131072, "");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * 2 * kTnOperand];

  // ---- work item: XCD-major so that the items one XCD runs at a time share
  // a token chunk and neighbouring tiles (their operand rows meet in its L2)
  const int tiles_n = g.n / 256;
  const int64_t tiles = (int64_t)(g.m / 256) * tiles_n;
  const int64_t items = tiles * g.splits;
  const int64_t per_xcd = (items + 7) / 8;
  const int64_t item = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= items) return;
  const int split = (int)(item / tiles);
  const int64_t tile = item % tiles;
  const int i0 = (int)(tile / tiles_n) * 256;
  const int j0 = (int)(tile % tiles_n) * 256;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wf = wave & 1, wt = wave >> 1;
  const int l32 = lane & 31, lhalf = lane >> 5;

  const int64_t Kpad = (g.K + KS - 1) / KS * KS;
  const int64_t kbeg = (int64_t)split * g.kchunk;
  const int64_t kend = kbeg + g.kchunk < Kpad ? kbeg + g.kchunk : Kpad;
  const int nst = kend > kbeg ? (int)((kend - kbeg) / KS) : 0;

  // ---- loads: wave-wide load q of an operand fills bytes [L*1024, L*1024+1024)
  // of the stage (L = wave*NL + q): token row r, slot s, logical piece s^swz(r)
  uint32_t voffX[NL];
  int rowL[NL], pieceL[NL];
  const int ldyb = (int)(g.ldy * ES);  // bytes per Y row (< 2^26, checked at launch)
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    const int byte = (wave * NL + q) * 1024 + lane * 16;
    const int r = byte / RB;
    const int p = (byte % RB) / 16 ^ tn_swz(r);
    rowL[q] = r;
    pieceL[q] = p;
    voffX[q] = (uint32_t)(r * g.ldx * ES + p * 16);
  }
  const uint32_t lds0 = lds_addr(ring);
  // Stage st into ring slot sl.  Rows of X at and beyond K are zero in
  // memory; rows of Y beyond K-1 are read as row K-1 (finite values times
  // zero).  Stages past the end re-load the last one into a slot that is
  // never read, so every stage issues the same number of loads.
  auto issue = [&](int st, int sl) __attribute__((always_inline)) {
    st = st < nst ? st : nst - 1;
    const int64_t k0 = kbeg + (int64_t)st * KS;
    const uint8_t* bx = g.x + (k0 * g.ldx + i0) * ES;
    const uint8_t* by = g.y + (k0 * g.ldy + j0) * ES;
    const uint32_t mx = lds0 + sl * 2 * kTnOperand + wave * NL * 1024;
    const uint32_t my = mx + kTnOperand;
    // last row of Y in this stage (KS-1 except in the stage holding row K-1)
    const int last = (int)(g.K - 1 - k0 < KS - 1 ? g.K - 1 - k0 : KS - 1);
    const M0Keep keep;
#pragma unroll
    for (int q = 0; q < NL; ++q) load_lds16_s_kept(voffX[q], bx, mx + q * 1024);
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const int r = rowL[q] < last ? rowL[q] : last;
      load_lds16_s_kept((uint32_t)(r * ldyb + pieceL[q] * 16), by, my + q * 1024);
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx16{};

  const lds_u8* lbase = (const lds_u8*)(const __attribute__((address_space(3))) void*)ring;
  // Fragment of 32 columns (block blk of this wave's 128) at MFMA step ss of
  // the operand tile at byte `tb`: 8 K values of column cb + l32 per lane,
  // as stored (Y still in bf16).
  auto frag = [&](uint32_t tb, int cb, int ss) __attribute__((always_inline)) {
    u32x4 f;
    if constexpr (GT == GEMM_F16) {
      const int j = lane & 15;
      const int col = cb + ((lane >> 4) & 1) * 16 + (j & 3) * 4;
      const int r0 = ss * KK + lhalf * 8 + (j >> 2);
      const uint32_t pc = (uint32_t)(col * 2) / 16, in = (uint32_t)(col * 2) % 16;
      const u32x2 lo = read_tr16(lbase, tb + r0 * RB + ((pc ^ tn_swz(r0)) * 16) + in);
      const u32x2 hi = read_tr16(lbase, tb + (r0 + 4) * RB + ((pc ^ tn_swz(r0 + 4)) * 16) + in);
      f = u32x4{lo.x, lo.y, hi.x, hi.y};
    } else {
      const int col = cb + l32;
      const uint32_t pc = (uint32_t)(col * 4) / 16, in = (uint32_t)(col * 4) % 16;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = ss * KK + lhalf * 4 + c;
        f[c] = __float_as_uint(*(const lds_f32*)(lbase + tb + r * RB + ((pc ^ tn_swz(r)) * 16) + in));
      }
    }
    return f;
  };

  // Ring protocol.  Stage kt's loads were issued NS-1 stages ahead.  The
  // wait and barrier for stage kt+1 come before the last MFMA step of stage
  // kt, so that stage kt+1's first fragments are read while that step's
  // MFMAs run; within a stage, step s+1's fragments are read during step s.
  // Waiting for this wave's LDS reads at each barrier makes the slot that
  // the next issue overwrites free in every wave.
  constexpr int SP = KS / KK;  // MFMA steps per stage
  static_assert(SP % 2 == 0, "a stage starts in fragment buffer 0");
  u32x4 af[2][4], bf[2][4];
  auto read_step = [&](int slot, int ss, u32x4* a4, u32x4* b4) __attribute__((always_inline)) {
    const uint32_t tx = (uint32_t)(slot * 2 * kTnOperand);
#pragma unroll
    for (int a = 0; a < 4; ++a) a4[a] = frag(tx, wf * 128 + a * 32, ss);
#pragma unroll
    for (int b = 0; b < 4; ++b) b4[b] = frag(tx + kTnOperand, wt * 128 + b * 32, ss);
  };
  // fp16 X is rounded to bf16 (Y, the bf16 rows of e divided by the tokens'
  // scales, may lie outside fp16's range) a fragment at a time, each feeding
  // 4 MFMAs, so the conversions overlap the matrix pipe instead of preceding it
  auto mfma_step = [&](const u32x4* a4, const u32x4* b4) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      u32x4 x = a4[a];
      if constexpr (GT == GEMM_F16) {
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = f16x2_to_bf16x2(x[c]);
#pragma unroll
        for (int b = 0; b < 4; ++b) Mma<GEMM_BF16>::run(x, b4[b], acc[a][b]);
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) Mma<GT>::run(x, b4[b], acc[a][b]);
      }
    }
  };
  if (nst > 0) {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s, s);
    ENGRAM_WAIT_VM((NS - 2) * 2 * NL);
    ENGRAM_BARRIER();
    read_step(0, 0, af[0], bf[0]);
    for (int kt = 0; kt < nst; ++kt) {
      issue(kt + NS - 1, (kt + NS - 1) % NS);  // the slot stage kt-1 used
      const int slot = kt % NS;
#pragma unroll
      for (int ss = 0; ss < SP; ++ss) {
        const int cur = ss & 1, nxt = cur ^ 1;  // SP is even: stage k starts in buffer 0
        if (ss + 1 < SP) {
          read_step(slot, ss + 1, af[nxt], bf[nxt]);
        } else {
          __builtin_amdgcn_sched_barrier(0);  // the previous step's MFMAs stay ahead of the wait
          ENGRAM_WAIT_VM_LDS((NS - 2) * 2 * NL);  // stage kt+1 in LDS, this wave's reads done
          ENGRAM_BARRIER();
          if (kt + 1 < nst) read_step((kt + 1) % NS, 0, af[nxt], bf[nxt]);
        }
        mfma_step(af[cur], bf[cur]);
      }
    }
    ENGRAM_WAIT_VM(0);  // the loads of stages past the end
  }

  // ---- epilogue: lane owns column j0 + wt*128 + b*32 + l32 and rows
  // i0 + wf*128 + a*32 + 8q + 4*lhalf + r (accumulator element 4q + r)
  float* out = g.out + (size_t)split * g.m * g.n;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t i = i0 + wf * 128 + a * 32 + q * 8 + lhalf * 4 + r;
          const int64_t j = j0 + wt * 128 + b * 32 + l32;
          out[i * g.n + j] = acc_read(acc[a][b][q * 4 + r]);
        }
}

// dst[e] = sum_s src[s][e], s in order
__global__ __launch_bounds__(256) void tn_reduce_kernel(const float* __restrict__ src,
                                                        float* __restrict__ dst, int64_t count4,
                                                        int splits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count4) return;
  const floatx4* s4 = reinterpret_cast<const floatx4*>(src);
  floatx4 acc = s4[i];
  for (int s = 1; s < splits; ++s) acc += s4[(int64_t)s * count4 + i];
  reinterpret_cast<floatx4*>(dst)[i] = acc;
}

int tn_splits(int64_t K, int32_t m, int32_t n) {
  // enough items for 256 CUs with little idle time in the last round, each
  // split at least 4 chunks of kTnPadTokens tokens
  const int64_t tiles = (int64_t)(m / 256) * (n / 256);
  const int64_t kc = (K + kTnPadTokens - 1) / kTnPadTokens;
  int smax = (int)std::min<int64_t>(32, std::max<int64_t>(1, kc / 4));
  for (int s = 1; s <= smax; ++s) {
    const int64_t items = tiles * s;
    const int64_t rounds = (items + 255) / 256;
    if (items >= 256 && items * 10 >= rounds * 256 * 9) return s;
  }
  return smax;
}

hipError_t launch_gemm_tn(GemmType type, const GemmTnArgs& g0, float* dst, hipStream_t s) {
  GemmTnArgs g = g0;
  if (g.m % 256 || g.n % 256 || g.m <= 0 || g.n <= 0 || g.K < 0 || g.splits < 1)
    return hipErrorInvalidValue;
  if (type != GEMM_F16 && type != GEMM_F32) return hipErrorInvalidValue;
  // 32-bit per-lane offsets inside a stage; chunks of whole stages
  const int es = type == GEMM_F16 ? 2 : 4;
  if ((int64_t)kTnPadTokens * std::max(g.ldx, g.ldy) * es >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  if (g.kchunk % kTnPadTokens != 0) return hipErrorInvalidValue;
  if (g.splits == 1) g.out = dst;
  const int64_t items = (int64_t)(g.m / 256) * (g.n / 256) * g.splits;
  const int64_t blocks = (items + 7) / 8 * 8;
  if (type == GEMM_F16)
    hipLaunchKernelGGL(gemm_tn_kernel<GEMM_F16>, dim3((unsigned)blocks), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_tn_kernel<GEMM_F32>, dim3((unsigned)blocks), dim3(256), 0, s, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.splits == 1) return e;
  const int64_t count4 = (int64_t)g.m * g.n / 4;
  hipLaunchKernelGGL(tn_reduce_kernel, dim3((unsigned)((count4 + 255) / 256)), dim3(256), 0, s,
                     g.out, dst, count4, g.splits);
  return hipGetLastError();
}

}  // namespace engram
