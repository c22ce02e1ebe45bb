// Launchers of the Engram HIP kernels (internal to libengram.so).
#pragma once

#include "common.h"

namespace engram {

// ---------------------------------------------------------------- hashing
hipError_t launch_hash(const int32_t* tokens, const int32_t* canon, int64_t N, int32_t T,
                       int32_t* idx, const HashArgs& args, hipStream_t s);

// ---------------------------------------------------------------- gather
// e[n][j*D..(j+1)*D) = base[j][idx[n][j]] for J tables of rows of row_bytes.
struct GatherArgs {
  const uint8_t* base[ENGRAM_MAX_TABLES];
  int32_t J;
  int32_t row_chunks;  // row_bytes / 16
  const float* row_scale;  // launch_gather only: null, or [N] (bf16 rows): e[n] /= row_scale[n]
};
hipError_t launch_gather(const int32_t* idx, uint8_t* e, int64_t N, const GatherArgs& g,
                         hipStream_t s);
// hash + gather with the rows repeated inside a tile of tokens read once (LDS);
// lds bytes per block, 0 when a tile's rows exceed what it may stage
size_t dedup_gather_lds_bytes(int32_t J, int32_t row_chunks);
hipError_t launch_dedup_gather(const int32_t* tokens, const int32_t* canon, int64_t N, int32_t T,
                               const HashArgs& a, const GatherArgs& g, uint8_t* e, int32_t* idx_out,
                               hipStream_t s);
// hash + gather in one launch; idx_out [N][J] (may be null) receives the indices
hipError_t launch_hash_gather(const int32_t* tokens, const int32_t* canon, int64_t N, int32_t T,
                              const HashArgs& a, const GatherArgs& g, uint8_t* e, int32_t* idx_out,
                              hipStream_t s);

// ---------------------------------------------------------------- GEMM
// C^T[f][m] = sum_k A[f][k] * B[m][k]; A: [F][K] (weights), B: [M][K] (tokens).
// GEMM_FP8: E4M3 operands with per-row scales (scale_a per A row, scale_b per B row)
enum GemmType { GEMM_BF16 = 0, GEMM_F16 = 1, GEMM_F32 = 2, GEMM_FP8 = 3 };
enum GemmEpilogue {
  EPI_KV = 0,   // forward: f < d -> gate partial sums (and optional k), f >= d -> v
  EPI_STORE_F32 = 1  // plain fp32 store of C[m][f] (backward de)
};
struct GemmArgs {
  const uint8_t* A;
  const uint8_t* B;
  int64_t M;
  int32_t F, K;
  int32_t group_m;     // token tiles walked per f-tile inside one XCD group
  int32_t reverse_m;   // nonzero: token tiles in descending order
  int32_t persistent;  // nonzero: one workgroup per CU loops over its XCD's tiles
  int32_t stage_bytes; // bytes of K per LDS stage: 64 (4-deep ring) or 128 (2-deep)
  // EPI_KV
  int32_t d;           // hidden width: f < branches*d are the branch keys, the rest v
  int32_t branches;    // keys of this many branches (0 or 1: one)
  int32_t io_dtype;    // ENGRAM_F32 / ENGRAM_BF16 of h, k_out, v_out
  const uint8_t* h;    // [branches][M][d]
  const float* gamma_q;
  const float* gamma_k;
  float* partials;     // [branches][M][d/BF][3]: sum k^2, sum g_q g_k h k, sum h^2
  uint8_t* k_out;      // [branches][M][d] or null
  uint8_t* v_out;      // [M][d]
  // EPI_STORE_F32
  float* c_out;        // [M][F]
  const float* col_scale;  // null, or [M]: C[m][:] is divided by col_scale[m] (a power of two)
  // B gathered from tables (forward only): B[m][j*D + c] = tables[j][idx[m][j]][c]
  const int32_t* idx;  // [M][J] or null (then B is read as a dense matrix)
  const uint8_t* tables[ENGRAM_MAX_TABLES];
  int32_t J, D;
  // GEMM_FP8: C^T[f][m] = scale_a[f] scale_b[m] sum_k A[f][k] B[m][k] over the codes
  const float* scale_a;  // [F]
  const float* scale_b;  // [M]
};
// Feature-tile width of the GEMM (the k/v boundary and partials use it).
constexpr int kGemmBF = 256;
bool gemm_supported(GemmType type, const GemmArgs& g, bool gather);
hipError_t launch_gemm(GemmType type, GemmEpilogue epi, const GemmArgs& g, hipStream_t s);

// ---------------------------------------------------------------- gate + conv
struct GateConvArgs {
  int64_t B, T;
  int32_t d, taps, nkt, io_dtype;
  int32_t branches;       // gates and outputs of this many branches; v is shared
  float eps;
  const float* partials;  // [branches][N][nkt][3]
  const uint8_t* v;       // [N][d]
  const float* conv_w;    // [d][taps]
  uint8_t* y;             // [branches][N][d]
  float* stats;           // [branches][N][4] or null
};
hipError_t launch_gate_conv(const GateConvArgs& a, hipStream_t s);

// ---------------------------------------------------------------- backward
struct BwdArgs {
  int64_t B, T;
  int32_t d, taps, io_dtype;
  const uint8_t* dy;      // [N][d]
  const uint8_t* v;       // [N][d]
  const uint8_t* k;       // [N][d]
  const uint8_t* h;       // [N][d]
  const float* stats;     // [N][4]
  const float* conv_w;    // [d][taps]
  const float* gamma_q;
  const float* gamma_k;
  uint8_t* dkv;           // [N][(branches+1)d] fp16 (bf16 io) or fp32 (f32 io): dk of each
                          // branch, then dv
  int32_t branches;       // M (1 for one branch)
  int32_t branch;         // the branch of this launch: its dy, h, k, stats, dh, pacc
  float* dv_acc;          // [N][d] fp32 when branches > 1: the shared v's gradient so far
  int32_t dv_mode;        // 0: write dv; 1: dv_acc = dv; 2: dv_acc += dv; 3: write dv + dv_acc
  // parameter gradients (null = not wanted)
  float* pacc;            // [nblk][d][taps+1]: per workgroup, sum_t dz_t vt_{t-i} per tap and
                          // sum_t (ds rq rk / sqrt d) h_t k_t (the RMSNorm scales' shared sum)
  uint8_t* dh;            // [N][d] io dtype: the gate's part of dL/dh
  int32_t pad_rows;       // zero rows N .. N+pad_rows-1 of dkv are written too
  const float* scale;     // [N] power-of-two factor of each token's dkv row, or null (1)
};
hipError_t launch_bwd_gate_conv(const BwdArgs& a, hipStream_t s);

// Per-token power-of-two scale s_t of the fp16 [dk | dv] rows (bf16 io): an
// upper bound of |dk_t|, |dv_t| from the upstream gradient, v and the saved
// gate statistics, times s_t, stays below 2^14.
struct BwdScaleArgs {
  int64_t B, T;
  int32_t d, taps, branches;
  const uint8_t* dy;      // [M][N][d] bf16
  const uint8_t* v;       // [N][d] bf16
  const float* stats;     // [M][N][4]
  const float* conv_w;    // [d][taps]
  const float* gamma_q;   // [M][d] or null
  const float* gamma_k;   // [M][d] or null
  float* scale;           // [N] out
};
hipError_t launch_bwd_scale(const BwdScaleArgs& a, hipStream_t s);
// out[n][:] = rows of e (bf16, [N][cols]) divided by scale[n] (exact: powers of two)
hipError_t launch_scale_rows_bf16(const uint8_t* e, const float* scale, int64_t N, int32_t cols,
                                  uint8_t* out, hipStream_t s);

// power-of-two helpers of the backward's per-token scales
__host__ __device__ inline float pow2_inverse(float s) {
  // s = 2^E (normal): 2^-E, exactly
  return __uint_as_float(0x7F000000u - __float_as_uint(s));
}
int64_t bwd_blocks(int64_t B, int64_t T);  // workgroups of the backward, rows of pacc
// pacc -> dconv [d][taps] and the RMSNorm scale gradients dgq = g_k S, dgk =
// g_q S (each output may be null); tmp holds bwd_param_tmp_floats() floats
int64_t bwd_param_tmp_floats(int64_t nblk, int32_t d, int32_t taps);
hipError_t launch_bwd_param_sums(const float* pacc, float* tmp, int64_t nblk, int32_t d,
                                 int32_t taps, const float* gamma_q, const float* gamma_k,
                                 float* dconv, float* dgq, float* dgk, hipStream_t s);

// ---------------------------------------------------------------- E4M3 quantization
// codes [rows][cols] and scales [rows] of a bf16 / fp32 matrix (cols % 8 == 0)
hipError_t launch_quant_rows(const uint8_t* src, int32_t io_dtype, int64_t rows, int32_t cols,
                             uint8_t* codes, float* scales, hipStream_t s);
// e_n = concat_j base[j][idx[n][j]] (bf16 rows) quantized per token: e8 [N][d_mem], se [N];
// one wavefront holds a token's row pieces, so d_mem <= kQuantMaxDmem
constexpr int kQuantMaxDmem = 4096;
hipError_t launch_gather_quant(const int32_t* idx, int64_t N, const GatherArgs& g, int32_t d_mem,
                               uint8_t* e8, float* se, hipStream_t s);

// ---------------------------------------------------------------- sharded exchange
struct ShardRows {
  int64_t rows[ENGRAM_MAX_TABLES];  // S_j = ceil(M_j / G): rows each GPU owns of table j
};
struct ShardTables {
  const uint8_t* base[ENGRAM_MAX_TABLES];  // this GPU's [S_j][D] shard of each table
};
struct ShardGrads {
  float* base[ENGRAM_MAX_TABLES];  // this GPU's [S_j][D] fp32 gradient of each shard
};
// Group sorted distinct keys ((j << 32) | row) by owner: send_ids (and with
// rows, the D-float rows) in send order, send_counts [G], send_pos [count]
// (send position of key s) and, with inverse, inverse[i] = send_pos[inverse[i]].
struct ShardPackArgs {
  const uint64_t* keys;
  const uint32_t* count_u32;  // device count of keys (one of the two)
  const int64_t* count_i64;
  int64_t capacity;           // upper bound of the count
  int32_t J, G;
  ShardRows shard_rows;
  int64_t* first;             // [J*G + 1] scratch
  int64_t* dest_base;         // [G*J] scratch
  int64_t* send_counts;       // [G] out
  uint32_t* send_ids;         // [capacity] out
  int32_t* send_pos;          // [capacity] out (may be null without inverse)
  const float* rows;          // [capacity][D] or null
  float* send_rows;           // [capacity][D] out with rows
  int32_t pieces;             // D / 4 with rows
  int32_t* inverse;           // [n_inverse] in/out or null
  int64_t n_inverse;
};
hipError_t launch_shard_pack(const ShardPackArgs& a, hipStream_t s);
hipError_t launch_shard_serve(const ShardTables& st, const uint32_t* ids, int64_t n, uint8_t* rows_out,
                              int32_t row_bytes, hipStream_t s);
hipError_t launch_shard_grad_add(const ShardGrads& sg, const uint32_t* ids, const float* rows,
                                 int64_t n, int32_t dim, hipStream_t s);

// dst[0..bytes) = src[0..bytes) (bytes % 16 == 0, 16-byte aligned buffers)
hipError_t launch_stream_copy(void* dst, const void* src, uint64_t bytes, hipStream_t s);

// Weight gradients dW[i][j] = sum_t X[t][i] Y[t][j] over token-major operands.
constexpr int kTnPadTokens = 64;  // X rows are padded to, and chunks are, multiples of this
struct GemmTnArgs {
  const uint8_t* x;  // [round_up(K, 64)][ldx] fp16 (GEMM_F16) or fp32; rows >= K are zero
  const uint8_t* y;  // [K][ldy] bf16 (GEMM_F16, widened in registers) or fp32
  int64_t ldx, ldy;  // row strides in elements
  int64_t K;         // tokens
  int32_t m, n;      // output rows (columns of X) and columns (of Y), multiples of 256
  int32_t splits;    // token chunks of kchunk tokens (the last may be short or empty)
  int64_t kchunk;    // a multiple of kTnPadTokens
  float* out;        // [splits][m][n] fp32 slices (unused with one split)
};
int tn_splits(int64_t K, int32_t m, int32_t n);
// p[0..n) = 0 (a kernel, so that it can sit in a captured graph)
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
// dst [m][n] fp32 = the sum of the splits' slices, in order
hipError_t launch_gemm_tn(GemmType type, const GemmTnArgs& g, float* dst, hipStream_t s);

// W_kv [2d][d_mem] (io dtype) -> Wt [d_mem][2d] (fp16 for bf16 io, fp32 for f32 io)
hipError_t launch_transpose_w(const uint8_t* w, uint8_t* wt, int32_t rows, int32_t cols,
                              int32_t io_dtype, hipStream_t s);

// Sort-by-row + segmented reduction of the table gradient.
struct SortBufs {
  uint32_t* keys[2];   // [J][N] ping-pong
  uint32_t* vals[2];   // [J][N]
  uint32_t* hist;      // [J][256][nblk]
  uint32_t* seg_count; // [J][nblk2] per-block head counts, then scanned
  uint32_t* seg_start; // [N*J]
  uint64_t* seg_key;   // [N*J]
  uint32_t* total;     // [1]
};
struct ScatterArgs {
  int64_t N;
  int32_t J, D;
  const int32_t* idx;     // [N][J]
  const float* de;        // [N][J*D]
  int32_t key_bits;       // bits of the largest row index
  float* dense[ENGRAM_MAX_TABLES];
  int64_t* keys_out;      // sparse
  float* rows_out;
  int64_t* count_out;
};
size_t sort_workspace_bytes(int64_t N, int32_t J);
void carve_sort(uint8_t* base, int64_t N, int32_t J, SortBufs* b);
hipError_t launch_sorted_scatter(const ScatterArgs& a, const SortBufs& b, int32_t mode,
                                 hipStream_t s);
hipError_t launch_atomic_scatter(const ScatterArgs& a, hipStream_t s);
// Distinct (table, row) keys of idx [N][J]: b.seg_key[0 .. b.total[0]) in
// table-major ascending order, and inverse[n][j] = position of idx[n][j]'s
// key among them.
hipError_t launch_dedup(const int32_t* idx, int64_t N, int32_t J, int32_t key_bits,
                        const SortBufs& b, int32_t* inverse, hipStream_t s);

}  // namespace engram
