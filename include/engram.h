/*
 * engram.h -- C ABI of the MI355X (gfx950) Engram conditional-memory library
 * (libengram.so).
 *
 * The operation is the Engram module described on the pages about DeepSeek's
 * "Conditional Memory via Scalable Lookup":
 *   - "DeepSeek AI II" (taking-lying-flat blog), section "DeepSeek Engram":
 *     tokenizer compression (a surjection P from raw to canonical ids), suffix
 *     N-grams g_{t,n} of canonical ids, K hash heads per order n, each with its
 *     own table E_{n,k} of prime size M_{n,k}, a multiplicative-XOR hash, the
 *     concatenated memory vector e_t, key/value projections W_K, W_V, RMSNorm
 *     on query h_t and key k_t before a scalar gate alpha_t in (0,1), the
 *     gated value alpha_t v_t, a short depthwise causal convolution, and the
 *     residual add H <- H + Y;
 *   - same page, system-efficiency part: retrieval depends on token ids only,
 *     so indices are known before the forward pass; training sends the row
 *     gradients back to the table rows; inference can keep the tables in host
 *     memory and fetch the needed rows over PCIe ahead of use;
 *   - the QbitAI mirror of the paper: one independent table per hash head.
 * The pages print no formulas; the forms used here are:
 *   c_t      = P[x_t]  (c_t = pad_id for t < 0, per sequence)
 *   idx_j(t) = (XOR_{i<n} (m_{j,i} * c_{t-i} mod 2^64)) mod M_j,  j = o*K + k
 *   e_t      = concat_j E_j[idx_j(t)]                     (d_mem = J*D)
 *   k_t = W_K e_t,  v_t = W_V e_t                          (W_* is [d][d_mem])
 *   alpha_t  = sigmoid(<g_q h_t rq_t, g_k k_t rk_t> / sqrt(d)),
 *              rq_t = (mean(h_t^2)+eps)^-1/2,  rk_t = (mean(k_t^2)+eps)^-1/2
 *   vt_t     = alpha_t v_t
 *   z_t      = sum_{i<taps} w[:,i] * vt_{t-i}               (vt = 0 before t=0)
 *   Y_t      = SiLU(z_t) + vt_t
 *
 * Conventions for every entry point:
 *   - Ownership: the caller allocates every device, pinned-host and workspace
 *     buffer; the library never allocates or frees device or pinned memory
 *     (only the host-side planner of engram_prefetch_plan uses ordinary host
 *     memory for its scratch, and the optional timing calls create events).
 *   - Streams: work is queued on the caller's hipStream_t (passed as void*,
 *     NULL = the default stream) without host synchronisation.  Calls are
 *     reentrant and may run on several streams at once if their buffers do
 *     not overlap.
 *   - Errors: arguments are validated on the host before any GPU work; a
 *     rejected call returns a non-zero engram_status and queues nothing.  A
 *     failed launch returns ENGRAM_E_HIP; faults inside kernels surface when
 *     the caller synchronises.  Token ids must lie in [0, vocab): this is a
 *     precondition that the device does not check unless the config asks
 *     for ENGRAM_FLAG_CHECK_IDS (the host planner always checks).
 *   - Layout: row-major, densely packed; N = B*T tokens, token n = b*T + t.
 *     Every pointer must be 16-byte aligned.
 *   - dtype: ENGRAM_F32 (float) or ENGRAM_BF16 (bfloat16) for tables,
 *     weights, hidden states, outputs and upstream gradients; the gate and
 *     conv arithmetic is always fp32, GEMMs accumulate in fp32.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ENGRAM_OK = 0,
  ENGRAM_E_INVALID = 1,     /* null pointer, bad size/shape, misalignment */
  ENGRAM_E_UNSUPPORTED = 2, /* well-formed but outside what the kernels handle */
  ENGRAM_E_WORKSPACE = 3,   /* workspace missing or smaller than engram_workspace_size() */
  ENGRAM_E_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  ENGRAM_E_SCRATCH = 5      /* engram_forward_noalloc: the call needs more than its fixed
                               scratch (ENGRAM_NOALLOC_SCRATCH_BYTES) */
} engram_status;

enum { ENGRAM_F32 = 0, ENGRAM_BF16 = 1 };

#define ENGRAM_MAX_ORDERS 4
#define ENGRAM_MAX_TABLES 32

/* engram_config.flags */
enum {
  /* Forward: read table rows inside the projection's operand loads instead of
   * gathering e into the workspace first (saves e's write and re-read, but the
   * row-indexed loads cost the projection more than the gather costs).  Ignored
   * when saved->e is requested or the shape is outside the fused loads. */
  ENGRAM_FLAG_FUSED_GATHER = 1u,
  /* The projections as one dense FP8 matmul ("DeepSeek AI II", section
   * "DeepSeek Engram", multi-branch integration): each row of W_KV and each
   * token's e_t are quantized to E4M3 with their own scale (as
   * engram_quantize_fp8), and the E4M3 matrix cores accumulate in fp32.  bf16
   * only, d_mem <= 4096; not with ENGRAM_FLAG_FUSED_GATHER (else
   * ENGRAM_E_UNSUPPORTED).  The backward is unchanged (it
   * takes the saved k, v of this forward and the bf16 weights). */
  ENGRAM_FLAG_FP8_PROJ = 2u,
  /* Token-id check for engram_hash_indices and engram_forward (over device
   * tables).  Retrieval depends on the token ids alone ("DeepSeek AI II",
   * section "DeepSeek Engram"), so an id outside [0, vocab) has no defined
   * canonical id.  Unchecked, such an id is a precondition violation: the
   * kernels would read canon_map out of bounds.  With this flag the call
   * zeroes *bad_ids, the kernels read every out-of-range id as canonical
   * pad_id (canon_map is never indexed out of bounds) and add one to
   * *bad_ids per such id, and the call then synchronises the stream and
   * returns ENGRAM_E_INVALID when *bad_ids > 0.  The outputs are still
   * written in full (with pad_id in place of the bad ids).  Costs one
   * stream synchronisation per call; compact-mode forwards read no ids. */
  ENGRAM_FLAG_CHECK_IDS = 4u,
  /* Forward over device tables: the hash + gather reads a (table, row) that
   * repeats inside a tile of 16 consecutive tokens once, into LDS, and writes
   * every token's copy from there ("DeepSeek AI II", system-efficiency part:
   * N-gram use is Zipf-distributed, so a few rows take most of the reads).
   * Same results as without the flag.  ENGRAM_E_UNSUPPORTED when a tile's
   * rows (16 * J * D * sizeof(dtype) bytes) exceed 64 KB.  Ignored in
   * compact mode (the plan already holds each row once), with
   * ENGRAM_FLAG_FUSED_GATHER and with ENGRAM_FLAG_FP8_PROJ. */
  ENGRAM_FLAG_GATHER_DEDUP = 8u
};

/* Shapes and addressing constants.  Host struct, read during the call only. */
typedef struct {
  int32_t vocab;          /* raw ids lie in [0, vocab) */
  int32_t canon_vocab;    /* canonical ids lie in [0, canon_vocab) */
  int32_t num_orders;     /* 1..ENGRAM_MAX_ORDERS */
  int32_t orders[ENGRAM_MAX_ORDERS]; /* N-gram orders, strictly ascending, each 1..4 */
  int32_t heads;          /* K hash heads per order; J = num_orders*heads <= 32 */
  int32_t dim;            /* D columns per table row; D*sizeof(dtype) % 16 == 0, J*D % 256 == 0;
                             D <= 256 for the backward */
  int32_t hidden;         /* d, width of h_t, k_t, v_t, Y_t; d % 256 == 0, d <= 8192 (bf16)
                             or 4096 (fp32) in the forward, d <= 4096 in the backward */
  int32_t conv_kernel;    /* taps of the causal depthwise conv, 1..8 */
  int32_t dtype;          /* ENGRAM_F32 or ENGRAM_BF16 */
  float rms_eps;          /* eps inside both RMSNorms (e.g. 1e-6) */
  int32_t pad_id;         /* canonical id used for positions before t = 0 */
  const int64_t* table_rows;   /* host [J]: M_j, 1 <= M_j < 2^31 (prime by design) */
  const uint64_t* multipliers; /* host [J][max order]: m_{j,i} multiplies c_{t-i} */
  uint32_t flags;              /* ENGRAM_FLAG_* bits, 0 for the defaults */
  int32_t branches;            /* M residual branches sharing the tables and W_V, each with
                                  its own W_K, hidden state, gate and output ("DeepSeek AI
                                  II", section "DeepSeek Engram", multi-branch integration);
                                  0 or 1 = one branch, at most ENGRAM_MAX_BRANCHES */
  uint32_t* bad_ids;           /* device [1], 4-byte aligned: out-of-range ids counted under
                                  ENGRAM_FLAG_CHECK_IDS (required then, ignored otherwise) */
} engram_config;

#define ENGRAM_MAX_BRANCHES 8

/* Learned parameters (device pointers). */
typedef struct {
  const int32_t* canon_map;               /* [vocab] raw id -> canonical id */
  const void* tables[ENGRAM_MAX_TABLES];  /* table j: [M_j][D] dtype */
  const void* w_kv;       /* [(M+1)d][d_mem] dtype: rows m*d..(m+1)*d-1 are W_K of branch m,
                             the last d rows W_V (M = branches; [2d][d_mem] for one branch) */
  const float* gamma_q;   /* [M][d] RMSNorm scale of each branch's query, NULL = all ones */
  const float* gamma_k;   /* [M][d] RMSNorm scale of each branch's key, NULL = all ones */
  const float* conv_w;    /* [d][conv_kernel] fp32, tap i multiplies vt_{t-i} */
} engram_params;

/* Optional forward outputs (device).  NULL members are not written.  The
 * table-gradient backward needs idx, stats, k and v.  M = branches. */
typedef struct {
  int32_t* idx;   /* [N][J] row indices idx_j(t) (table-local; compact-local in compact mode) */
  float* stats;   /* [M][N][4]: alpha_t, rq_t, rk_t, <g_q h_t, g_k k_t> (the last without rq, rk) */
  void* k;        /* [M][N][d] dtype */
  void* v;        /* [N][d] dtype */
  void* e;        /* [N][d_mem] dtype, the gathered memory vectors */
} engram_saved;

/*
 * Compact row buffer produced by engram_prefetch_plan() and consumed by
 * engram_forward() when the tables live in host memory.  All buffers are
 * caller-owned; capacity_rows >= N*J always suffices.
 */
typedef struct {
  int64_t capacity_rows;  /* rows that uniq_host, staging_host and rows_dev hold */
  int64_t total_rows;     /* out: unique rows over all tables */
  int64_t* counts;        /* host [J], out: unique rows per table */
  int32_t* uniq_host;     /* host [capacity_rows], out: ascending table-local rows, table after table */
  int32_t* inverse_host;  /* pinned host [N][J], out: row of token n, table j, in the compact buffer */
  void* staging_host;     /* pinned host [capacity_rows][D] dtype, out: the unique rows */
  void* rows_dev;         /* device [capacity_rows][D] dtype: async-copy destination of the rows */
  int32_t* inverse_dev;   /* device [N][J]: async-copy destination of inverse_host */
  void* ready_event;      /* hipEvent_t recorded on the side stream after the copies
                             (engram_forward waits on it when non-NULL) */
  uint32_t flags;         /* ENGRAM_PLAN_* bits, 0 for the defaults */
  /* HBM row ring: a cache of the rows earlier calls copied ("DeepSeek AI II",
   * system-efficiency part: Zipf-distributed N-gram use lets the frequent
   * rows sit in a faster tier).  ring_rows = 0: off (rows_dev holds this
   * call's rows only).  Otherwise rows_dev holds ring_rows rows used as a
   * ring.  Planning (a call without ENGRAM_PLAN_REUSE) points the inverse
   * map at rows an earlier call left in the ring, when no copy of this plan
   * or of the next one can overwrite them, reserves ring positions from
   * ring_head on for the rest, and leaves only those in counts, uniq_host
   * and total_rows; the copying call moves just them.  Each plan must be
   * copied before the next one is made.  A forward on plan k and the copies
   * of plan k+1 may be queued together only with consumed_event (below):
   * the copies rewrite inverse_dev, and without the ring rows_dev too. */
  int64_t ring_rows;      /* R >= 2 * capacity_rows, < 2^31; rows_dev holds R rows */
  int64_t* ring_pos;      /* host [sum_j M_j]: ring position (a count of appended rows) where
                             each table row was last copied, -1 = none; the caller sets all
                             to -1 before the first call and keeps it with the ring */
  int64_t ring_head;      /* in/out: rows appended to the ring so far */
  int64_t ring_hits;      /* out: distinct rows of the last planning call found in the ring */
  void* consumed_event;   /* NULL, or a hipEvent_t that orders the next plan's copies after
                             this plan's forward: a compact-mode engram_forward records it on
                             its stream once it has read rows_dev and inverse_dev for the last
                             time, and the copies of engram_prefetch_plan wait for it on the
                             side stream.  With it a forward on plan k may overlap the call
                             that copies plan k+1. */
} engram_compact;

/* engram_compact.flags */
enum {
  /* counts, uniq_host, inverse_host and total_rows already hold the plan of
   * these tokens (from an earlier call): skip hashing and sorting, only
   * gather and copy.  Lets the indices be planned ahead of time. */
  ENGRAM_PLAN_REUSE = 1u
};

/* Table-gradient output of engram_backward_table_grad(). */
enum {
  ENGRAM_GRAD_SORTED_SPARSE = 0, /* sort by (table,row) + segmented fp32 reduce -> {keys, rows, count} */
  ENGRAM_GRAD_SORTED_DENSE = 1,  /* same reduction, each unique row added into dense[j] (deterministic) */
  ENGRAM_GRAD_ATOMIC_DENSE = 2   /* fp32 atomicAdd of every token's slice into dense[j] (order varies) */
};

typedef struct {
  int32_t mode;          /* ENGRAM_GRAD_* */
  int64_t* keys;         /* SPARSE: device [N*J], out: (j << 32) | row, ascending */
  float* rows;           /* SPARSE: device [N*J][D], out: summed gradient of each key */
  int64_t* count;        /* SPARSE: device [1], out: number of keys */
  float* dense[ENGRAM_MAX_TABLES]; /* DENSE: device [M_j][D] fp32, gradients are ADDED (caller zeroes) */
} engram_table_grad;

/*
 * Gradients of the module's own parameters and of the hidden state, output of
 * engram_backward().  Every member may be NULL (not computed).  Outputs are
 * overwritten, not added to.  Chain rule through the forward of "DeepSeek AI
 * II", section "DeepSeek Engram" (the pages print no backward).
 */
typedef struct {
  float* w_kv;     /* [(M+1)d][d_mem] fp32: dL/dW_KV = sum_t [dk_t; dv_t] e_t^T, rows as in
                      params->w_kv (each branch's key rows, then the value rows) */
  float* conv_w;   /* [d][conv_kernel] fp32: sum_t dz_t[c] vt_{t-i}[c] */
  float* gamma_q;  /* [M][d] fp32: dL/dg_q (of params->gamma_q, or of all-ones scales when NULL) */
  float* gamma_k;  /* [M][d] fp32: dL/dg_k */
  void* hidden;    /* [M][B][T][d] dtype: the gate's part of dL/dh_t through the query's
                      RMSNorm (the residual H + Y adds G itself, which is the caller's) */
} engram_param_grad;

enum {
  ENGRAM_OP_FORWARD = 0,
  ENGRAM_OP_BACKWARD = 1,         /* engram_backward with table gradients only */
  ENGRAM_OP_BACKWARD_PARAMS = 2,  /* engram_backward with parameter gradients too */
  ENGRAM_OP_SHARD = 3             /* engram_shard_requests and engram_shard_grads */
};

#define ENGRAM_SHARD_MAX_GPUS 64

/* Bytes of device workspace the operation needs for B x T tokens (0 on bad config). */
size_t engram_workspace_size(const engram_config* cfg, int64_t B, int64_t T, int32_t op);

/* Static text for a status code. */
const char* engram_status_string(engram_status s);

/*
 * Canonicalisation + multi-head hashing ("DeepSeek AI II", section "DeepSeek
 * Engram": tokenizer compression, suffix N-grams, multi-head hashing into
 * prime-sized tables).  tokens: device [B][T] raw ids; canon_map: device
 * [vocab]; idx: device [B*T][J] int32 output.  Each batch row is its own
 * sequence (positions before its start read pad_id).
 */
engram_status engram_hash_indices(const engram_config* cfg, const int32_t* canon_map,
                                  const int32_t* tokens, int64_t B, int64_t T, int32_t* idx,
                                  void* stream);

/*
 * Forward pass: hashing, row gather and concatenation, key/value projection,
 * RMSNorm-dot-sigmoid gate, gated value, causal depthwise conv + SiLU +
 * residual ("DeepSeek AI II", section "DeepSeek Engram": retrieval, then
 * context-aware gating and the short causal convolution).
 *   tokens: device [B][T] (ignored in compact mode); hidden: device [M][B][T][d]
 *   dtype, the hidden state of each branch (M = branches); y: device
 *   [M][B][T][d] dtype output, each branch's Y (the caller adds it to its H);
 *   saved: NULL or buffers to keep (see engram_saved);
 *   compact: NULL, or the plan of engram_prefetch_plan(): rows are read from
 *   compact->rows_dev through compact->inverse_dev instead of params->tables;
 *   workspace: device, >= engram_workspace_size(cfg, B, T, ENGRAM_OP_FORWARD).
 */
engram_status engram_forward(const engram_config* cfg, const engram_params* params,
                             const int32_t* tokens, const void* hidden, int64_t B, int64_t T,
                             void* y, const engram_saved* saved, const engram_compact* compact,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): engram_forward without the workspace argument.  Its scratch
 * (the gathered e, v and the gate partial sums) is a fixed device array of
 * ENGRAM_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends; the call itself allocates nothing (no hipMalloc, no
 * events, no allocating library routine).  Inputs and outputs are the
 * caller's, as for engram_forward.  A call that needs more scratch than
 * that (engram_workspace_size(cfg, B, T, ENGRAM_OP_FORWARD) bounds it)
 * returns ENGRAM_E_SCRATCH before any GPU work.  The array belongs to the
 * current device (the stream must be one of its streams).  Every call on a
 * GPU shares that GPU's array and finds the last call's contents there
 * (nothing in the forward needs it cleared), so calls that overlap on one
 * GPU -- on two streams, or from two threads -- race: serialise them.
 */
#define ENGRAM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
engram_status engram_forward_noalloc(const engram_config* cfg, const engram_params* params,
                                     const int32_t* tokens, const void* hidden, int64_t B, int64_t T,
                                     void* y, const engram_saved* saved,
                                     const engram_compact* compact, void* stream);

/*
 * Table-gradient backward ("DeepSeek AI II", system-efficiency part: in
 * training the gradients of the gathered rows are dispatched back to the rows
 * they came from).  Chain rule through the conv, the gate, the RMSNorm of the
 * key and both projections to de_t, then dE_j[r] = sum_{t: idx_j(t)=r}
 * de_t[j*D:(j+1)*D] with fp32 accumulation.
 *   hidden, dy: device [M][B][T][d] dtype (M = branches); saved: idx,
 *   stats, k, v from engram_forward on the same inputs (required); out: see
 *   engram_table_grad (the gradients of all branches, summed);
 *   workspace: >= engram_workspace_size(cfg, B, T, ENGRAM_OP_BACKWARD).
 */
engram_status engram_backward_table_grad(const engram_config* cfg, const engram_params* params,
                                         const void* hidden, const void* dy, int64_t B, int64_t T,
                                         const engram_saved* saved, engram_table_grad* out,
                                         void* workspace, size_t ws_bytes, void* stream);

/*
 * Training backward: the table gradients of engram_backward_table_grad() and
 * the gradients of the projections, the conv taps, the RMSNorm scales and
 * the hidden state (see engram_param_grad), from one pass through the conv
 * and the gate.  table_out or param_out may be NULL (not computed), not both.
 *   saved: idx, stats, k, v as for the table gradients; saved->e, when given,
 *   is read for dW_KV, otherwise the rows are gathered again from
 *   params->tables through saved->idx (which must then be table-local: a
 *   forward over device tables, not a compact plan);
 *   workspace: >= engram_workspace_size(cfg, B, T, ENGRAM_OP_BACKWARD_PARAMS)
 *   when param_out is given, else ENGRAM_OP_BACKWARD.
 * With bf16 io the contractions take [dk_t | dv_t] in fp16, each token's
 * row times a power of two s_t chosen from a bound of its values so that
 * any scale of dy stays inside fp16's range (the factor comes out exactly:
 * de_t / s_t; dW_KV from the rows rounded to bf16 and e_t / s_t in bf16).
 * dW_KV sums in fp32 over token chunks, the chunks in a fixed order
 * (deterministic).
 * With M branches (the loss is the sum over the branches' outputs): hidden,
 * dy, saved->k and saved->stats hold every branch ([M][...] as in
 * engram_forward); the table, W_V and conv gradients sum the branches;
 * dW_KV has the rows of params->w_kv ([(M+1)d][d_mem]); the RMSNorm scale
 * gradients are [M][d] and the hidden-state gradient [M][B][T][d].
 * d a multiple of 256, and d_mem of 256 for the parameter gradients.
 */
engram_status engram_backward(const engram_config* cfg, const engram_params* params,
                              const void* hidden, const void* dy, int64_t B, int64_t T,
                              const engram_saved* saved, engram_table_grad* table_out,
                              engram_param_grad* param_out, void* workspace, size_t ws_bytes,
                              void* stream);

/*
 * Prefetch plan for tables held in host memory ("DeepSeek AI II",
 * system-efficiency part: indices are fixed by the token ids before the
 * forward pass, so rows are fetched asynchronously over PCIe while earlier
 * layers compute).  Runs on host threads: hashes tokens_host, sorts the
 * distinct rows of every table (plan->uniq_host, plan->counts), builds the
 * compact inverse map (plan->inverse_host), and -- when host_tables is not
 * NULL -- gathers the rows from the host tables into plan->staging_host and
 * queues hipMemcpyAsync of rows and inverse map to the device buffers on
 * side_stream, then records plan->ready_event there.  The rows are gathered
 * and queued in chunks, so the copy of one chunk runs while the next is
 * gathered.  With plan->ring_rows > 0 only the rows missing from the ring
 * are gathered and copied (see engram_compact).  Returns when the host work
 * is done; the copies run asynchronously and read inverse_host and
 * staging_host until ready_event fires, so a call on the same plan first
 * waits for that event (with no event, the caller must not reuse those
 * buffers before the copies end).  With ENGRAM_PLAN_REUSE in plan->flags the plan fields are
 * taken as given (a plan-only call made them) and only gather and copy run.
 *   canon_map_host: host [vocab]; tokens_host: host [B][T];
 *   host_tables: NULL (plan only) or host [J] pointers to [M_j][D] dtype, in
 *   any host memory (pageable is fine: host threads gather the rows from them
 *   into the pinned staging buffer, which is what the async copy reads).
 */
engram_status engram_prefetch_plan(const engram_config* cfg, const int32_t* canon_map_host,
                                   const int32_t* tokens_host, int64_t B, int64_t T,
                                   const void* const* host_tables, engram_compact* plan,
                                   void* side_stream);

/*
 * E4M3 quantization as the FP8 projection applies it ("DeepSeek AI II",
 * section "DeepSeek Engram", multi-branch integration: the projections as one
 * dense FP8 matmul): per row, s = max|x| / 448 (1 for an all-zero row) and
 * the OCP E4M3 codes of x / s (fp32 division, round to nearest even).
 *   src: device [rows][cols] dtype (ENGRAM_BF16 or ENGRAM_F32), cols % 8 == 0,
 *   16-byte aligned; codes: device [rows][cols] out, 8-byte aligned; scales:
 *   device [rows] fp32 out.  Errors: ENGRAM_E_UNSUPPORTED for another dtype,
 *   ENGRAM_E_INVALID for a null or misaligned pointer or a bad size.
 */
engram_status engram_quantize_fp8(const void* src, int32_t dtype, int64_t rows, int32_t cols,
                                  uint8_t* codes, float* scales, void* stream);

/*
 * Table-sharded row exchange: the device steps of one GPU ("DeepSeek AI II",
 * system-efficiency part: tables too large for one GPU are sharded over GPUs,
 * and each step exchanges the requested rows, then their gradients, by
 * All-to-All).  With G GPUs (1 <= G <= ENGRAM_SHARD_MAX_GPUS), GPU g owns rows
 * [g S_j, (g+1) S_j) of table j, S_j = ceil(M_j / G) < 2^27, and a request
 * names a row by the id (j << 27) | (row - g S_j).  The All-to-All transfers
 * themselves (RCCL) are the caller's; these calls prepare and consume their
 * buffers.  Errors: ENGRAM_E_INVALID for null or misaligned buffers or G out
 * of range, ENGRAM_E_UNSUPPORTED for shards of 2^27 rows or more.
 */

/* Sender, forward: the distinct rows that idx (device [N][J], table-local
 * rows from a forward's saved idx or engram_hash_indices) requests, grouped
 * by owner.
 *   send_ids: device [N*J] out: owner 0's requests first, each owner's table
 *   by table in ascending rows; send_counts: device [G] int64 out;
 *   inverse: device [N][J] int32 out: where token n's row of table j sits in
 *   the send order, which is the order the owners' replies come back in.
 *   The compact-mode forward then reads the replies (engram_compact:
 *   rows_dev = the replies, inverse_dev = inverse, no host plan).
 *   workspace >= engram_workspace_size(cfg, 1, N, ENGRAM_OP_SHARD). */
engram_status engram_shard_requests(const engram_config* cfg, int32_t G, const int32_t* idx,
                                    int64_t N, uint32_t* send_ids, int64_t* send_counts,
                                    int32_t* inverse, void* workspace, size_t ws_bytes,
                                    void* stream);

/* Owner, forward: rows_out[i] = row (ids[i] & (2^27 - 1)) of this GPU's
 * shard of table ids[i] >> 27, for n received request ids.
 *   shard_tables: device [J] pointers to [S_j][D] dtype; rows_out: device
 *   [n][D] dtype. */
engram_status engram_shard_serve(const engram_config* cfg, int32_t G,
                                 const void* const* shard_tables, const uint32_t* ids, int64_t n,
                                 void* rows_out, void* stream);

/* Sender, backward: the sparse table gradient (keys, rows, count of
 * engram_backward with ENGRAM_GRAD_SORTED_SPARSE) grouped by owner in the
 * order of engram_shard_requests.  count: device [1]; capacity >= count (N*J
 * suffices); send_ids: device [capacity] out; send_rows: device [capacity][D]
 * fp32 out; send_counts: device [G] out.
 *   workspace >= engram_workspace_size(cfg, 1, 1, ENGRAM_OP_SHARD). */
engram_status engram_shard_grads(const engram_config* cfg, int32_t G, const int64_t* keys,
                                 const float* rows, const int64_t* count, int64_t capacity,
                                 uint32_t* send_ids, float* send_rows, int64_t* send_counts,
                                 void* workspace, size_t ws_bytes, void* stream);

/* Owner, backward: adds the received gradient rows into this GPU's shards
 * of the fp32 table gradient, one sender's block after the other (a fixed
 * order, no atomics: ids are distinct within a block).
 *   ids, rows: device, nblocks blocks back to back, block b of
 *   counts_host[b] ids and [counts_host[b]][D] fp32 rows; shard_grads: device
 *   [J] pointers to [S_j][D] fp32, added to. */
engram_status engram_shard_reduce(const engram_config* cfg, int32_t G, float* const* shard_grads,
                                  const uint32_t* ids, const float* rows,
                                  const int64_t* counts_host, int32_t nblocks, void* stream);

/*
 * Measurement reference: a plain device-to-device copy of bytes (a multiple
 * of 16; both buffers 16-byte aligned, not overlapping) queued on stream.
 * Its rate is the achievable HBM bandwidth that the memory-bound kernels are
 * compared with, beside the 8 TB/s peak.  ENGRAM_E_INVALID for bad sizes or
 * pointers.
 */
engram_status engram_device_copy(void* dst, const void* src, size_t bytes, void* stream);

/*
 * Kernel timing for measurement: while enabled, every kernel the library
 * launches is bracketed by a pair of hipEvents on its stream.
 * engram_profile_read() synchronises those events and returns, per kernel
 * name, the number of launches and the summed milliseconds (at most
 * max_entries entries; names are written NUL-separated into names).
 * Returns the number of entries, or -1 on error.
 */
void engram_profile_enable(int32_t on);
void engram_profile_reset(void);
int32_t engram_profile_read(char* names, size_t names_len, int64_t* launches, double* total_ms,
                            int32_t max_entries);

#ifdef __cplusplus
}
#endif
#endif /* ENGRAM_H */
