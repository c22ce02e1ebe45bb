// C ABI of libengram.so: argument validation (host only, before any GPU
// work), workspace sizing and carving, launch orchestration on the caller's
// stream, the host-side prefetch planner, and optional kernel timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "kernels.h"

using namespace engram;

namespace {

struct Shape {
  int J, D, d, d_mem, taps, max_order, es;
  int32_t dtype;
  int key_bits;
  uint32_t flags;
  int M;  // branches
};

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
// LDS stage shape of the MFMA GEMMs (bytes of K per stage; see gemm.hip).
// Two 128-byte stages: the four-deep ring of 64-byte stages hides more load
// latency (fewer cycles per tile) but runs at a lower clock under the power
// limit and measured slower.
#ifndef ENGRAM_FWD_STAGE_BYTES
#define ENGRAM_FWD_STAGE_BYTES 128
#endif
constexpr int32_t kFwdStageBytes = ENGRAM_FWD_STAGE_BYTES;
#ifndef ENGRAM_GEMM_PERSISTENT
#define ENGRAM_GEMM_PERSISTENT 1
#endif
constexpr int32_t kBwdStageBytes = 128;
// token tiles per group in the de contraction's tile walk (its five f-tiles
// per token tile): 2 measured 2-3.5 % faster than the projection's 4
#ifndef ENGRAM_DE_GROUP_M
#define ENGRAM_DE_GROUP_M 2
#endif
inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

engram_status check_config(const engram_config* c, Shape* s) {
  if (!c || !c->table_rows || !c->multipliers) return ENGRAM_E_INVALID;
  if (c->num_orders < 1 || c->num_orders > ENGRAM_MAX_ORDERS) return ENGRAM_E_INVALID;
  if (c->heads < 1) return ENGRAM_E_INVALID;
  const int J = c->num_orders * c->heads;
  if (J > ENGRAM_MAX_TABLES) return ENGRAM_E_UNSUPPORTED;
  int max_order = 0;
  for (int o = 0; o < c->num_orders; ++o) {
    if (c->orders[o] < 1 || c->orders[o] > ENGRAM_MAX_ORDERS) return ENGRAM_E_INVALID;
    if (o > 0 && c->orders[o] <= c->orders[o - 1]) return ENGRAM_E_INVALID;
    max_order = std::max(max_order, c->orders[o]);
  }
  if (c->dtype != ENGRAM_F32 && c->dtype != ENGRAM_BF16) return ENGRAM_E_UNSUPPORTED;
  if (c->vocab < 1 || c->canon_vocab < 1) return ENGRAM_E_INVALID;
  if (c->pad_id < 0) return ENGRAM_E_INVALID;
  if (c->dim < 1 || c->hidden < 1) return ENGRAM_E_INVALID;
  if (c->conv_kernel < 1 || c->conv_kernel > 8) return ENGRAM_E_UNSUPPORTED;
  if (!(c->rms_eps >= 0.f)) return ENGRAM_E_INVALID;
  if (c->flags & ~(uint32_t)(ENGRAM_FLAG_FUSED_GATHER | ENGRAM_FLAG_FP8_PROJ | ENGRAM_FLAG_CHECK_IDS |
                             ENGRAM_FLAG_GATHER_DEDUP))
    return ENGRAM_E_INVALID;
  if ((c->flags & ENGRAM_FLAG_CHECK_IDS) && (!c->bad_ids || ((uintptr_t)c->bad_ids & 3u)))
    return ENGRAM_E_INVALID;
  // the FP8 projection quantizes bf16 rows; the fused row gather reads bf16 tables itself
  if ((c->flags & ENGRAM_FLAG_FP8_PROJ) &&
      (c->dtype != ENGRAM_BF16 || (c->flags & ENGRAM_FLAG_FUSED_GATHER)))
    return ENGRAM_E_UNSUPPORTED;
  if (c->branches < 0 || c->branches > ENGRAM_MAX_BRANCHES) return ENGRAM_E_INVALID;
  const int es = (int)dtype_size(c->dtype);
  if ((c->dim * es) % 16 != 0) return ENGRAM_E_UNSUPPORTED;
  const int d_mem = J * c->dim;
  if (d_mem % kGemmBF != 0) return ENGRAM_E_UNSUPPORTED;
  if ((c->flags & ENGRAM_FLAG_FP8_PROJ) && d_mem > kQuantMaxDmem) return ENGRAM_E_UNSUPPORTED;
  if ((c->flags & ENGRAM_FLAG_GATHER_DEDUP) && dedup_gather_lds_bytes(J, c->dim * es / 16) == 0)
    return ENGRAM_E_UNSUPPORTED;
  if (c->hidden % kGemmBF != 0) return ENGRAM_E_UNSUPPORTED;
  if (c->hidden / (c->dtype == ENGRAM_BF16 ? 8 : 4) > 1024) return ENGRAM_E_UNSUPPORTED;
  int64_t max_rows = 1;
  for (int j = 0; j < J; ++j) {
    if (c->table_rows[j] < 1 || c->table_rows[j] >= (int64_t(1) << 31)) return ENGRAM_E_INVALID;
    max_rows = std::max(max_rows, (int64_t)c->table_rows[j]);
  }
  int bits = 1;
  while (bits < 31 && (int64_t(1) << bits) < max_rows) ++bits;
  s->J = J;
  s->D = c->dim;
  s->d = c->hidden;
  s->d_mem = d_mem;
  s->taps = c->conv_kernel;
  s->max_order = max_order;
  s->es = es;
  s->dtype = c->dtype;
  s->key_bits = bits;
  s->flags = c->flags;
  s->M = c->branches > 0 ? c->branches : 1;
  return ENGRAM_OK;
}

HashArgs make_hash_args(const engram_config* c, const Shape& s) {
  HashArgs a;
  std::memset(&a, 0, sizeof(a));
  a.J = s.J;
  a.num_orders = c->num_orders;
  a.heads = c->heads;
  a.max_order = s.max_order;
  a.pad_id = c->pad_id;
  for (int o = 0; o < c->num_orders; ++o) a.orders[o] = c->orders[o];
  for (int j = 0; j < s.J; ++j) {
    a.prime[j] = (uint32_t)c->table_rows[j];
    a.recip[j] = mod_recip(a.prime[j]);
    for (int i = 0; i < s.max_order; ++i) a.mult[j * s.max_order + i] = c->multipliers[j * s.max_order + i];
  }
  a.bad = (c->flags & ENGRAM_FLAG_CHECK_IDS) ? c->bad_ids : nullptr;
  a.vocab = c->vocab;
  return a;
}

// ENGRAM_FLAG_CHECK_IDS: zero the caller's counter before the hash kernels
// run (a kernel, not a memset, so the call can sit in a captured graph)...
engram_status id_check_begin(const engram_config* c, hipStream_t s) {
  if (!(c->flags & ENGRAM_FLAG_CHECK_IDS)) return ENGRAM_OK;
  return launch_zero_f32(reinterpret_cast<float*>(c->bad_ids), 1, s) == hipSuccess ? ENGRAM_OK
                                                                                  : ENGRAM_E_HIP;
}
// ... and after the call's kernels: wait for them and report bad ids.
engram_status id_check_end(const engram_config* c, hipStream_t s) {
  if (!(c->flags & ENGRAM_FLAG_CHECK_IDS)) return ENGRAM_OK;
  uint32_t bad = 0;
  if (hipMemcpyAsync(&bad, c->bad_ids, sizeof(bad), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return ENGRAM_E_HIP;
  return bad ? ENGRAM_E_INVALID : ENGRAM_OK;
}

inline engram_status hip_status(hipError_t e) { return e == hipSuccess ? ENGRAM_OK : ENGRAM_E_HIP; }

// ---------------------------------------------------------------- timing
std::mutex g_prof_mu;
bool g_prof_on = false;
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};
std::vector<ProfRec> g_prof;

// Set while an allocation-free call runs on this thread: no timing events.
thread_local bool t_quiet = false;
struct QuietTiming {
  bool prev;
  explicit QuietTiming(bool on) : prev(t_quiet) { t_quiet = t_quiet || on; }
  ~QuietTiming() { t_quiet = prev; }
};

class Timed {
 public:
  Timed(const char* name, hipStream_t s) : name_(name), s_(s) {
    {
      std::lock_guard<std::mutex> l(g_prof_mu);
      on_ = g_prof_on && !t_quiet;
    }
    if (on_) {
      on_ = hipEventCreate(&a_) == hipSuccess && hipEventCreate(&b_) == hipSuccess &&
            hipEventRecord(a_, s_) == hipSuccess;
    }
  }
  ~Timed() {
    if (!on_) return;
    if (hipEventRecord(b_, s_) != hipSuccess) return;
    std::lock_guard<std::mutex> l(g_prof_mu);
    g_prof.push_back({name_, a_, b_});
  }

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t a_{}, b_{};
  bool on_ = false;
};

// ---------------------------------------------------------------- fixed scratch
// engram_forward_noalloc's workspace: a device array in the library's code
// object, so the call allocates nothing.  In host code `scratch` names a
// host-side stand-in, not the device address: the address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that pointer is handed to kernels.  Every call on a device shares its
// array, so calls that overlap on one device race.
constexpr size_t kScratchBytes = ENGRAM_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

engram_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ENGRAM_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ENGRAM_E_UNSUPPORTED;
  std::lock_guard<std::mutex> l(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return ENGRAM_E_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return ENGRAM_OK;
}

// ---------------------------------------------------------------- workspace
struct FwdWs {
  int32_t* idx;
  uint8_t* e;
  uint8_t* v;
  float* partials;
  // ENGRAM_FLAG_FP8_PROJ: E4M3 codes and scales of e and of W_KV
  uint8_t* e8;
  float* se;
  uint8_t* w8;
  float* sw;
};

// By default e is gathered into memory and the projection reads it as a dense
// matrix.  With ENGRAM_FLAG_FUSED_GATHER the projection reads the table rows
// directly (row gather fused into its B operand) unless the caller asks for e
// or the shape is outside what the fused loads handle.
bool fused_gather(const Shape& s, const engram_saved* sv) {
  if (!(s.flags & ENGRAM_FLAG_FUSED_GATHER) || (s.flags & ENGRAM_FLAG_FP8_PROJ)) return false;
  if (sv && sv->e) return false;
  GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  ga.F = (s.M + 1) * s.d;
  ga.K = s.d_mem;
  ga.group_m = 1;
  ga.stage_bytes = kFwdStageBytes;
  ga.J = s.J;
  ga.D = s.D;
  return gemm_supported(s.dtype == ENGRAM_BF16 ? GEMM_BF16 : GEMM_F32, ga, true);
}

size_t forward_ws(const Shape& s, int64_t N, const engram_saved* sv, FwdWs* out, uint8_t* base,
                  bool worst_case = false) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> uint8_t* {
    uint8_t* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  FwdWs w{};
  w.idx = (sv && sv->idx) ? sv->idx : (int32_t*)take((size_t)N * s.J * 4);
  const bool fp8 = (s.flags & ENGRAM_FLAG_FP8_PROJ) != 0;
  if (sv && sv->e)
    w.e = (uint8_t*)sv->e;
  else if (!fp8 && (worst_case || !fused_gather(s, sv)))
    w.e = take((size_t)N * s.d_mem * s.es);
  else
    w.e = nullptr;
  if (fp8) {  // E4M3 codes and scales of e (per token) and of W_KV (per row)
    const int64_t F = (int64_t)(s.M + 1) * s.d;
    w.e8 = take((size_t)N * s.d_mem);
    w.se = (float*)take((size_t)N * 4);
    w.w8 = take((size_t)F * s.d_mem);
    w.sw = (float*)take((size_t)F * 4);
  }
  w.v = (sv && sv->v) ? (uint8_t*)sv->v : take((size_t)N * s.d * s.es);
  w.partials = (float*)take((size_t)s.M * N * (s.d / kGemmBF) * 3 * 4);
  if (out) *out = w;
  return off;
}

struct BwdWs {
  float* scale;    // [N] bf16 io: power of two of each token's fp16 [dk | dv] row
  uint8_t* dkv;    // [round_up(N, 64)][2d]: the weight-gradient GEMM reads whole stages
  uint8_t* wt;
  float* de;
  uint8_t* sort;
  // parameter gradients
  uint8_t* e;      // [N][d_mem] dtype, rows gathered again (when e was not saved)
  float* dw_part;  // [splits][2d][d_mem] (splits > 1)
  float* pacc;     // [M][nblk][d][taps+1]
  float* ptmp;     // bwd_param_tmp_floats
  float* dv_acc;   // [N][d] fp32 with M > 1 branches
  int32_t splits;
};

int64_t round_pad(int64_t n) { return (n + kTnPadTokens - 1) / kTnPadTokens * kTnPadTokens; }

// table: de GEMM and scatter buffers; params: the parameter-gradient buffers
// (e only when need_e)
size_t backward_ws(const Shape& s, int64_t B, int64_t T, BwdWs* out, uint8_t* base,
                   bool table = true, bool params = false, bool need_e = true) {
  const int64_t N = B * T;
  const int eg = s.dtype == ENGRAM_BF16 ? 2 : 4;  // fp16 or fp32 GEMM operands
  size_t off = 0;
  auto take = [&](size_t bytes) -> uint8_t* {
    uint8_t* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  BwdWs w{};
  const int64_t cols = (int64_t)(s.M + 1) * s.d;  // [dk of each branch | dv]
  if (s.dtype == ENGRAM_BF16) w.scale = (float*)take((size_t)N * 4);
  w.dkv = take((size_t)round_pad(N) * cols * eg);
  if (s.M > 1) w.dv_acc = (float*)take((size_t)N * s.d * 4);
  if (table) {
    w.wt = take((size_t)s.d_mem * cols * eg);
    w.de = (float*)take((size_t)N * s.d_mem * 4);
    w.sort = take(sort_workspace_bytes(N, s.J));
  }
  if (params) {
    if (need_e) w.e = take((size_t)N * s.d_mem * s.es);
    w.splits = tn_splits(N, (int32_t)cols, s.d_mem);
    if (w.splits > 1) w.dw_part = (float*)take((size_t)w.splits * cols * s.d_mem * 4);
    const int64_t nb = std::max<int64_t>(1, bwd_blocks(B, T));
    w.pacc = (float*)take((size_t)s.M * nb * s.d * (s.taps + 1) * 4);
    w.ptmp = (float*)take(
        (size_t)std::max<int64_t>(1, bwd_param_tmp_floats(s.M * nb, s.d, s.taps)) * 4);
  }
  if (out) *out = w;
  return off;
}

// sharded exchange: sort buffers, send positions and the per-(table, owner) bounds
size_t shard_ws(const Shape& s, int64_t N, uint8_t* base, SortBufs* sb, int32_t** send_pos,
                int64_t** first, int64_t** dest_base) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> uint8_t* {
    uint8_t* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  uint8_t* sort = take(sort_workspace_bytes(N, s.J));
  uint8_t* sp = take((size_t)N * s.J * 4);
  uint8_t* fi = take(((size_t)s.J * ENGRAM_SHARD_MAX_GPUS + 1) * 8);
  uint8_t* db = take((size_t)s.J * ENGRAM_SHARD_MAX_GPUS * 8);
  if (base) {
    if (sb) carve_sort(sort, N, s.J, sb);
    if (send_pos) *send_pos = (int32_t*)sp;
    *first = (int64_t*)fi;
    *dest_base = (int64_t*)db;
  }
  return off;
}

// S_j = ceil(M_j / G); UNSUPPORTED when a shard needs 27 bits or more
engram_status shard_rows(const engram_config* cfg, const Shape& s, int32_t G, ShardRows* sr) {
  if (G < 1 || G > ENGRAM_SHARD_MAX_GPUS || s.J * G > 1024) return ENGRAM_E_INVALID;
  for (int j = 0; j < s.J; ++j) {
    sr->rows[j] = (cfg->table_rows[j] + G - 1) / G;
    if (sr->rows[j] >= (int64_t(1) << 27)) return ENGRAM_E_UNSUPPORTED;
  }
  return ENGRAM_OK;
}

}  // namespace

extern "C" {

size_t engram_workspace_size(const engram_config* cfg, int64_t B, int64_t T, int32_t op) {
  Shape s;
  if (check_config(cfg, &s) != ENGRAM_OK || B < 0 || T < 0) return 0;
  const int64_t N = B * T;
  if (op == ENGRAM_OP_FORWARD) return forward_ws(s, N, nullptr, nullptr, nullptr, true);
  if (op == ENGRAM_OP_BACKWARD) return backward_ws(s, B, T, nullptr, nullptr);
  if (op == ENGRAM_OP_BACKWARD_PARAMS) return backward_ws(s, B, T, nullptr, nullptr, true, true, true);
  if (op == ENGRAM_OP_SHARD) {
    int64_t* f = nullptr;
    int64_t* d = nullptr;
    return shard_ws(s, N, nullptr, nullptr, nullptr, &f, &d);
  }
  return 0;
}

const char* engram_status_string(engram_status st) {
  switch (st) {
    case ENGRAM_OK:
      return "ok";
    case ENGRAM_E_INVALID:
      return "invalid argument";
    case ENGRAM_E_UNSUPPORTED:
      return "unsupported shape or dtype";
    case ENGRAM_E_WORKSPACE:
      return "workspace missing or too small";
    case ENGRAM_E_HIP:
      return "HIP runtime or launch error";
    case ENGRAM_E_SCRATCH:
      return "input needs more than the fixed scratch of the allocation-free entry point";
  }
  return "unknown status";
}

engram_status engram_hash_indices(const engram_config* cfg, const int32_t* canon_map,
                                  const int32_t* tokens, int64_t B, int64_t T, int32_t* idx,
                                  void* stream) {
  Shape s;
  engram_status st = check_config(cfg, &s);
  if (st != ENGRAM_OK) return st;
  if (B < 0 || T < 0 || T > INT32_MAX) return ENGRAM_E_INVALID;
  if (B * T == 0) return ENGRAM_OK;
  if (!canon_map || !tokens || !idx) return ENGRAM_E_INVALID;
  hipStream_t hs = (hipStream_t)stream;
  HashArgs ha = make_hash_args(cfg, s);
  if ((st = id_check_begin(cfg, hs)) != ENGRAM_OK) return st;
  {
    Timed tm("hash", hs);
    if (launch_hash(tokens, canon_map, B * T, (int32_t)T, idx, ha, hs) != hipSuccess) return ENGRAM_E_HIP;
  }
  return id_check_end(cfg, hs);
}

// The forward of engram_forward; with noalloc (engram_forward_noalloc) the
// workspace is this device's fixed scratch array instead of the caller's.
static engram_status forward_impl(const engram_config* cfg, const engram_params* p,
                                  const int32_t* tokens, const void* hidden, int64_t B, int64_t T,
                                  void* y, const engram_saved* saved, const engram_compact* compact,
                                  void* workspace, size_t ws_bytes, void* stream, bool noalloc) {
  Shape s;
  engram_status st = check_config(cfg, &s);
  if (st != ENGRAM_OK) return st;
  if (!p || B < 0 || T < 0 || T > INT32_MAX || B > 65535) return ENGRAM_E_INVALID;
  const int64_t N = B * T;
  if (N == 0) return ENGRAM_OK;
  if ((uint64_t)N * (uint64_t)s.J >= (uint64_t(1) << 31)) return ENGRAM_E_UNSUPPORTED;
  // 16-byte pieces of e are numbered in 32 bits by the gather
  if ((uint64_t)N * (uint64_t)s.d_mem * (uint64_t)s.es / 16 >= (uint64_t(1) << 32) - 4096)
    return ENGRAM_E_UNSUPPORTED;
  if (!hidden || !y || !p->w_kv || !p->conv_w) return ENGRAM_E_INVALID;
  if (!aligned16(hidden) || !aligned16(y) || !aligned16(p->w_kv) || !aligned16(p->conv_w))
    return ENGRAM_E_INVALID;
  if ((p->gamma_q && !aligned16(p->gamma_q)) || (p->gamma_k && !aligned16(p->gamma_k)))
    return ENGRAM_E_INVALID;
  if (compact) {
    if (!compact->rows_dev || !compact->inverse_dev) return ENGRAM_E_INVALID;
    if (!aligned16(compact->rows_dev) || !aligned16(compact->inverse_dev)) return ENGRAM_E_INVALID;
  } else {
    if (!tokens || !p->canon_map) return ENGRAM_E_INVALID;
    for (int j = 0; j < s.J; ++j)
      if (!p->tables[j] || !aligned16(p->tables[j])) return ENGRAM_E_INVALID;
  }
  if (saved) {
    if ((saved->k && !aligned16(saved->k)) || (saved->v && !aligned16(saved->v)) ||
        (saved->e && !aligned16(saved->e)) || (saved->stats && !aligned16(saved->stats)) ||
        (saved->idx && !aligned16(saved->idx)))
      return ENGRAM_E_INVALID;
  }
  const size_t need = forward_ws(s, N, saved, nullptr, nullptr);
  QuietTiming quiet(noalloc);  // no timing events: they are allocations too
  if (noalloc) {
    if (need > kScratchBytes) return ENGRAM_E_SCRATCH;
    if ((st = scratch_ptr(&workspace)) != ENGRAM_OK) return st;
    ws_bytes = kScratchBytes;
  }
  if (need > 0 && (!workspace || ws_bytes < need || !aligned16(workspace))) return ENGRAM_E_WORKSPACE;
  FwdWs w;
  forward_ws(s, N, saved, &w, (uint8_t*)workspace);
  hipStream_t hs = (hipStream_t)stream;

  GatherArgs g;
  std::memset(&g, 0, sizeof(g));
  g.J = s.J;
  g.row_chunks = s.D * s.es / 16;
  const int32_t* idx = w.idx;
  if (compact) {
    if (compact->ready_event) {
      if (hipStreamWaitEvent(hs, (hipEvent_t)compact->ready_event, 0) != hipSuccess)
        return ENGRAM_E_HIP;
    }
    idx = compact->inverse_dev;
    for (int j = 0; j < s.J; ++j) g.base[j] = (const uint8_t*)compact->rows_dev;
    if (saved && saved->idx) {
      if (hipMemcpyAsync(saved->idx, compact->inverse_dev, (size_t)N * s.J * 4,
                         hipMemcpyDeviceToDevice, hs) != hipSuccess)
        return ENGRAM_E_HIP;
    }
  }
  const bool fp8 = (s.flags & ENGRAM_FLAG_FP8_PROJ) != 0;
  const bool fused = w.e == nullptr && !fp8;
  // Gathering bf16 e from the tables, one kernel hashes and gathers (the
  // indices go to memory only for the caller); the row-indexed projection,
  // the quantizing gather and the compact mode read indices from memory.
  const bool hash_in_gather = !compact && w.e && !fp8;
  if (!compact) {
    const HashArgs ha = make_hash_args(cfg, s);
    if ((st = id_check_begin(cfg, hs)) != ENGRAM_OK) return st;
    for (int j = 0; j < s.J; ++j) g.base[j] = (const uint8_t*)p->tables[j];
    if (hash_in_gather && (s.flags & ENGRAM_FLAG_GATHER_DEDUP)) {
      Timed tm("dedup_gather", hs);
      if (launch_dedup_gather(tokens, p->canon_map, N, (int32_t)T, ha, g, w.e,
                              saved && saved->idx ? saved->idx : nullptr, hs) != hipSuccess)
        return ENGRAM_E_HIP;
    } else if (hash_in_gather) {
      Timed tm("hash_gather", hs);
      if (launch_hash_gather(tokens, p->canon_map, N, (int32_t)T, ha, g, w.e,
                             saved && saved->idx ? saved->idx : nullptr, hs) != hipSuccess)
        return ENGRAM_E_HIP;
    } else {
      Timed tm("hash", hs);
      if (launch_hash(tokens, p->canon_map, N, (int32_t)T, w.idx, ha, hs) != hipSuccess)
        return ENGRAM_E_HIP;
    }
  }
  if (w.e && !hash_in_gather) {  // bf16 e: the projection's operand, or kept for the caller
    Timed tm("gather", hs);
    if (launch_gather(idx, w.e, N, g, hs) != hipSuccess) return ENGRAM_E_HIP;
  }
  if (fp8) {
    const int64_t F = (int64_t)(s.M + 1) * s.d;
    {
      Timed tm("quant_w", hs);
      if (launch_quant_rows((const uint8_t*)p->w_kv, s.dtype, F, s.d_mem, w.w8, w.sw, hs) != hipSuccess)
        return ENGRAM_E_HIP;
    }
    Timed tm("gather_quant", hs);
    if (launch_gather_quant(idx, N, g, s.d_mem, w.e8, w.se, hs) != hipSuccess) return ENGRAM_E_HIP;
  }
  // compact mode: the plan's device buffers are read for the last time by
  // the gather (or, fused, by the projection below)
  auto consumed = [&]() -> bool {
    return !compact || !compact->consumed_event ||
           hipEventRecord((hipEvent_t)compact->consumed_event, hs) == hipSuccess;
  };
  if (!fused && !consumed()) return ENGRAM_E_HIP;
  {
    GemmArgs ga;
    std::memset(&ga, 0, sizeof(ga));
    ga.A = fp8 ? w.w8 : (const uint8_t*)p->w_kv;
    ga.B = fp8 ? w.e8 : w.e;
    ga.scale_a = w.sw;
    ga.scale_b = w.se;
    if (fused) {
      ga.idx = idx;
      ga.J = s.J;
      ga.D = s.D;
      for (int j = 0; j < s.J; ++j) ga.tables[j] = g.base[j];
    }
    ga.M = N;
    ga.F = (s.M + 1) * s.d;
    ga.K = s.d_mem;
    ga.group_m = 4;
    // last token tiles first: the gather wrote them last, so more of their e
    // rows are still in the Infinity Cache (measured ~1 % faster)
    ga.reverse_m = 1;
    ga.persistent = ENGRAM_GEMM_PERSISTENT;
    // E4M3 uses the same 128-byte stages (two 64-element K steps each): the
    // four-deep ring of 64-byte stages measured 1-2 % slower, with 8x the LDS
    // bank conflicts of the two-piece fragment reads
    ga.stage_bytes = kFwdStageBytes;
    ga.d = s.d;
    ga.branches = s.M;
    ga.io_dtype = s.dtype;
    ga.h = (const uint8_t*)hidden;
    ga.gamma_q = p->gamma_q;
    ga.gamma_k = p->gamma_k;
    ga.partials = w.partials;
    ga.k_out = saved ? (uint8_t*)saved->k : nullptr;
    ga.v_out = w.v;
    {
      Timed tm(fused ? "gather_proj_gemm" : (fp8 ? "proj_gemm_fp8" : "proj_gemm"), hs);
      const GemmType gt = fp8 ? GEMM_FP8 : (s.dtype == ENGRAM_BF16 ? GEMM_BF16 : GEMM_F32);
      if (launch_gemm(gt, EPI_KV, ga, hs) != hipSuccess) return ENGRAM_E_HIP;
    }
    if (fused && !consumed()) return ENGRAM_E_HIP;
  }
  {
    GateConvArgs gc;
    gc.B = B;
    gc.T = T;
    gc.d = s.d;
    gc.taps = s.taps;
    gc.nkt = s.d / kGemmBF;
    gc.branches = s.M;
    gc.io_dtype = s.dtype;
    gc.eps = cfg->rms_eps;
    gc.partials = w.partials;
    gc.v = w.v;
    gc.conv_w = p->conv_w;
    gc.y = (uint8_t*)y;
    gc.stats = saved ? saved->stats : nullptr;
    Timed tm("gate_conv", hs);
    if (launch_gate_conv(gc, hs) != hipSuccess) return ENGRAM_E_HIP;
  }
  return compact ? ENGRAM_OK : id_check_end(cfg, hs);
}

engram_status engram_forward(const engram_config* cfg, const engram_params* p,
                             const int32_t* tokens, const void* hidden, int64_t B, int64_t T,
                             void* y, const engram_saved* saved, const engram_compact* compact,
                             void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(cfg, p, tokens, hidden, B, T, y, saved, compact, workspace, ws_bytes, stream,
                      false);
}

engram_status engram_forward_noalloc(const engram_config* cfg, const engram_params* p,
                                     const int32_t* tokens, const void* hidden, int64_t B, int64_t T,
                                     void* y, const engram_saved* saved,
                                     const engram_compact* compact, void* stream) {
  return forward_impl(cfg, p, tokens, hidden, B, T, y, saved, compact, nullptr, 0, stream, true);
}

engram_status engram_backward(const engram_config* cfg, const engram_params* p,
                              const void* hidden, const void* dy, int64_t B, int64_t T,
                              const engram_saved* saved, engram_table_grad* out,
                              engram_param_grad* pg, void* workspace, size_t ws_bytes,
                              void* stream) {
  Shape s;
  engram_status st = check_config(cfg, &s);
  if (st != ENGRAM_OK) return st;
  if (!p || (!out && !pg) || B < 0 || T < 0 || T > INT32_MAX || B > 65535) return ENGRAM_E_INVALID;
  if (s.d / 4 > 1024) return ENGRAM_E_UNSUPPORTED;
  if (s.D > 256) return ENGRAM_E_UNSUPPORTED;  // one 16-byte piece per lane of a row
  const int64_t N = B * T;
  if ((uint64_t)N * (uint64_t)s.J >= (uint64_t(1) << 31)) return ENGRAM_E_UNSUPPORTED;
  if (out) {
    if (out->mode < ENGRAM_GRAD_SORTED_SPARSE || out->mode > ENGRAM_GRAD_ATOMIC_DENSE)
      return ENGRAM_E_INVALID;
    if (out->mode == ENGRAM_GRAD_SORTED_SPARSE) {
      if (!out->keys || !out->rows || !out->count || !aligned16(out->rows)) return ENGRAM_E_INVALID;
    } else {
      for (int j = 0; j < s.J; ++j)
        if (!out->dense[j] || !aligned16(out->dense[j])) return ENGRAM_E_INVALID;
    }
  }
  const bool want_w = pg && pg->w_kv;
  const bool want_sums = pg && (pg->conv_w || pg->gamma_q || pg->gamma_k);
  const bool bf = s.dtype == ENGRAM_BF16;
  // dW reads e: gathered again unless saved; with bf16 io each row divided by
  // its token's scale, into the workspace either way
  const bool regather = want_w && !(saved && saved->e);
  const bool need_e = want_w && (regather || bf);
  if (pg) {
    if (s.d_mem % 256 != 0) return ENGRAM_E_UNSUPPORTED;  // whole 256-wide dW tiles
    if (pg->hidden && !aligned16(pg->hidden)) return ENGRAM_E_INVALID;
    if (want_w && !aligned16(pg->w_kv)) return ENGRAM_E_INVALID;
  }
  if (N > 0) {
    if (!hidden || !dy || !saved || !saved->idx || !saved->stats || !saved->k || !saved->v)
      return ENGRAM_E_INVALID;
    if (!p->w_kv || !p->conv_w) return ENGRAM_E_INVALID;
    if (!aligned16(hidden) || !aligned16(dy) || !aligned16(saved->k) || !aligned16(saved->v) ||
        !aligned16(saved->stats) || !aligned16(p->w_kv))
      return ENGRAM_E_INVALID;
    if (want_w && saved->e && !aligned16(saved->e)) return ENGRAM_E_INVALID;
    if (regather)
      for (int j = 0; j < s.J; ++j)
        if (!p->tables[j] || !aligned16(p->tables[j])) return ENGRAM_E_INVALID;
  }
  const size_t need = backward_ws(s, B, T, nullptr, nullptr, out != nullptr, pg != nullptr, need_e);
  if (!workspace || ws_bytes < need || !aligned16(workspace)) return ENGRAM_E_WORKSPACE;
  BwdWs w;
  backward_ws(s, B, T, &w, (uint8_t*)workspace, out != nullptr, pg != nullptr, need_e);
  hipStream_t hs = (hipStream_t)stream;

  const int64_t nblk = bwd_blocks(B, T);
  if (bf && N > 0) {
    BwdScaleArgs sa;
    sa.B = B;
    sa.T = T;
    sa.d = s.d;
    sa.taps = s.taps;
    sa.branches = s.M;
    sa.dy = (const uint8_t*)dy;
    sa.v = (const uint8_t*)saved->v;
    sa.stats = saved->stats;
    sa.conv_w = p->conv_w;
    sa.gamma_q = p->gamma_q;
    sa.gamma_k = p->gamma_k;
    sa.scale = w.scale;
    Timed tm("bwd_scale", hs);
    if (launch_bwd_scale(sa, hs) != hipSuccess) return ENGRAM_E_HIP;
  }
  const int64_t cols = (int64_t)(s.M + 1) * s.d;
  const size_t act = (size_t)N * s.d * s.es;  // bytes of one branch's [N][d] activations
  // one launch per branch; the shared v's gradient gathers over them
  for (int m = 0; m < s.M && N > 0; ++m) {
    BwdArgs ba;
    std::memset(&ba, 0, sizeof(ba));
    ba.B = B;
    ba.T = T;
    ba.d = s.d;
    ba.taps = s.taps;
    ba.io_dtype = s.dtype;
    ba.dy = (const uint8_t*)dy + m * act;
    ba.v = (const uint8_t*)saved->v;
    ba.k = (const uint8_t*)saved->k + m * act;
    ba.h = (const uint8_t*)hidden + m * act;
    ba.stats = saved->stats + (size_t)m * N * 4;
    ba.conv_w = p->conv_w;
    ba.gamma_q = p->gamma_q ? p->gamma_q + (size_t)m * s.d : nullptr;
    ba.gamma_k = p->gamma_k ? p->gamma_k + (size_t)m * s.d : nullptr;
    ba.dkv = w.dkv;
    ba.branches = s.M;
    ba.branch = m;
    ba.dv_acc = w.dv_acc;
    ba.dv_mode = s.M == 1 ? 0 : (m == 0 ? 1 : (m + 1 < s.M ? 2 : 3));
    ba.scale = w.scale;
    if (pg) {
      ba.pacc = want_sums ? w.pacc + (size_t)m * nblk * s.d * (s.taps + 1) : nullptr;
      ba.dh = pg->hidden ? (uint8_t*)pg->hidden + m * act : nullptr;
      ba.pad_rows = want_w && m == 0 ? (int32_t)(round_pad(N) - N) : 0;
    }
    Timed tm(pg ? "bwd_gate_conv_params" : "bwd_gate_conv", hs);
    if (launch_bwd_gate_conv(ba, hs) != hipSuccess) return ENGRAM_E_HIP;
  }
  if (out && N > 0) {
    {
      Timed tm("transpose_w", hs);
      if (launch_transpose_w((const uint8_t*)p->w_kv, w.wt, (int32_t)cols, s.d_mem, s.dtype, hs) !=
          hipSuccess)
        return ENGRAM_E_HIP;
    }
    GemmArgs ga;
    std::memset(&ga, 0, sizeof(ga));
    ga.A = w.wt;
    ga.B = w.dkv;
    ga.M = N;
    ga.F = s.d_mem;
    ga.K = (int32_t)cols;
    ga.group_m = ENGRAM_DE_GROUP_M;
    ga.stage_bytes = kBwdStageBytes;
    ga.persistent = ENGRAM_GEMM_PERSISTENT;
    ga.c_out = w.de;
    ga.col_scale = w.scale;
    Timed tm("de_gemm", hs);
    if (launch_gemm(bf ? GEMM_F16 : GEMM_F32, EPI_STORE_F32, ga, hs) != hipSuccess)
      return ENGRAM_E_HIP;
  }
  if (pg) {
    if (want_sums) {
      if (N > 0) {
        Timed tm("bwd_param_sums", hs);
        if (s.M == 1) {
          if (launch_bwd_param_sums(w.pacc, w.ptmp, nblk, s.d, s.taps, p->gamma_q, p->gamma_k,
                                    pg->conv_w, pg->gamma_q, pg->gamma_k, hs) != hipSuccess)
            return ENGRAM_E_HIP;
        } else {
          // the conv is shared: its sums run over every branch's blocks; the
          // RMSNorm scales are per branch
          if (pg->conv_w && launch_bwd_param_sums(w.pacc, w.ptmp, s.M * nblk, s.d, s.taps, nullptr,
                                                  nullptr, pg->conv_w, nullptr, nullptr,
                                                  hs) != hipSuccess)
            return ENGRAM_E_HIP;
          for (int m = 0; m < s.M && (pg->gamma_q || pg->gamma_k); ++m) {
            const size_t o = (size_t)m * s.d;
            if (launch_bwd_param_sums(w.pacc + (size_t)m * nblk * s.d * (s.taps + 1), w.ptmp, nblk,
                                      s.d, s.taps, p->gamma_q ? p->gamma_q + o : nullptr,
                                      p->gamma_k ? p->gamma_k + o : nullptr, nullptr,
                                      pg->gamma_q ? pg->gamma_q + o : nullptr,
                                      pg->gamma_k ? pg->gamma_k + o : nullptr, hs) != hipSuccess)
              return ENGRAM_E_HIP;
          }
        }
      } else {
        // no tokens: the sums are zero
        if (pg->conv_w && launch_zero_f32(pg->conv_w, (int64_t)s.d * s.taps, hs) != hipSuccess)
          return ENGRAM_E_HIP;
        if (pg->gamma_q && launch_zero_f32(pg->gamma_q, (int64_t)s.M * s.d, hs) != hipSuccess)
          return ENGRAM_E_HIP;
        if (pg->gamma_k && launch_zero_f32(pg->gamma_k, (int64_t)s.M * s.d, hs) != hipSuccess)
          return ENGRAM_E_HIP;
      }
    }
    if (want_w) {
      const uint8_t* e = need_e ? w.e : (const uint8_t*)(saved ? saved->e : nullptr);
      if (need_e && !regather && N > 0) {
        Timed tm("scale_rows", hs);
        if (launch_scale_rows_bf16((const uint8_t*)saved->e, w.scale, N, s.d_mem, w.e, hs) != hipSuccess)
          return ENGRAM_E_HIP;
      }
      if (regather && N > 0) {
        GatherArgs g;
        std::memset(&g, 0, sizeof(g));
        g.J = s.J;
        g.row_chunks = s.D * s.es / 16;
        for (int j = 0; j < s.J; ++j) g.base[j] = (const uint8_t*)p->tables[j];
        g.row_scale = w.scale;  // bf16: e_t / s_t; fp32: null
        Timed tm("gather", hs);
        if (launch_gather(saved->idx, w.e, N, g, hs) != hipSuccess) return ENGRAM_E_HIP;
      }
      if (N == 0) {
        if (launch_zero_f32(pg->w_kv, cols * s.d_mem, hs) != hipSuccess)
          return ENGRAM_E_HIP;
      } else {
        GemmTnArgs ta;
        std::memset(&ta, 0, sizeof(ta));
        ta.x = w.dkv;
        ta.y = e;
        ta.ldx = cols;
        ta.ldy = s.d_mem;
        ta.K = N;
        ta.m = (int32_t)cols;
        ta.n = s.d_mem;
        ta.splits = w.splits;
        ta.kchunk = ((N + kTnPadTokens - 1) / kTnPadTokens + w.splits - 1) / w.splits * kTnPadTokens;
        ta.out = w.dw_part;
        Timed tm("dw_gemm", hs);
        if (launch_gemm_tn(bf ? GEMM_F16 : GEMM_F32, ta, pg->w_kv, hs) != hipSuccess)
          return ENGRAM_E_HIP;
      }
    }
  }
  if (!out) return ENGRAM_OK;
  ScatterArgs sa;
  std::memset(&sa, 0, sizeof(sa));
  sa.N = N;
  sa.J = s.J;
  sa.D = s.D;
  sa.idx = saved ? saved->idx : nullptr;
  sa.de = w.de;
  sa.key_bits = s.key_bits;
  for (int j = 0; j < s.J; ++j) sa.dense[j] = out->dense[j];
  sa.keys_out = out->keys;
  sa.rows_out = out->rows;
  sa.count_out = out->count;
  if (out->mode == ENGRAM_GRAD_ATOMIC_DENSE) {
    Timed tm("atomic_scatter", hs);
    return hip_status(launch_atomic_scatter(sa, hs));
  }
  SortBufs sb;
  carve_sort(w.sort, N, s.J, &sb);
  Timed tm("sorted_scatter", hs);
  return hip_status(launch_sorted_scatter(sa, sb, out->mode, hs));
}

engram_status engram_backward_table_grad(const engram_config* cfg, const engram_params* p,
                                         const void* hidden, const void* dy, int64_t B, int64_t T,
                                         const engram_saved* saved, engram_table_grad* out,
                                         void* workspace, size_t ws_bytes, void* stream) {
  if (!out) return ENGRAM_E_INVALID;
  return engram_backward(cfg, p, hidden, dy, B, T, saved, out, nullptr, workspace, ws_bytes, stream);
}

engram_status engram_prefetch_plan(const engram_config* cfg, const int32_t* canon_map_host,
                                   const int32_t* tokens_host, int64_t B, int64_t T,
                                   const void* const* host_tables, engram_compact* plan,
                                   void* side_stream) {
  Shape s;
  engram_status st = check_config(cfg, &s);
  if (st != ENGRAM_OK) return st;
  if (!plan || B < 0 || T < 0) return ENGRAM_E_INVALID;
  const int64_t N = B * T;
  const int J = s.J;
  if (N > 0 && (!canon_map_host || !tokens_host)) return ENGRAM_E_INVALID;
  if (!plan->counts || !plan->uniq_host || !plan->inverse_host) return ENGRAM_E_INVALID;
  if (plan->capacity_rows < 0) return ENGRAM_E_INVALID;
  if (plan->flags & ~(uint32_t)ENGRAM_PLAN_REUSE) return ENGRAM_E_INVALID;
  const bool reuse = (plan->flags & ENGRAM_PLAN_REUSE) != 0;
  if (reuse && (plan->total_rows < 0 || plan->total_rows > plan->capacity_rows))
    return ENGRAM_E_INVALID;
  if (host_tables) {
    if (!plan->staging_host || !plan->rows_dev || !plan->inverse_dev) return ENGRAM_E_INVALID;
    for (int j = 0; j < J; ++j)
      if (!host_tables[j]) return ENGRAM_E_INVALID;
  }
  const bool ring = plan->ring_rows != 0;
  if (ring && (plan->ring_rows < 2 * plan->capacity_rows || plan->ring_rows < 1 ||
               plan->ring_rows >= (int64_t(1) << 31) || !plan->ring_pos || plan->ring_head < 0))
    return ENGRAM_E_INVALID;
  if (!reuse)
    for (int64_t n = 0; n < N; ++n)
      if (tokens_host[n] < 0 || tokens_host[n] >= cfg->vocab) return ENGRAM_E_INVALID;
  // the previous copies of this plan read inverse_host and staging_host until
  // its event fires: wait before rewriting them
  if (plan->ready_event && hipEventSynchronize((hipEvent_t)plan->ready_event) != hipSuccess)
    return ENGRAM_E_HIP;
  const HashArgs ha = make_hash_args(cfg, s);
  const int nthr = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  auto parallel = [&](int64_t count, auto&& fn) {
    const int64_t per = (count + nthr - 1) / nthr;
    std::vector<std::thread> th;
    for (int t = 0; t < nthr; ++t) {
      const int64_t lo = t * per, hi = std::min(count, lo + per);
      if (lo >= hi) break;
      th.emplace_back([&, lo, hi] { fn(lo, hi); });
    }
    for (auto& x : th) x.join();
  };

  std::vector<int64_t> base(J + 1, 0);
  if (reuse) {
    for (int j = 0; j < J; ++j) {
      if (plan->counts[j] < 0) return ENGRAM_E_INVALID;
      base[j + 1] = base[j] + plan->counts[j];
    }
    if (base[J] != plan->total_rows) return ENGRAM_E_INVALID;
    for (int j = 0; j < J; ++j)  // the rows must lie inside their tables
      for (int64_t u = base[j]; u < base[j + 1]; ++u)
        if (plan->uniq_host[u] < 0 || plan->uniq_host[u] >= cfg->table_rows[j])
          return ENGRAM_E_INVALID;
  } else {
  // 1. indices on the host, same hash as the device kernel
  std::vector<int32_t> idx((size_t)N * J);
  parallel(N, [&](int64_t lo, int64_t hi) {
    for (int64_t n = lo; n < hi; ++n) {
      const int64_t t = n % T;
      uint32_t c[ENGRAM_MAX_ORDERS] = {0, 0, 0, 0};
      for (int i = 0; i < s.max_order; ++i)
        c[i] = (t - i >= 0) ? (uint32_t)canon_map_host[tokens_host[n - i]] : (uint32_t)cfg->pad_id;
      int j = 0;
      for (int o = 0; o < cfg->num_orders; ++o)
        for (int k = 0; k < cfg->heads; ++k, ++j)
          idx[(size_t)n * J + j] = (int32_t)hash_one(ha, j, cfg->orders[o], c);
    }
  });
  // 2. distinct rows of every table, ascending
  std::vector<std::vector<int32_t>> uniq(J);
  parallel(J, [&](int64_t lo, int64_t hi) {
    for (int64_t j = lo; j < hi; ++j) {
      std::vector<int32_t>& u = uniq[j];
      u.resize((size_t)N);
      for (int64_t n = 0; n < N; ++n) u[n] = idx[(size_t)n * J + j];
      std::sort(u.begin(), u.end());
      u.erase(std::unique(u.begin(), u.end()), u.end());
    }
  });
  for (int j = 0; j < J; ++j) base[j + 1] = base[j] + (int64_t)uniq[j].size();
  const int64_t total = base[J];
  if (total > plan->capacity_rows) return ENGRAM_E_INVALID;
  for (int j = 0; j < J; ++j) {
    plan->counts[j] = (int64_t)uniq[j].size();
    if (!uniq[j].empty())
      std::memcpy(plan->uniq_host + base[j], uniq[j].data(), uniq[j].size() * sizeof(int32_t));
  }
  plan->total_rows = total;
  // 3. inverse map into the compact buffer
  parallel(N, [&](int64_t lo, int64_t hi) {
    for (int64_t n = lo; n < hi; ++n)
      for (int j = 0; j < J; ++j) {
        const int32_t key = idx[(size_t)n * J + j];
        const auto it = std::lower_bound(uniq[j].begin(), uniq[j].end(), key);
        plan->inverse_host[(size_t)n * J + j] = (int32_t)(base[j] + (it - uniq[j].begin()));
      }
  });
  // 4. with the ring: rows an earlier call left in the ring are not copied
  //    again.  The inverse map gets its final ring rows, the misses get ring
  //    positions from ring_head on, and the plan keeps the misses only
  //    (counts, uniq_host, total_rows), so the copying call moves just those.
  if (ring) {
    // A row in the ring is usable when neither this call's appends nor the
    // next call's (each at most capacity_rows) reach its slot.
    const int64_t R = plan->ring_rows, head = plan->ring_head;
    const int64_t oldest = head + 2 * plan->capacity_rows - R;
    std::vector<int64_t> toff(J + 1, 0);
    for (int j = 0; j < J; ++j) toff[j + 1] = toff[j] + cfg->table_rows[j];
    std::vector<int32_t> dev((size_t)total);   // ring row of each distinct row
    std::vector<uint8_t> hit((size_t)total);
    std::vector<int64_t> miss_base(J + 1, 0);
    // ring_pos is read at ascending but scattered rows (one cache line
    // each), so both sweeps prefetch kPf rows ahead to keep many in flight
    constexpr int64_t kPf = 32;
    parallel(J, [&](int64_t lo, int64_t hi) {
      for (int64_t j = lo; j < hi; ++j) {
        const int64_t* rp = plan->ring_pos + toff[j];
        const int32_t* uj = uniq[j].data();
        const int64_t n = (int64_t)uniq[j].size();
        for (int64_t i = 0; i < n; ++i) {
          if (i + kPf < n) __builtin_prefetch(rp + uj[i + kPf], 1);
          const int64_t P = rp[uj[i]];
          const bool h = P >= 0 && P >= oldest && P < head;
          hit[base[j] + i] = h;
          if (h) dev[base[j] + i] = (int32_t)(P % R);
        }
      }
    });
    for (int j = 0; j < J; ++j) {
      int64_t m = 0;
      for (int64_t u = base[j]; u < base[j + 1]; ++u) m += !hit[u];
      miss_base[j + 1] = miss_base[j] + m;
    }
    parallel(J, [&](int64_t lo, int64_t hi) {
      for (int64_t j = lo; j < hi; ++j) {
        int64_t* rp = plan->ring_pos + toff[j];
        const int32_t* uj = uniq[j].data();
        const int64_t n = (int64_t)uniq[j].size();
        int64_t m = miss_base[j];
        for (int64_t i = 0; i < n; ++i) {
          if (i + kPf < n) __builtin_prefetch(rp + uj[i + kPf], 1);
          if (hit[base[j] + i]) continue;
          const int64_t P = head + m;
          rp[uj[i]] = P;
          dev[base[j] + i] = (int32_t)(P % R);
          plan->uniq_host[m++] = uj[i];  // misses only, table after table
        }
        plan->counts[j] = miss_base[j + 1] - miss_base[j];
      }
    });
    parallel(N, [&](int64_t lo, int64_t hi) {
      for (int64_t n = lo; n < hi; ++n)
        for (int j = 0; j < J; ++j) {
          int32_t& x = plan->inverse_host[(size_t)n * J + j];
          x = dev[(size_t)x];
        }
    });
    plan->total_rows = miss_base[J];
    plan->ring_head = head + miss_base[J];
    plan->ring_hits = total - miss_base[J];
    for (int j = 0; j <= J; ++j) base[j] = miss_base[j];
  }
  }  // !reuse
  if (!host_tables) return ENGRAM_OK;
  // Rows to copy: the plan's rows; with the ring they are the misses and go
  // to the ring positions the planning reserved, ending at ring_head.
  const int64_t ncopy = plan->total_rows;
  const int64_t dst0 = ring ? plan->ring_head - ncopy : 0;
  if (ring && dst0 < 0) return ENGRAM_E_INVALID;
  // 4. the inverse map first, then the rows chunk by chunk: gather a chunk
  //    into pinned staging on the host threads, queue its copy, gather the next
  hipStream_t hs = (hipStream_t)side_stream;
  // the forward on the previous plan may still be about to read the device
  // buffers these copies rewrite
  if (plan->consumed_event && hipStreamWaitEvent(hs, (hipEvent_t)plan->consumed_event, 0) != hipSuccess)
    return ENGRAM_E_HIP;
  if (N > 0 && hipMemcpyAsync(plan->inverse_dev, plan->inverse_host, (size_t)N * J * 4,
                              hipMemcpyHostToDevice, hs) != hipSuccess)
    return ENGRAM_E_HIP;
  const size_t rb = (size_t)s.D * s.es;
  const int64_t chunk = std::max<int64_t>(1, (int64_t)((32u << 20) / rb));  // ~32 MB of rows
  // staged rows [a, b) to ring (or buffer) rows from dst0 + a, split at the ring's end
  auto copy_rows = [&](int64_t a, int64_t b) -> bool {
    while (a < b) {
      int64_t d = dst0 + a, n = b - a;
      if (ring) {
        d %= plan->ring_rows;
        n = std::min(n, plan->ring_rows - d);
      }
      if (hipMemcpyAsync((uint8_t*)plan->rows_dev + (size_t)d * rb,
                         (const uint8_t*)plan->staging_host + (size_t)a * rb, (size_t)n * rb,
                         hipMemcpyHostToDevice, hs) != hipSuccess)
        return false;
      a += n;
    }
    return true;
  };
  for (int64_t c0 = 0; c0 < ncopy; c0 += chunk) {
    const int64_t c1 = std::min(ncopy, c0 + chunk);
    parallel(c1 - c0, [&](int64_t lo, int64_t hi) {
      lo += c0;
      hi += c0;
      int j = (int)(std::upper_bound(base.begin(), base.end(), lo) - base.begin()) - 1;
      for (int64_t u = lo; u < hi; ++u) {
        while (u >= base[j + 1]) ++j;
        const int32_t row = plan->uniq_host[u];
        std::memcpy((uint8_t*)plan->staging_host + (size_t)u * rb,
                    (const uint8_t*)host_tables[j] + (size_t)row * rb, rb);
      }
    });
    if (!copy_rows(c0, c1)) return ENGRAM_E_HIP;
  }
  if (plan->ready_event && hipEventRecord((hipEvent_t)plan->ready_event, hs) != hipSuccess)
    return ENGRAM_E_HIP;
  return ENGRAM_OK;
}

engram_status engram_quantize_fp8(const void* src, int32_t dtype, int64_t rows, int32_t cols,
                                  uint8_t* codes, float* scales, void* stream) {
  if (dtype != ENGRAM_BF16 && dtype != ENGRAM_F32) return ENGRAM_E_UNSUPPORTED;
  if (rows < 0 || cols <= 0 || cols % 8 != 0) return ENGRAM_E_INVALID;
  if (rows == 0) return ENGRAM_OK;
  if (!src || !codes || !scales || !aligned16(src) || ((uintptr_t)codes & 7)) return ENGRAM_E_INVALID;
  hipStream_t hs = (hipStream_t)stream;
  Timed tm("quant_rows", hs);
  return hip_status(launch_quant_rows((const uint8_t*)src, dtype, rows, cols, codes, scales, hs));
}

engram_status engram_shard_requests(const engram_config* cfg, int32_t G, const int32_t* idx,
                                    int64_t N, uint32_t* send_ids, int64_t* send_counts,
                                    int32_t* inverse, void* workspace, size_t ws_bytes,
                                    void* stream) {
  Shape s;
  engram_status st = check_config(cfg, &s);
  if (st != ENGRAM_OK) return st;
  ShardRows sr;
  if ((st = shard_rows(cfg, s, G, &sr)) != ENGRAM_OK) return st;
  if (N < 0 || (uint64_t)N * (uint64_t)s.J >= (uint64_t(1) << 31)) return ENGRAM_E_INVALID;
  if (!send_counts || (N > 0 && (!idx || !send_ids || !inverse))) return ENGRAM_E_INVALID;
  const size_t need = shard_ws(s, N, nullptr, nullptr, nullptr, nullptr, nullptr);
  if (!workspace || ws_bytes < need || !aligned16(workspace)) return ENGRAM_E_WORKSPACE;
  SortBufs sb;
  ShardPackArgs pa;
  std::memset(&pa, 0, sizeof(pa));
  shard_ws(s, N, (uint8_t*)workspace, &sb, &pa.send_pos, &pa.first, &pa.dest_base);
  hipStream_t hs = (hipStream_t)stream;
  {
    Timed tm("shard_dedup", hs);
    if (launch_dedup(idx, N, s.J, s.key_bits, sb, inverse, hs) != hipSuccess) return ENGRAM_E_HIP;
  }
  pa.keys = sb.seg_key;
  pa.count_u32 = sb.total;
  pa.capacity = N * s.J;
  pa.J = s.J;
  pa.G = G;
  pa.shard_rows = sr;
  pa.send_counts = send_counts;
  pa.send_ids = send_ids;
  pa.inverse = inverse;
  pa.n_inverse = N * s.J;
  Timed tm("shard_pack", hs);
  return hip_status(launch_shard_pack(pa, hs));
}

engram_status engram_shard_serve(const engram_config* cfg, int32_t G,
                                 const void* const* shard_tables, const uint32_t* ids, int64_t n,
                                 void* rows_out, void* stream) {
  Shape s;
  engram_status st = check_config(cfg, &s);
  if (st != ENGRAM_OK) return st;
  ShardRows sr;
  if ((st = shard_rows(cfg, s, G, &sr)) != ENGRAM_OK) return st;
  if (n < 0 || !shard_tables) return ENGRAM_E_INVALID;
  if (n == 0) return ENGRAM_OK;
  if (!ids || !rows_out || !aligned16(rows_out)) return ENGRAM_E_INVALID;
  ShardTables t;
  std::memset(&t, 0, sizeof(t));
  for (int j = 0; j < s.J; ++j) {
    if (!shard_tables[j] || !aligned16(shard_tables[j])) return ENGRAM_E_INVALID;
    t.base[j] = (const uint8_t*)shard_tables[j];
  }
  hipStream_t hs = (hipStream_t)stream;
  Timed tm("shard_serve", hs);
  return hip_status(launch_shard_serve(t, ids, n, (uint8_t*)rows_out, s.D * s.es, hs));
}

engram_status engram_shard_grads(const engram_config* cfg, int32_t G, const int64_t* keys,
                                 const float* rows, const int64_t* count, int64_t capacity,
                                 uint32_t* send_ids, float* send_rows, int64_t* send_counts,
                                 void* workspace, size_t ws_bytes, void* stream) {
  Shape s;
  engram_status st = check_config(cfg, &s);
  if (st != ENGRAM_OK) return st;
  ShardRows sr;
  if ((st = shard_rows(cfg, s, G, &sr)) != ENGRAM_OK) return st;
  if (capacity < 0 || capacity >= (int64_t(1) << 31) || !count || !send_counts)
    return ENGRAM_E_INVALID;
  if (capacity > 0 && (!keys || !rows || !send_ids || !send_rows || !aligned16(rows) ||
                       !aligned16(send_rows)))
    return ENGRAM_E_INVALID;
  const size_t need = shard_ws(s, 1, nullptr, nullptr, nullptr, nullptr, nullptr);
  if (!workspace || ws_bytes < need || !aligned16(workspace)) return ENGRAM_E_WORKSPACE;
  ShardPackArgs pa;
  std::memset(&pa, 0, sizeof(pa));
  shard_ws(s, 1, (uint8_t*)workspace, nullptr, nullptr, &pa.first, &pa.dest_base);
  pa.keys = (const uint64_t*)keys;
  pa.count_i64 = count;
  pa.capacity = capacity;
  pa.J = s.J;
  pa.G = G;
  pa.shard_rows = sr;
  pa.send_counts = send_counts;
  pa.send_ids = send_ids;
  pa.rows = rows;
  pa.send_rows = send_rows;
  pa.pieces = s.D / 4;
  hipStream_t hs = (hipStream_t)stream;
  Timed tm("shard_grad_pack", hs);
  return hip_status(launch_shard_pack(pa, hs));
}

engram_status engram_shard_reduce(const engram_config* cfg, int32_t G, float* const* shard_grads,
                                  const uint32_t* ids, const float* rows,
                                  const int64_t* counts_host, int32_t nblocks, void* stream) {
  Shape s;
  engram_status st = check_config(cfg, &s);
  if (st != ENGRAM_OK) return st;
  ShardRows sr;
  if ((st = shard_rows(cfg, s, G, &sr)) != ENGRAM_OK) return st;
  if (nblocks < 0 || (nblocks > 0 && !counts_host) || !shard_grads) return ENGRAM_E_INVALID;
  int64_t total = 0;
  for (int b = 0; b < nblocks; ++b) {
    if (counts_host[b] < 0) return ENGRAM_E_INVALID;
    total += counts_host[b];
  }
  if (total == 0) return ENGRAM_OK;
  if (!ids || !rows || !aligned16(rows)) return ENGRAM_E_INVALID;
  ShardGrads g;
  std::memset(&g, 0, sizeof(g));
  for (int j = 0; j < s.J; ++j) {
    if (!shard_grads[j] || !aligned16(shard_grads[j])) return ENGRAM_E_INVALID;
    g.base[j] = shard_grads[j];
  }
  hipStream_t hs = (hipStream_t)stream;
  Timed tm("shard_reduce", hs);
  int64_t off = 0;
  for (int b = 0; b < nblocks; ++b) {
    if (launch_shard_grad_add(g, ids + off, rows + off * s.D, counts_host[b], s.D, hs) != hipSuccess)
      return ENGRAM_E_HIP;
    off += counts_host[b];
  }
  return ENGRAM_OK;
}

engram_status engram_device_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes % 16 != 0) return ENGRAM_E_INVALID;
  if (bytes == 0) return ENGRAM_OK;
  if (!dst || !src || !aligned16(dst) || !aligned16(src)) return ENGRAM_E_INVALID;
  hipStream_t hs = (hipStream_t)stream;
  Timed tm("device_copy", hs);
  return hip_status(launch_stream_copy(dst, src, bytes, hs));
}

void engram_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> l(g_prof_mu);
  g_prof_on = on != 0;
}

void engram_profile_reset(void) {
  std::lock_guard<std::mutex> l(g_prof_mu);
  for (auto& r : g_prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
}

int32_t engram_profile_read(char* names, size_t names_len, int64_t* launches, double* total_ms,
                            int32_t max_entries) {
  std::vector<ProfRec> recs;
  {
    std::lock_guard<std::mutex> l(g_prof_mu);
    recs.swap(g_prof);
  }
  std::vector<std::string> keys;
  std::vector<int64_t> cnt;
  std::vector<double> ms;
  int32_t rc = 0;
  for (auto& r : recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
      rc = -1;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
    size_t i = 0;
    while (i < keys.size() && keys[i] != r.name) ++i;
    if (i == keys.size()) {
      keys.push_back(r.name);
      cnt.push_back(0);
      ms.push_back(0.0);
    }
    cnt[i] += 1;
    ms[i] += t;
  }
  if (rc < 0) return -1;
  size_t off = 0;
  int32_t n = 0;
  for (size_t i = 0; i < keys.size() && n < max_entries; ++i) {
    if (names) {
      if (off + keys[i].size() + 1 > names_len) break;
      std::memcpy(names + off, keys[i].c_str(), keys[i].size() + 1);
      off += keys[i].size() + 1;
    }
    if (launches) launches[n] = cnt[i];
    if (total_ms) total_ms[n] = ms[i];
    ++n;
  }
  return n;
}

}  // extern "C"
