/*
 * Engram conditional-memory oracle: a plain, slow, double-precision CPU
 * statement of what the hot path computes.  TEST INFRASTRUCTURE ONLY: it is
 * loaded by tests/, by __graft_entry__.smoke() and by the bench's CPU
 * baseline, never by the library it checks, and it shares no code with it.
 *
 * Sources (web pages on DeepSeek's "Conditional Memory via Scalable Lookup"):
 *   [P1] "DeepSeek AI II" (taking-lying-flat blog), section
 *        "DeepSeek Engram": tokenizer compression, suffix N-grams,
 *        multi-head hashing into prime-sized tables, concatenation, the
 *        context-aware gate with RMSNorm on query and key, the gated value,
 *        the short depthwise causal convolution, the residual add; section
 *        on system efficiency: deterministic id-only addressing, training
 *        gradients dispatched back to table shards, prefetch from host.
 *   [P2] machine-heart news mirror of the Engram paper, sections
 *        "hashed N-gram sparse retrieval" and "system efficiency".
 *   [P5] QbitAI mirror: one independent table per hash head, all heads of
 *        all orders concatenated into the memory vector e_t.
 * The pages print no formulas for the hash, gate or conv; the forms taken
 * here (multiply-XOR mod prime, sigmoid of the scaled RMSNorm dot product,
 * kernel-4 depthwise conv + SiLU + residual) are the plainest readings, each
 * listed with its alternatives in the design notes.
 *
 * Parity pins: every function below is checked by tests/test_oracle_*.py
 * against brute force, closed forms, library routines or finite
 * differences; none is "parity unpinned".
 *
 * Input dtypes (of the tables, of the weights, of the hidden states and
 * upstream gradient, each given separately):
 *   0 = float32, 1 = bfloat16 bit patterns (uint16), 2 = float64.
 * All arithmetic is double; outputs are double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define OR_MAX_ORDERS 4

typedef struct {
  /* addressing [P1 "DeepSeek Engram": tokenizer compression, multi-head hashing] */
  int32_t num_orders;
  int32_t orders[OR_MAX_ORDERS]; /* N-gram orders, ascending */
  int32_t heads;                 /* K hash heads per order */
  int32_t max_order;             /* row length of mult[] */
  const uint64_t* mult;          /* [J][max_order]: mult[j][i] multiplies c_{t-i} */
  const int64_t* table_rows;     /* [J] prime table sizes M_j */
  int32_t pad_id;                /* canonical id standing in before the sequence start */
  const int32_t* canon_map;      /* [vocab] surjection raw id -> canonical id */
  int32_t vocab;
  const int32_t* tokens;         /* [B][T] raw ids */
  int64_t B, T;
  /* memory */
  int32_t dim;                   /* D columns per table row */
  int32_t dtype;                 /* of the tables */
  int32_t w_dtype;               /* of w_k, w_v */
  int32_t act_dtype;             /* of h and dy */
  const void* const* tables;     /* [J] pointers to [M_j][D] */
  /* fusion [P1 gate + conv] */
  int32_t hidden;                /* d */
  const void* w_k;               /* [d][d_mem], k_t = W_K e_t */
  const void* w_v;               /* [d][d_mem], v_t = W_V e_t */
  const void* h;                 /* [B][T][d] */
  const double* gamma_q;         /* [d] RMSNorm scale of the query, NULL = 1 */
  const double* gamma_k;         /* [d] RMSNorm scale of the key, NULL = 1 */
  double eps;
  int32_t taps;                  /* conv kernel width */
  const double* conv_w;          /* [d][taps], tap i multiplies position t-i */
  /* FP8 projection [P1 "DeepSeek Engram", multi-branch integration: the
   * projections as one dense FP8 matmul]: nonzero = e_t is quantized to e4m3
   * per token before W_K and W_V apply (W is passed already quantized) */
  int32_t fp8_e;
} oracle_problem;

static int n_tables(const oracle_problem* p) { return p->num_orders * p->heads; }
static int64_t d_mem(const oracle_problem* p) { return (int64_t)n_tables(p) * p->dim; }

static double load_val(const void* base, int32_t dtype, int64_t i) {
  if (dtype == 0) return (double)((const float*)base)[i];
  if (dtype == 2) return ((const double*)base)[i];
  uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* ------------------------------------------------------------------ FP8
 * OCP 8-bit floating point, E4M3 ("fn": bias 7, no infinities, largest
 * finite 448 = 1.75 * 2^8, code S.1111.111 is NaN).  Normal codes (exponent
 * field E >= 1) are (1 + m/8) 2^(E-7); E = 0 holds the subnormals m 2^-9.
 */
double oracle_e4m3_decode(uint8_t code) {
  int sgn = code >> 7, E = (code >> 3) & 15, m = code & 7;
  double v = E ? ldexp(1.0 + m / 8.0, E - 7) : ldexp((double)m, -9);
  return sgn ? -v : v;
}

/* Round x (any finite double) to the nearest E4M3 value, ties to the even
 * mantissa, magnitudes above 448 saturating to 448. */
uint8_t oracle_e4m3_encode(double x) {
  uint8_t sgn = x < 0 ? 0x80 : 0;
  double a = fabs(x);
  if (a >= 448.0) return sgn | 0x7E;
  if (a < ldexp(1.0, -6)) {                       /* subnormal range: units of 2^-9 */
    double u = a * 512.0;
    double r = floor(u);
    double f = u - r;
    if (f > 0.5 || (f == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    return sgn | (uint8_t)r;                      /* r == 8 is the smallest normal, code 0x08 */
  }
  int e;
  double fr = frexp(a, &e);                       /* a = fr 2^e, fr in [0.5, 1) */
  int E = e - 1;                                   /* a = (2 fr) 2^E, 2 fr in [1, 2) */
  double u = (2.0 * fr - 1.0) * 8.0;              /* mantissa in units of 1/8 */
  double r = floor(u);
  double f = u - r;
  if (f > 0.5 || (f == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  if (r == 8.0) {
    r = 0.0;
    E += 1;
  }
  if (E > 8 || (E == 8 && r > 6.0)) return sgn | 0x7E;
  return sgn | (uint8_t)(((E + 7) << 3) | (int)r);
}

/* Per-row quantization: s = max_i |x_i| / 448 and codes e4m3(x_i / s), both
 * in fp32 arithmetic (the scale and the quotient rounded to fp32 as a device
 * computes them); an all-zero row gets s = 1.  deq (optional) = decode * s. */
void oracle_quantize_row(const double* x, int64_t n, uint8_t* codes, float* scale, double* deq) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf((float)x[i]);
    if (a > amax) amax = a;
  }
  float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int64_t i = 0; i < n; ++i) {
    float q = (float)x[i] / s;
    uint8_t c = oracle_e4m3_encode((double)q);
    if (codes) codes[i] = c;
    if (deq) deq[i] = oracle_e4m3_decode(c) * (double)s;
  }
  *scale = s;
}

/* rows x cols of a dtype-coded array (see load_val) */
int oracle_quantize_rows(const void* src, int32_t dtype, int64_t rows, int64_t cols, uint8_t* codes,
                         float* scales, double* deq) {
  double* x = (double*)malloc(sizeof(double) * (cols ? cols : 1));
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) x[c] = load_val(src, dtype, r * cols + c);
    oracle_quantize_row(x, cols, codes ? codes + r * cols : NULL, scales + r,
                        deq ? deq + r * cols : NULL);
  }
  free(x);
  return 0;
}

/* ------------------------------------------------------------------ M0
 * [P1 "DeepSeek Engram", tokenizer compression] x'_t = P(x_t); positions
 * before the start of a sequence take the padding id.
 */
static int32_t canonical_at(const oracle_problem* p, int64_t b, int64_t t) {
  if (t < 0) return p->pad_id;
  return p->canon_map[p->tokens[b * p->T + t]];
}

/* ------------------------------------------------------------------ M1
 * [P1 "DeepSeek Engram", multi-head hashing; P5 one table per head]
 * For order n and head k (table j = order_index*K + k):
 *   idx_j(t) = ( XOR_{i<n} (mult[j][i] * c_{t-i} mod 2^64) ) mod M_j
 * with unsigned 64-bit arithmetic.
 */
int oracle_hash_at(const oracle_problem* p, int64_t b, int64_t t, int32_t* idx_out) {
  int j = 0;
  for (int o = 0; o < p->num_orders; ++o) {
    int n = p->orders[o];
    for (int k = 0; k < p->heads; ++k, ++j) {
      uint64_t x = 0;
      for (int i = 0; i < n; ++i) {
        uint64_t c = (uint64_t)(uint32_t)canonical_at(p, b, t - i);
        x ^= p->mult[(int64_t)j * p->max_order + i] * c; /* wraps mod 2^64 */
      }
      idx_out[j] = (int32_t)(x % (uint64_t)p->table_rows[j]);
    }
  }
  return 0;
}

/* idx for a list of flat positions pos[q] = b*T + t; out [npos][J] */
int oracle_hash(const oracle_problem* p, int64_t npos, const int64_t* pos, int32_t* out) {
  int J = n_tables(p);
#pragma omp parallel for schedule(static)
  for (int64_t q = 0; q < npos; ++q)
    oracle_hash_at(p, pos[q] / p->T, pos[q] % p->T, out + q * J);
  return 0;
}

/* ------------------------------------------------------------------ M2
 * [P1 "DeepSeek Engram": concatenate all retrieved embeddings into e_t;
 * P5: all heads of all orders]  e_t[j*D + c] = E_j[idx_j(t)][c]
 */
static void gather_row(const oracle_problem* p, const int32_t* idx, double* e) {
  int J = n_tables(p);
  for (int j = 0; j < J; ++j)
    for (int c = 0; c < p->dim; ++c)
      e[(int64_t)j * p->dim + c] = load_val(p->tables[j], p->dtype, (int64_t)idx[j] * p->dim + c);
}

int oracle_gather(const oracle_problem* p, int64_t npos, const int32_t* idx, double* e_out) {
#pragma omp parallel for schedule(static)
  for (int64_t q = 0; q < npos; ++q) gather_row(p, idx + q * n_tables(p), e_out + q * d_mem(p));
  return 0;
}

/* ------------------------------------------------------------------ M3
 * [P1 "DeepSeek Engram": e_t is the shared input of the key and value
 * projections]  out[c] = sum_i W[c][i] e[i]
 */
static void project(const oracle_problem* p, const void* W, const double* e, double* out) {
  int64_t dm = d_mem(p);
  for (int c = 0; c < p->hidden; ++c) {
    double s = 0.0;
    for (int64_t i = 0; i < dm; ++i) s += load_val(W, p->w_dtype, (int64_t)c * dm + i) * e[i];
    out[c] = s;
  }
}

/* [P1 "DeepSeek Engram": RMSNorm on query h_t and key k_t before a scalar
 * gate in (0,1)]  q = g_q h / rms(h), k^ = g_k k / rms(k),
 * s = <q, k^>/sqrt(d), alpha = sigmoid(s).  rms(x) = sqrt(mean(x^2)+eps).
 * Also returns 1/rms(h), 1/rms(k) and the raw score s.
 */
static double gate(const oracle_problem* p, const double* h, const double* k,
                   double* rq_out, double* rk_out, double* s_out) {
  int d = p->hidden;
  double sh = 0.0, sk = 0.0;
  for (int c = 0; c < d; ++c) {
    sh += h[c] * h[c];
    sk += k[c] * k[c];
  }
  double rq = 1.0 / sqrt(sh / d + p->eps);
  double rk = 1.0 / sqrt(sk / d + p->eps);
  double dot = 0.0;
  for (int c = 0; c < d; ++c) {
    double gq = p->gamma_q ? p->gamma_q[c] : 1.0;
    double gk = p->gamma_k ? p->gamma_k[c] : 1.0;
    dot += (gq * h[c] * rq) * (gk * k[c] * rk);
  }
  double s = dot / sqrt((double)d);
  if (rq_out) *rq_out = rq;
  if (rk_out) *rk_out = rk;
  if (s_out) *s_out = s;
  return sigmoid(s);
}

/* Exposed for the gate pins: alpha for given h, k vectors (double). */
double oracle_gate_value(const oracle_problem* p, const double* h, const double* k) {
  return gate(p, h, k, NULL, NULL, NULL);
}

/* Per-position state of the forward at one token. */
typedef struct {
  double* e;   /* [d_mem] */
  double* h;   /* [d] */
  double* k;   /* [d] */
  double* v;   /* [d] */
  double* vt;  /* [d] gated value alpha*v */
  double alpha, rq, rk, s;
} tok_state;

static void tok_alloc(const oracle_problem* p, tok_state* st) {
  int d = p->hidden;
  st->e = (double*)malloc(sizeof(double) * d_mem(p));
  st->h = (double*)malloc(sizeof(double) * d);
  st->k = (double*)malloc(sizeof(double) * d);
  st->v = (double*)malloc(sizeof(double) * d);
  st->vt = (double*)malloc(sizeof(double) * d);
}

static void tok_free(tok_state* st) {
  free(st->e); free(st->h); free(st->k); free(st->v); free(st->vt);
}

/* Retrieval and gating at token (b,t); t < 0 yields a zero gated value
 * (the causal convolution sees zeros before the sequence start). */
static void token_forward(const oracle_problem* p, int64_t b, int64_t t, tok_state* st) {
  int d = p->hidden;
  if (t < 0) {
    memset(st->vt, 0, sizeof(double) * d);
    memset(st->v, 0, sizeof(double) * d);
    st->alpha = 0.0;
    return;
  }
  int32_t idx[64];
  oracle_hash_at(p, b, t, idx);
  gather_row(p, idx, st->e);
  if (p->fp8_e) {  /* e_t in e4m3 with its own scale, as the FP8 projection reads it */
    float s;
    oracle_quantize_row(st->e, d_mem(p), NULL, &s, st->e);
  }
  for (int c = 0; c < d; ++c) st->h[c] = load_val(p->h, p->act_dtype, (b * p->T + t) * d + c);
  project(p, p->w_k, st->e, st->k);
  project(p, p->w_v, st->e, st->v);
  st->alpha = gate(p, st->h, st->k, &st->rq, &st->rk, &st->s);
  for (int c = 0; c < d; ++c) st->vt[c] = st->alpha * st->v[c]; /* [P1] v~ = alpha v */
}

/* [P1 "DeepSeek Engram": short-kernel depthwise causal convolution]
 * z_t[c] = sum_{i<taps} w[c][i] * vt_{t-i}[c]; Y_t = SiLU(z_t) + vt_t.
 * win[i] is vt at position t-i. */
static void conv_out(const oracle_problem* p, double* const* win, double* z, double* y) {
  int d = p->hidden;
  for (int c = 0; c < d; ++c) {
    double acc = 0.0;
    for (int i = 0; i < p->taps; ++i) acc += p->conv_w[(int64_t)c * p->taps + i] * win[i][c];
    if (z) z[c] = acc;
    if (y) y[c] = acc * sigmoid(acc) + win[0][c];
  }
}

/* The conv alone on a given gated-value sequence vt [T][d] -> z, y [T][d]
 * (exposed for the impulse-response and causality pins). */
int oracle_conv(const oracle_problem* p, int64_t T, const double* vt, double* z, double* y) {
  int d = p->hidden;
  double* zero = (double*)calloc(d, sizeof(double));
  double* win[16];
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < p->taps; ++i) win[i] = (t - i >= 0) ? (double*)(vt + (t - i) * d) : zero;
    conv_out(p, win, z ? z + t * d : NULL, y ? y + t * d : NULL);
  }
  free(zero);
  return 0;
}

/*
 * Forward at a list of flat positions pos[q] = b*T + t.
 * Outputs (each may be NULL): y [npos][d], alpha [npos], k [npos][d],
 * v [npos][d], e [npos][d_mem].
 * Each position is computed on its own: the gated values at t-taps+1..t,
 * then the conv.
 */
int oracle_forward(const oracle_problem* p, int64_t npos, const int64_t* pos, double* y,
                   double* alpha, double* k, double* v, double* e) {
  int d = p->hidden;
  int taps = p->taps;
#pragma omp parallel
  {
    tok_state st[16];
    for (int i = 0; i < taps; ++i) tok_alloc(p, &st[i]);
#pragma omp for schedule(dynamic, 1)
    for (int64_t q = 0; q < npos; ++q) {
      int64_t b = pos[q] / p->T, t = pos[q] % p->T;
      double* win[16];
      for (int i = 0; i < taps; ++i) {
        token_forward(p, b, t - i, &st[i]);
        win[i] = st[i].vt;
      }
      if (y) conv_out(p, win, NULL, y + q * d);
      if (alpha) alpha[q] = st[0].alpha;
      if (k) memcpy(k + q * d, st[0].k, sizeof(double) * d);
      if (v) memcpy(v + q * d, st[0].v, sizeof(double) * d);
      if (e) memcpy(e + q * d_mem(p), st[0].e, sizeof(double) * d_mem(p));
    }
    for (int i = 0; i < taps; ++i) tok_free(&st[i]);
  }
  return 0;
}

/*
 * Backward at one token t of sequence b for L = sum_t <G_t, Y_t>, G = dy
 * (dtype of the problem, [B][T][d]).  Derived by the chain rule from the
 * forward above (the pages print no backward):
 *   dz_u   = G_u * sig(z_u) * (1 + z_u (1 - sig(z_u)))            u = t..t+taps-1
 *   dvt_t  = G_t + sum_i w[:,i] * dz_{t+i}
 *   dalpha = <dvt_t, v_t>,  dv_t = alpha_t dvt_t
 *   ds     = dalpha * alpha (1 - alpha)
 *   dk^    = ds * q / sqrt(d)                  (q = g_q h rq)
 *   g      = g_k * dk^,  dk = rk g - rk^3 k <g,k> / d
 * st[0 .. 2 taps-2] receive the forward at t-taps+1 .. t+taps-1 (st[taps-1]
 * is t itself), dz[i*d + c] the conv-input gradient at t+i; dk, dv [d] and
 * *ds_out are written.
 */
typedef struct {
  double* dz;   /* [taps][d] */
  double* z;    /* [d] */
  double* dvt;  /* [d] */
  double* g;    /* [d] */
} bwd_scratch;

static void bwd_alloc(const oracle_problem* p, bwd_scratch* w) {
  int d = p->hidden;
  w->dz = (double*)malloc(sizeof(double) * d * p->taps);
  w->z = (double*)malloc(sizeof(double) * d);
  w->dvt = (double*)malloc(sizeof(double) * d);
  w->g = (double*)malloc(sizeof(double) * d);
}

static void bwd_free(bwd_scratch* w) { free(w->dz); free(w->z); free(w->dvt); free(w->g); }

static void token_backward(const oracle_problem* p, const void* dy, int64_t b, int64_t t,
                           tok_state* st, bwd_scratch* w, double* dk, double* dv, double* ds_out) {
  int d = p->hidden;
  int taps = p->taps;
  int W = 2 * taps - 1; /* positions t-taps+1 .. t+taps-1 */
  double* dz = w->dz;
  double* z = w->z;
  double* dvt = w->dvt;
  double* g = w->g;
  for (int s = 0; s < W; ++s) {
    int64_t u = t - (taps - 1) + s;
    if (u < p->T) token_forward(p, b, u, &st[s]);
  }
  /* dz at u = t + i, i < taps */
  for (int i = 0; i < taps; ++i) {
    int64_t u = t + i;
    if (u >= p->T) {
      memset(dz + (int64_t)i * d, 0, sizeof(double) * d);
      continue;
    }
    double* win[16];
    for (int a = 0; a < taps; ++a) win[a] = st[(taps - 1) + i - a].vt;
    conv_out(p, win, z, NULL);
    for (int c = 0; c < d; ++c) {
      double G = load_val(dy, p->act_dtype, (b * p->T + u) * d + c);
      double sg = sigmoid(z[c]);
      dz[(int64_t)i * d + c] = G * sg * (1.0 + z[c] * (1.0 - sg));
    }
  }
  tok_state* s0 = &st[taps - 1];
  double dalpha = 0.0;
  for (int c = 0; c < d; ++c) {
    double acc = load_val(dy, p->act_dtype, (b * p->T + t) * d + c);
    for (int i = 0; i < taps; ++i) acc += p->conv_w[(int64_t)c * taps + i] * dz[(int64_t)i * d + c];
    dvt[c] = acc;
    dalpha += acc * s0->v[c];
  }
  for (int c = 0; c < d; ++c) dv[c] = s0->alpha * dvt[c];
  double ds = dalpha * s0->alpha * (1.0 - s0->alpha);
  double gk_dot = 0.0;
  for (int c = 0; c < d; ++c) {
    double gq = p->gamma_q ? p->gamma_q[c] : 1.0;
    double gk = p->gamma_k ? p->gamma_k[c] : 1.0;
    double dkhat = ds * gq * s0->h[c] * s0->rq / sqrt((double)d);
    g[c] = gk * dkhat;
    gk_dot += g[c] * s0->k[c];
  }
  double rk = s0->rk;
  for (int c = 0; c < d; ++c) dk[c] = rk * g[c] - rk * rk * rk * s0->k[c] * gk_dot / d;
  *ds_out = ds;
}

/*
 * Backward to the memory vector at the positions pos[q] = b*T + t:
 *   de_t = W_K^T dk_t + W_V^T dv_t        (dk, dv from token_backward)
 * Output de [npos][d_mem].
 */
int oracle_backward_de(const oracle_problem* p, const void* dy, int64_t npos, const int64_t* pos,
                       double* de_out) {
  int d = p->hidden;
  int taps = p->taps;
  int64_t dm = d_mem(p);
  int W = 2 * taps - 1;
#pragma omp parallel
  {
    tok_state st[32];
    for (int i = 0; i < W; ++i) tok_alloc(p, &st[i]);
    bwd_scratch ws;
    bwd_alloc(p, &ws);
    double* dk = (double*)malloc(sizeof(double) * d);
    double* dv = (double*)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t q = 0; q < npos; ++q) {
      int64_t b = pos[q] / p->T, t = pos[q] % p->T;
      double ds;
      token_backward(p, dy, b, t, st, &ws, dk, dv, &ds);
      double* de = de_out + q * dm;
      for (int64_t i = 0; i < dm; ++i) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c)
          acc += load_val(p->w_k, p->w_dtype, (int64_t)c * dm + i) * dk[c] +
                 load_val(p->w_v, p->w_dtype, (int64_t)c * dm + i) * dv[c];
        de[i] = acc;
      }
    }
    for (int i = 0; i < W; ++i) tok_free(&st[i]);
    bwd_free(&ws);
    free(dk); free(dv);
  }
  return 0;
}

/*
 * Gradients of the module's own parameters and of the hidden state, for the
 * same L, by the chain rule through the same forward:
 *   dW_K[c][i]  = sum_t dk_t[c] e_t[i],   dW_V[c][i] = sum_t dv_t[c] e_t[i]
 *                 (k_t = W_K e_t, v_t = W_V e_t)
 *   dconv[c][i] = sum_t dz_t[c] vt_{t-i}[c]      (z_t = sum_i w[c][i] vt_{t-i})
 *   with q = g_q h rq, k^ = g_k k rk, s = <q, k^>/sqrt(d):
 *   dq = ds k^ / sqrt(d),  dk^ = ds q / sqrt(d)
 *   dgamma_q[c] = sum_t dq[c] h_t[c] rq_t,   dgamma_k[c] = sum_t dk^[c] k_t[c] rk_t
 *   dh_t = rq f - rq^3 h_t <f, h_t> / d,  f = g_q dq     (RMSNorm backward;
 *          the gate's part only: the caller's residual H + Y adds G itself)
 * The sums run over the positions pos[0..npos) (all positions give the full
 * gradients; where G vanishes on t..t+taps-1 a position adds nothing).
 * Outputs, each may be NULL: dw_k, dw_v [d][d_mem], dconv [d][taps],
 * dgamma_q, dgamma_k [d] (sums), dh [npos][d] (per position).
 */
int oracle_backward_params(const oracle_problem* p, const void* dy, int64_t npos, const int64_t* pos,
                           double* dw_k, double* dw_v, double* dconv, double* dgamma_q,
                           double* dgamma_k, double* dh) {
  int d = p->hidden;
  int taps = p->taps;
  int64_t dm = d_mem(p);
  int W = 2 * taps - 1;
  const int64_t CH = 256; /* positions per chunk: computed in parallel, summed in order */
  /* per position of a chunk: dk, dv, e, dz (x) vt window, dq h rq, dk^ k rk */
  int64_t per = 2 * d + dm + (int64_t)d * taps + 2 * d;
  double* buf = (double*)malloc(sizeof(double) * CH * per);
  if (dw_k) memset(dw_k, 0, sizeof(double) * d * dm);
  if (dw_v) memset(dw_v, 0, sizeof(double) * d * dm);
  if (dconv) memset(dconv, 0, sizeof(double) * d * taps);
  if (dgamma_q) memset(dgamma_q, 0, sizeof(double) * d);
  if (dgamma_k) memset(dgamma_k, 0, sizeof(double) * d);
  for (int64_t q0 = 0; q0 < npos; q0 += CH) {
    int64_t nq = npos - q0 < CH ? npos - q0 : CH;
#pragma omp parallel
    {
      tok_state st[32];
      for (int i = 0; i < W; ++i) tok_alloc(p, &st[i]);
      bwd_scratch ws;
      bwd_alloc(p, &ws);
#pragma omp for schedule(dynamic, 1)
      for (int64_t a = 0; a < nq; ++a) {
        int64_t b = pos[q0 + a] / p->T, t = pos[q0 + a] % p->T;
        double* o = buf + a * per;
        double *dk = o, *dv = o + d, *e = o + 2 * d, *cz = e + dm, *gqs = cz + (int64_t)d * taps,
               *gks = gqs + d;
        double ds;
        token_backward(p, dy, b, t, st, &ws, dk, dv, &ds);
        tok_state* s0 = &st[taps - 1];
        memcpy(e, s0->e, sizeof(double) * dm);
        for (int c = 0; c < d; ++c)
          for (int i = 0; i < taps; ++i) /* dz_t at index 0 of the scratch; vt_{t-i} = st[taps-1-i] */
            cz[(int64_t)c * taps + i] = ws.dz[c] * st[taps - 1 - i].vt[c];
        double sd = sqrt((double)d);
        double fh = 0.0;
        for (int c = 0; c < d; ++c) {
          double gq = p->gamma_q ? p->gamma_q[c] : 1.0;
          double gk = p->gamma_k ? p->gamma_k[c] : 1.0;
          double qv = gq * s0->h[c] * s0->rq;
          double kv = gk * s0->k[c] * s0->rk;
          double dq = ds * kv / sd;
          double dkh = ds * qv / sd;
          gqs[c] = dq * s0->h[c] * s0->rq;
          gks[c] = dkh * s0->k[c] * s0->rk;
          fh += gq * dq * s0->h[c];
        }
        if (dh) {
          double rq = s0->rq;
          for (int c = 0; c < d; ++c) {
            double gq = p->gamma_q ? p->gamma_q[c] : 1.0;
            double gk = p->gamma_k ? p->gamma_k[c] : 1.0;
            double f = gq * ds * (gk * s0->k[c] * s0->rk) / sd;
            dh[(q0 + a) * d + c] = rq * f - rq * rq * rq * s0->h[c] * fh / d;
          }
        }
      }
      for (int i = 0; i < W; ++i) tok_free(&st[i]);
      bwd_free(&ws);
    }
    for (int64_t a = 0; a < nq; ++a) {
      const double* o = buf + a * per;
      const double *dk = o, *dv = o + d, *e = o + 2 * d, *cz = e + dm, *gqs = cz + (int64_t)d * taps,
                   *gks = gqs + d;
      for (int c = 0; c < d; ++c) {
        if (dw_k)
          for (int64_t i = 0; i < dm; ++i) dw_k[(int64_t)c * dm + i] += dk[c] * e[i];
        if (dw_v)
          for (int64_t i = 0; i < dm; ++i) dw_v[(int64_t)c * dm + i] += dv[c] * e[i];
        if (dconv)
          for (int i = 0; i < taps; ++i) dconv[(int64_t)c * taps + i] += cz[(int64_t)c * taps + i];
        if (dgamma_q) dgamma_q[c] += gqs[c];
        if (dgamma_k) dgamma_k[c] += gks[c];
      }
    }
  }
  free(buf);
  return 0;
}

/*
 * Table gradient for selected rows [P1 system efficiency: in training the
 * gradients of the gathered rows are sent back to the rows they came from]:
 *   dE_j[r] = sum over (b,t) with idx_j(b,t) = r of de_t[j*D:(j+1)*D]
 * rows_j[q], rows_r[q] name the q-th requested row; out [nrows][D].
 * `idx_all` [B*T][J] are the indices of every position (oracle_hash).
 */
int oracle_table_grad_rows(const oracle_problem* p, const void* dy, const int32_t* idx_all,
                           int64_t nrows, const int32_t* rows_j, const int32_t* rows_r, double* out) {
  int J = n_tables(p);
  int D = p->dim;
  int64_t N = p->B * p->T;
  int64_t dm = d_mem(p);
  /* positions that touch any requested row */
  int64_t cap = 1024, npos = 0;
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * cap);
  for (int64_t n = 0; n < N; ++n) {
    int hit = 0;
    for (int64_t q = 0; q < nrows && !hit; ++q)
      hit = idx_all[n * J + rows_j[q]] == rows_r[q];
    if (hit) {
      if (npos == cap) {
        cap *= 2;
        pos = (int64_t*)realloc(pos, sizeof(int64_t) * cap);
      }
      pos[npos++] = n;
    }
  }
  double* de = (double*)malloc(sizeof(double) * (npos ? npos : 1) * dm);
  oracle_backward_de(p, dy, npos, pos, de);
  memset(out, 0, sizeof(double) * nrows * D);
  for (int64_t q = 0; q < nrows; ++q)
    for (int64_t a = 0; a < npos; ++a)
      if (idx_all[pos[a] * J + rows_j[q]] == rows_r[q])
        for (int c = 0; c < D; ++c) out[q * D + c] += de[a * dm + (int64_t)rows_j[q] * D + c];
  free(de);
  free(pos);
  return (int)(npos > 0x7fffffff ? 0x7fffffff : npos);
}

/*
 * Dense table gradient of every table (small problems only):
 * grads[j] points to [M_j][D] doubles, zero-filled here.
 */
int oracle_table_grad_dense(const oracle_problem* p, const void* dy, double* const* grads) {
  int J = n_tables(p);
  int D = p->dim;
  int64_t N = p->B * p->T;
  int64_t dm = d_mem(p);
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (N ? N : 1));
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (N ? N : 1) * J);
  double* de = (double*)malloc(sizeof(double) * (N ? N : 1) * dm);
  for (int64_t n = 0; n < N; ++n) pos[n] = n;
  oracle_hash(p, N, pos, idx);
  oracle_backward_de(p, dy, N, pos, de);
  for (int j = 0; j < J; ++j) memset(grads[j], 0, sizeof(double) * p->table_rows[j] * D);
  for (int64_t n = 0; n < N; ++n)
    for (int j = 0; j < J; ++j)
      for (int c = 0; c < D; ++c)
        grads[j][(int64_t)idx[n * J + j] * D + c] += de[n * dm + (int64_t)j * D + c];
  free(pos); free(idx); free(de);
  return 0;
}

/*
 * Prefetch plan [P1 system efficiency: indices are fixed by the token ids
 * before the forward pass, so the rows can be fetched ahead]:
 * for each table j, U_j = ascending distinct rows among idx[:, j] and
 * inv[n][j] = position of idx[n][j] in U_j.
 * uniq_out holds the U_j back to back (capacity N*J), counts[j] = |U_j|.
 */
static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int oracle_prefetch_plan(int64_t N, int32_t J, const int32_t* idx, int32_t* uniq_out, int64_t* counts,
                         int32_t* inv_out) {
  int32_t* col = (int32_t*)malloc(sizeof(int32_t) * (N ? N : 1));
  int64_t base = 0;
  for (int j = 0; j < J; ++j) {
    for (int64_t n = 0; n < N; ++n) col[n] = idx[n * J + j];
    qsort(col, (size_t)N, sizeof(int32_t), cmp_i32);
    int64_t u = 0;
    for (int64_t n = 0; n < N; ++n)
      if (n == 0 || col[n] != col[n - 1]) uniq_out[base + u++] = col[n];
    counts[j] = u;
    for (int64_t n = 0; n < N; ++n) {
      int32_t key = idx[n * J + j];
      int64_t lo = 0, hi = u - 1;
      while (lo < hi) {
        int64_t mid = (lo + hi) >> 1;
        if (uniq_out[base + mid] < key) lo = mid + 1; else hi = mid;
      }
      inv_out[n * J + j] = (int32_t)lo;
    }
    base += u;
  }
  free(col);
  return 0;
}

/* Threads the parallel loops above use (for reporting the oracle's timing). */
int oracle_threads(void) { return omp_get_max_threads(); }
