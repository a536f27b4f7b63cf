/*
 * kda_oracle.c -- plain fp64 CPU oracle of the Kimi Delta Attention (KDA) layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this file:
 * only the tests, the package smoke check and the benchmark's CPU-baseline leg
 * load it.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (sources: TensorFold issue #850 "Ling-3.1-flash on CUDA",
 * the comment describing the shared KDA module, which lists the layer's parts
 * in order: conv window, safe or softplus gate, beta, q/k L2 norms, delta rule,
 * gated output norm; onnxruntime-genai PR #2843 description, which names the
 * ops CausalConvWithState / VarlenCausalConvWithState, GatedDeltaNet with
 * per-key-dim decay and a sigmoid gate activation with a lower bound, and
 * GatedRMSNorm with a sigmoid activation).  The pages print no formula; the
 * recurrence itself is the gated delta rule with per-key-dimension decay
 *     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t,
 * evaluated here in the algebraically equal form
 *     S' = Diag(a_t) S_{t-1};  u_t = b_t (v_t - S'^T k_t);  S_t = S' + k_t u_t^T.
 *
 * Every loop follows the definition directly; there is no blocking or fusion
 * other than the chunked form (kda_oracle_chunked), which is the chunk-parallel
 * restatement of the same recurrence and is pinned against the serial form.
 *
 * Layouts (all row-major, doubles):
 *   packed rows     q,k,g: [T_tot, H, dk]   v,o,z: [T_tot, H, dv]   beta: [T_tot, H]
 *   cu_seqlens      [N+1], cu[0] = 0, non-decreasing, cu[N] = T_tot
 *   state           [N, H, dk, dv]   (dv contiguous)
 *   conv channels   C = H*(2*dk+dv), ordered [q: H*dk | k: H*dk | v: H*dv]
 *   conv weight     [C, W]  (tap W-1 multiplies the current row)
 *   conv state      [N, W-1, C]  (oldest row first)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KDA_ORACLE_GATE_SOFTPLUS 0
#define KDA_ORACLE_GATE_SAFE 1
#define KDA_ORACLE_ACT_NONE 0
#define KDA_ORACLE_ACT_SILU 1

/* ------------------------------------------------------------------------ */
/* scalar functions                                                          */
/* ------------------------------------------------------------------------ */

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x), written so that it neither overflows nor loses
 * the small tail: max(x,0) + log1p(e^{-|x|}). */
static double softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

/* Log-decay gate (TensorFold #850: "the safe or softplus gate"; ORT #2843:
 * gate_activation='sigmoid' with gate_lower_bound).
 *   softplus: g = -softplus(x)          (a = e^g in (0, 1))
 *   safe:     g = lower_bound * sigmoid(x)   (a in (e^lb, 1)) */
static double gate_log_decay(double x, int mode, double lb) {
  if (mode == KDA_ORACLE_GATE_SAFE) return lb * sigmoid(x);
  return -softplus(x);
}

/* ------------------------------------------------------------------------ */
/* a tiny work queue over independent (sequence, head) units                 */
/* ------------------------------------------------------------------------ */

typedef void (*unit_fn)(void* ctx, int64_t unit);
typedef struct {
  unit_fn fn;
  void* ctx;
  int64_t n_units;
  int64_t next;
  pthread_mutex_t mu;
} pool_t;

static void* pool_worker(void* arg) {
  pool_t* p = (pool_t*)arg;
  for (;;) {
    pthread_mutex_lock(&p->mu);
    int64_t u = p->next++;
    pthread_mutex_unlock(&p->mu);
    if (u >= p->n_units) break;
    p->fn(p->ctx, u);
  }
  return NULL;
}

static void run_units(unit_fn fn, void* ctx, int64_t n_units, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n_units) nthreads = (int)(n_units > 0 ? n_units : 1);
  pool_t p;
  p.fn = fn;
  p.ctx = ctx;
  p.n_units = n_units;
  p.next = 0;
  pthread_mutex_init(&p.mu, NULL);
  if (nthreads == 1) {
    pool_worker(&p);
  } else {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, pool_worker, &p);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&p.mu);
}

/* ------------------------------------------------------------------------ */
/* 1. preamble: causal short conv with carried state, activation, L2 norms,  */
/*    gates and beta.                                                        */
/* ------------------------------------------------------------------------ */

typedef struct {
  int H, dk, dv, W, act, gate_mode;
  double lb, eps;
  const int64_t* cu;
  const double *q_raw, *k_raw, *v_raw, *conv_w, *cs_in, *g_raw, *beta_logit;
  double *cs_out, *q_hat, *k_hat, *v_out, *g_out, *beta_out;
} prep_ctx;

/* Row x_t of channel c of sequence n, where t may reach back into the carried
 * conv state: t in [-(W-1), len). */
static double conv_src(const prep_ctx* c, int n, int64_t t, int ch) {
  const int C = c->H * (2 * c->dk + c->dv);
  if (t < 0) return c->cs_in[((int64_t)n * (c->W - 1) + (t + c->W - 1)) * C + ch];
  int64_t row = c->cu[n] + t;
  const int qk = c->H * c->dk;
  if (ch < qk) return c->q_raw[row * qk + ch];
  if (ch < 2 * qk) return c->k_raw[row * qk + (ch - qk)];
  return c->v_raw[row * (int64_t)(c->H * c->dv) + (ch - 2 * qk)];
}

/* one unit = one sequence (the conv couples all heads' channels only through
 * the shared layout, so a sequence is the natural unit) */
static void prep_unit(void* vctx, int64_t n64) {
  const prep_ctx* c = (const prep_ctx*)vctx;
  const int n = (int)n64;
  const int H = c->H, dk = c->dk, dv = c->dv, W = c->W;
  const int C = H * (2 * dk + dv);
  const int64_t t0 = c->cu[n], len = c->cu[n + 1] - c->cu[n];
  double* y = (double*)malloc(sizeof(double) * (size_t)C);
  for (int64_t t = 0; t < len; ++t) {
    const int64_t row = t0 + t;
    /* conv: c_t = sum_j w[c][j] * x_{t-(W-1)+j}, then the activation */
    for (int ch = 0; ch < C; ++ch) {
      double acc = 0.0;
      for (int j = 0; j < W; ++j) acc += c->conv_w[(int64_t)ch * W + j] * conv_src(c, n, t - (W - 1) + j, ch);
      if (c->act == KDA_ORACLE_ACT_SILU) acc = acc * sigmoid(acc);
      y[ch] = acc;
    }
    /* q/k L2 norms per head over dk; v passes through */
    for (int h = 0; h < H; ++h) {
      const double* yq = y + h * dk;
      const double* yk = y + H * dk + h * dk;
      double sq = 0.0, sk = 0.0;
      for (int d = 0; d < dk; ++d) {
        sq += yq[d] * yq[d];
        sk += yk[d] * yk[d];
      }
      const double rq = 1.0 / sqrt(sq + c->eps), rk = 1.0 / sqrt(sk + c->eps);
      for (int d = 0; d < dk; ++d) {
        c->q_hat[(row * H + h) * dk + d] = yq[d] * rq;
        c->k_hat[(row * H + h) * dk + d] = yk[d] * rk;
      }
      for (int d = 0; d < dv; ++d) c->v_out[(row * H + h) * dv + d] = y[2 * H * dk + h * dv + d];
      /* gates: per-key-dim log decay, per-head beta */
      for (int d = 0; d < dk; ++d) {
        const int64_t i = (row * H + h) * dk + d;
        c->g_out[i] = gate_log_decay(c->g_raw[i], c->gate_mode, c->lb);
      }
      c->beta_out[row * H + h] = sigmoid(c->beta_logit[row * H + h]);
    }
  }
  /* carried conv state: the last W-1 source rows, copied bit for bit */
  for (int r = 0; r < W - 1; ++r) {
    const int64_t t = len - (W - 1) + r;
    for (int ch = 0; ch < C; ++ch) c->cs_out[((int64_t)n * (W - 1) + r) * C + ch] = conv_src(c, n, t, ch);
  }
  free(y);
}

int kda_oracle_prep(int H, int dk, int dv, int W, int act, int num_seqs, const int64_t* cu,
                    const double* q_raw, const double* k_raw, const double* v_raw, const double* conv_w,
                    const double* conv_state_in, double* conv_state_out, const double* g_raw,
                    const double* beta_logit, int gate_mode, double lower_bound, double eps, double* q_hat,
                    double* k_hat, double* v_out, double* g_out, double* beta_out, int nthreads) {
  if (H <= 0 || dk <= 0 || dv <= 0 || W < 1 || num_seqs < 0) return -1;
  prep_ctx c = {H, dk, dv, W, act, gate_mode, lower_bound, eps, cu, q_raw, k_raw, v_raw, conv_w,
                conv_state_in, g_raw, beta_logit, conv_state_out, q_hat, k_hat, v_out, g_out, beta_out};
  run_units(prep_unit, &c, num_seqs, nthreads);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* 2. token-serial recurrence                                                */
/* ------------------------------------------------------------------------ */

typedef struct {
  int H, dk, dv;
  const int64_t* cu;
  const double *q, *k, *v, *g, *beta;
  double *state, *o, *log_a, *log_k, *log_u;
} rec_ctx;

static void rec_unit(void* vctx, int64_t unit) {
  const rec_ctx* c = (const rec_ctx*)vctx;
  const int H = c->H, dk = c->dk, dv = c->dv;
  const int n = (int)(unit / H), h = (int)(unit % H);
  double* S = c->state + ((int64_t)n * H + h) * dk * dv;
  double* ktS = (double*)malloc(sizeof(double) * (size_t)dv);
  double* u = (double*)malloc(sizeof(double) * (size_t)dv);
  double* a = (double*)malloc(sizeof(double) * (size_t)dk);
  for (int64_t row = c->cu[n]; row < c->cu[n + 1]; ++row) {
    const double* kt = c->k + (row * H + h) * dk;
    const double* qt = c->q + (row * H + h) * dk;
    const double* vt = c->v + (row * H + h) * dv;
    const double* gt = c->g + (row * H + h) * dk;
    const double b = c->beta[row * H + h];
    for (int i = 0; i < dk; ++i) a[i] = exp(gt[i]);
    /* S' = Diag(a) S */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[i * dv + j] *= a[i];
    /* u = b (v - S'^T k) */
    for (int j = 0; j < dv; ++j) ktS[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) ktS[j] += kt[i] * S[i * dv + j];
    for (int j = 0; j < dv; ++j) u[j] = b * (vt[j] - ktS[j]);
    /* S = S' + k u^T */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[i * dv + j] += kt[i] * u[j];
    /* o = S^T q */
    double* ot = c->o + (row * H + h) * dv;
    for (int j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) ot[j] += qt[i] * S[i * dv + j];
    /* per-row log: decay, normalised key, update (what a verify window keeps) */
    if (c->log_a) memcpy(c->log_a + (row * H + h) * dk, a, sizeof(double) * (size_t)dk);
    if (c->log_k) memcpy(c->log_k + (row * H + h) * dk, kt, sizeof(double) * (size_t)dk);
    if (c->log_u) memcpy(c->log_u + (row * H + h) * dv, u, sizeof(double) * (size_t)dv);
  }
  free(ktS);
  free(u);
  free(a);
}

int kda_oracle_recurrent(int H, int dk, int dv, int num_seqs, const int64_t* cu, const double* q_hat,
                         const double* k_hat, const double* v, const double* g, const double* beta, double* state,
                         double* o, double* log_a, double* log_k, double* log_u, int nthreads) {
  if (H <= 0 || dk <= 0 || dv <= 0 || num_seqs < 0) return -1;
  rec_ctx c = {H, dk, dv, cu, q_hat, k_hat, v, g, beta, state, o, log_a, log_k, log_u};
  run_units(rec_unit, &c, (int64_t)num_seqs * H, nthreads);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* 3. chunked (WY / UT) form of the same recurrence                          */
/* ------------------------------------------------------------------------ */
/* For a chunk of L rows r = 0..L-1 entering with state S0:
 *   G_r = sum_{i<=r} g_i (per key dim), gamma_r = e^{G_r}
 *   A_ri = b_r sum_d k_r[d] k_i[d] e^{G_r[d]-G_i[d]}        (i < r)
 *   P_ri =     sum_d q_r[d] k_i[d] e^{G_r[d]-G_i[d]}        (i <= r)
 *   (I + A) U = Diag(b) (V - K^gamma S0)   -> U by forward substitution
 *   O   = Q^gamma S0 + P U
 *   S_L = Diag(gamma_{L-1}) S0 + sum_i Diag(e^{G_{L-1}-G_i}) k_i u_i^T
 * Unrolling the serial rule over the chunk gives exactly these; the pairwise
 * exponents are evaluated directly (never overflow: every exponent <= 0). */

typedef struct {
  int H, dk, dv, chunk;
  const int64_t* cu;
  const double *q, *k, *v, *g, *beta;
  double *state, *o;
} chk_ctx;

static void chunk_unit(void* vctx, int64_t unit) {
  const chk_ctx* c = (const chk_ctx*)vctx;
  const int H = c->H, dk = c->dk, dv = c->dv, C = c->chunk;
  const int n = (int)(unit / H), h = (int)(unit % H);
  double* S = c->state + ((int64_t)n * H + h) * dk * dv;
  double* G = (double*)malloc(sizeof(double) * (size_t)C * dk);
  double* A = (double*)malloc(sizeof(double) * (size_t)C * C);
  double* P = (double*)malloc(sizeof(double) * (size_t)C * C);
  double* U = (double*)malloc(sizeof(double) * (size_t)C * dv);
  double* Snew = (double*)malloc(sizeof(double) * (size_t)dk * dv);
  for (int64_t c0 = c->cu[n]; c0 < c->cu[n + 1]; c0 += C) {
    const int L = (int)((c->cu[n + 1] - c0) < C ? (c->cu[n + 1] - c0) : C);
#define KR(r) (c->k + ((c0 + (r)) * H + h) * dk)
#define QR(r) (c->q + ((c0 + (r)) * H + h) * dk)
#define VR(r) (c->v + ((c0 + (r)) * H + h) * dv)
#define BR(r) (c->beta[(c0 + (r)) * H + h])
    for (int d = 0; d < dk; ++d) {
      double run = 0.0;
      for (int r = 0; r < L; ++r) {
        run += c->g[((c0 + r) * H + h) * dk + d];
        G[r * dk + d] = run;
      }
    }
    for (int r = 0; r < L; ++r)
      for (int i = 0; i < L; ++i) {
        double sa = 0.0, sp = 0.0;
        if (i <= r)
          for (int d = 0; d < dk; ++d) {
            const double e = exp(G[r * dk + d] - G[i * dk + d]);
            sa += KR(r)[d] * KR(i)[d] * e;
            sp += QR(r)[d] * KR(i)[d] * e;
          }
        A[r * C + i] = (i < r) ? BR(r) * sa : 0.0;
        P[r * C + i] = (i <= r) ? sp : 0.0;
      }
    /* right-hand side  Diag(b) (V - K^gamma S0), then forward substitution */
    for (int r = 0; r < L; ++r) {
      for (int j = 0; j < dv; ++j) {
        double ks = 0.0;
        for (int d = 0; d < dk; ++d) ks += exp(G[r * dk + d]) * KR(r)[d] * S[d * dv + j];
        double x = BR(r) * (VR(r)[j] - ks);
        for (int i = 0; i < r; ++i) x -= A[r * C + i] * U[i * dv + j];
        U[r * dv + j] = x;
      }
    }
    /* O = Q^gamma S0 + P U */
    for (int r = 0; r < L; ++r) {
      double* orow = c->o + ((c0 + r) * H + h) * dv;
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int d = 0; d < dk; ++d) acc += exp(G[r * dk + d]) * QR(r)[d] * S[d * dv + j];
        for (int i = 0; i <= r; ++i) acc += P[r * C + i] * U[i * dv + j];
        orow[j] = acc;
      }
    }
    /* S_L = Diag(gamma_last) S0 + sum_i Diag(e^{G_last - G_i}) k_i u_i^T */
    for (int d = 0; d < dk; ++d)
      for (int j = 0; j < dv; ++j) {
        double acc = exp(G[(L - 1) * dk + d]) * S[d * dv + j];
        for (int i = 0; i < L; ++i) acc += exp(G[(L - 1) * dk + d] - G[i * dk + d]) * KR(i)[d] * U[i * dv + j];
        Snew[d * dv + j] = acc;
      }
    memcpy(S, Snew, sizeof(double) * (size_t)dk * dv);
#undef KR
#undef QR
#undef VR
#undef BR
  }
  free(G);
  free(A);
  free(P);
  free(U);
  free(Snew);
}

int kda_oracle_chunked(int H, int dk, int dv, int chunk, int num_seqs, const int64_t* cu, const double* q_hat,
                       const double* k_hat, const double* v, const double* g, const double* beta, double* state,
                       double* o, int nthreads) {
  if (H <= 0 || dk <= 0 || dv <= 0 || chunk <= 0 || num_seqs < 0) return -1;
  chk_ctx c = {H, dk, dv, chunk, cu, q_hat, k_hat, v, g, beta, state, o};
  run_units(chunk_unit, &c, (int64_t)num_seqs * H, nthreads);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* 4. sigmoid-gated output RMSNorm (ORT #2843: GatedRMSNorm, activation      */
/*    'sigmoid'):  y = o / sqrt(mean(o^2) + eps) * w * sigmoid(z)            */
/* ------------------------------------------------------------------------ */

int kda_oracle_gated_rmsnorm(int64_t rows, int dv, const double* o, const double* z, const double* w, double eps,
                             double* y) {
  if (rows < 0 || dv <= 0) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    const double* orow = o + r * dv;
    double ss = 0.0;
    for (int j = 0; j < dv; ++j) ss += orow[j] * orow[j];
    const double inv = 1.0 / sqrt(ss / dv + eps);
    for (int j = 0; j < dv; ++j) y[r * dv + j] = orow[j] * inv * w[j] * sigmoid(z[r * dv + j]);
  }
  return 0;
}
