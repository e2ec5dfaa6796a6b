/*
 * gdn_oracle.c -- plain fp64 CPU oracle of the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only users.  It shares no code, header,
 * table or helper with the GPU library, and neither side includes the other.
 *
 * What is computed, per (row r, value head h), the qk-head being
 * hq = h / (H_v / H_qk) (contiguous groups of value heads share one q/k head):
 *
 *   gates   x_t     = a_t + dt_bias[h]
 *           g_t     = -exp(A_log[h]) * softplus(x_t),  softplus(x) = log(1 + e^x)
 *           alpha_t = exp(g_t),   beta_t = 1 / (1 + exp(-b_t))
 *   state   S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *           (S is d_v x d_k; S q and v k^T then type-check)
 *   output  o_t = S_t q_t  (the state after token t's update)
 *
 * The recurrence and gate form are the gated delta rule of Yang, Kautz and
 * Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta Rule"
 * (ICLR 2025), eq. for the gated delta rule and its Mamba2-style decay gate.
 * The surrounding behaviour follows the pages on native three-step MTP
 * ("Native three-step MTP", section "What changed": fp32 sigmoid gates and a
 * GDN state update rounded alike in decode and verification) and the
 * onnxruntime-genai pull request "Run chained MTP drafting in the batch Engine"
 * (section "Correctness fix": drafts are rejected by restoring intermediate
 * recurrent checkpoints; a chunked GatedDeltaNet form handles long prefills).
 *
 * Two entry points compute the same function in two ways:
 *   gdn_oracle_sequential -- the definition, one token at a time;
 *   gdn_oracle_chunked    -- the chunkwise UT/WY form of Yang et al.,
 *     "Parallelizing Linear Transformers with the Delta Rule over Sequence
 *     Length" (NeurIPS 2024), sec. 3 (chunkwise parallel form), with the decay
 *     of the gated variant; used to pin the sequential form and vice versa.
 *
 * Packed ragged batch layout (all arrays host, row-major, fp64):
 *   rows are packed in order, a row's tokens in time order; row r owns tokens
 *   [cu_r, cu_r + L_r), cu_r = sum of the earlier rows' L.
 *   q, k    [N][H_qk][d_k]      v     [N][H_v][d_v]      a, b [N][H_v]
 *   A_log, dt_bias [H_v]
 *   S0      [B][H_v][d_v][d_k]  start state of each row (read only)
 *   S_final [B][H_v][d_v][d_k]  state after the row's last token (also the work
 *           buffer of the sequential form)
 *   ckpt    [B][n_slot][H_v][d_v][d_k]: slot j of row r holds the state after
 *           L_r - n_tail_r + j + 1 tokens, for j < n_tail_r <= min(L_r, n_slot);
 *           the other slots are not written (ckpt may be NULL if all n_tail are 0)
 *   o       [N][H_v][d_v]
 * Return 0, or -1 on a bad argument (nothing written).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads_used = 1;

/* Number of OpenMP threads the last call ran with. */
int gdn_oracle_threads_used(void) { return g_threads_used; }

static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

static double log_decay(double a, double A_log, double dt_bias) {
  return -exp(A_log) * softplus(a + dt_bias);
}

/* alpha_i, beta_i of n (token) gate logits of one head. */
void gdn_oracle_gates(int n, const double *a, const double *b, double A_log,
                      double dt_bias, double *alpha, double *beta) {
  for (int i = 0; i < n; ++i) {
    alpha[i] = exp(log_decay(a[i], A_log, dt_bias));
    beta[i] = 1.0 / (1.0 + exp(-b[i]));
  }
}

static int check_rows(int B, int Hqk, int Hv, int dk, int dv, const int *L,
                      const int *n_tail, int n_slot) {
  if (B < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hqk) return -1;
  for (int r = 0; r < B; ++r) {
    if (L[r] < 0) return -1;
    int nt = n_tail ? n_tail[r] : 0;
    if (nt < 0 || nt > L[r] || nt > n_slot) return -1;
  }
  return 0;
}

static void record_threads(void) {
#ifdef _OPENMP
  g_threads_used = omp_get_num_threads();
#else
  g_threads_used = 1;
#endif
}

int gdn_oracle_sequential(int B, int Hqk, int Hv, int dk, int dv, const int *L,
                          const int *n_tail, int n_slot, const double *q,
                          const double *k, const double *v, const double *a,
                          const double *b, const double *A_log,
                          const double *dt_bias, const double *S0,
                          double *S_final, double *ckpt, double *o,
                          int n_threads) {
  if (check_rows(B, Hqk, Hv, dk, dv, L, n_tail, n_slot) || !S_final) return -1;
  long *cu = malloc(sizeof(long) * (B + 1));
  cu[0] = 0;
  for (int r = 0; r < B; ++r) cu[r + 1] = cu[r] + L[r];
  const int group = Hv / Hqk;
  const long unit_sz = (long)dv * dk;
  if (n_threads <= 0) n_threads = 1;

#pragma omp parallel for num_threads(n_threads) schedule(dynamic)
  for (long unit = 0; unit < (long)B * Hv; ++unit) {
    if (unit == 0) record_threads();
    const int r = (int)(unit / Hv), h = (int)(unit % Hv), hq = h / group;
    double *S = S_final + unit * unit_sz; /* the state evolves in place in S_final */
    double *u = malloc(sizeof(double) * dv);
    memcpy(S, S0 + unit * unit_sz, sizeof(double) * unit_sz);
    const int nt = n_tail ? n_tail[r] : 0;
    for (int t = 0; t < L[r]; ++t) {
      const long tok = cu[r] + t;
      const double *kt = k + (tok * Hqk + hq) * dk;
      const double *qt = q + (tok * Hqk + hq) * dk;
      const double *vt = v + (tok * Hv + h) * dv;
      double alpha, beta;
      gdn_oracle_gates(1, a + tok * Hv + h, b + tok * Hv + h, A_log[h], dt_bias[h],
                       &alpha, &beta);
      /* u = S k, so that S (I - beta k k^T) = S - beta u k^T */
      for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[i * dk + j] * kt[j];
        u[i] = acc;
      }
      for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j)
          S[i * dk + j] = alpha * (S[i * dk + j] - beta * u[i] * kt[j]) +
                          beta * vt[i] * kt[j];
      double *ot = o + (tok * Hv + h) * dv;
      for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[i * dk + j] * qt[j];
        ot[i] = acc;
      }
      const int slot = t - (L[r] - nt);
      if (slot >= 0)
        memcpy(ckpt + (((long)r * n_slot + slot) * Hv + h) * unit_sz, S,
               sizeof(double) * unit_sz);
    }
    free(u);
  }
  free(cu);
  return 0;
}

/*
 * Chunkwise form.  Within a chunk of C tokens starting from state S_c, with
 * G_t = g_1 + ... + g_t (log-space cumulative decay, 1-based t) and the written
 * value u_t = beta_t (v_t - alpha_t S_{t-1} k_t):
 *   S_t = e^{G_t} S_c + sum_{s<=t} e^{G_t - G_s} u_s k_s^T
 * Stacking u_t^T as the rows of U (C x d_v) gives the unit lower-triangular
 * system (I + A) U = diag(beta) V - diag(beta e^G) K S_c^T with
 *   A_ts = beta_t e^{G_t - G_s} k_t . k_s  (s < t),  so with T = (I + A)^{-1}:
 *   W = T diag(beta e^G) K,  U' = T diag(beta) V,  U = U' - W S_c^T
 *   O = diag(e^G) Q S_c^T + (Gamma o Q K^T) U,  Gamma_ts = e^{G_t - G_s} (s <= t)
 *   S_{c+1} = e^{G_C} S_c + U^T diag(e^{G_C - G}) K
 * Exponents are formed only as differences G_t - G_s with s <= t (never
 * positive), so nothing overflows however strong the decay.
 */
int gdn_oracle_chunked(int B, int Hqk, int Hv, int dk, int dv, const int *L,
                       const int *n_tail, int n_slot, int chunk, const double *q,
                       const double *k, const double *v, const double *a,
                       const double *b, const double *A_log,
                       const double *dt_bias, const double *S0, double *S_final,
                       double *ckpt, double *o, int n_threads) {
  if (check_rows(B, Hqk, Hv, dk, dv, L, n_tail, n_slot) || chunk <= 0) return -1;
  long *cu = malloc(sizeof(long) * (B + 1));
  cu[0] = 0;
  for (int r = 0; r < B; ++r) cu[r + 1] = cu[r] + L[r];
  const int group = Hv / Hqk;
  const long unit_sz = (long)dv * dk;
  const int C = chunk;
  if (n_threads <= 0) n_threads = 1;

#pragma omp parallel for num_threads(n_threads) schedule(dynamic)
  for (long unit = 0; unit < (long)B * Hv; ++unit) {
    if (unit == 0) record_threads();
    const int r = (int)(unit / Hv), h = (int)(unit % Hv), hq = h / group;
    double *S = malloc(sizeof(double) * unit_sz);
    double *Sn = malloc(sizeof(double) * unit_sz);
    double *G = malloc(sizeof(double) * C), *be = malloc(sizeof(double) * C);
    double *A = calloc((size_t)C * C, sizeof(double));
    double *T = calloc((size_t)C * C, sizeof(double));
    double *W = malloc(sizeof(double) * C * dk);
    double *U = malloc(sizeof(double) * C * dv);
    memcpy(S, S0 + unit * unit_sz, sizeof(double) * unit_sz);
    const int nt = n_tail ? n_tail[r] : 0;

    for (int c0 = 0; c0 < L[r]; c0 += C) {
      const int n = (L[r] - c0 < C) ? L[r] - c0 : C;
      const long tok0 = cu[r] + c0;
#define KT(t) (k + ((tok0 + (t)) * Hqk + hq) * dk)
#define QT(t) (q + ((tok0 + (t)) * Hqk + hq) * dk)
#define VT(t) (v + ((tok0 + (t)) * Hv + h) * dv)
      double run = 0.0;
      for (int t = 0; t < n; ++t) {
        const long tok = tok0 + t;
        run += log_decay(a[tok * Hv + h], A_log[h], dt_bias[h]);
        G[t] = run;
        be[t] = 1.0 / (1.0 + exp(-b[tok * Hv + h]));
      }
      /* A (strictly lower) and T = (I + A)^{-1} by forward substitution */
      for (int t = 0; t < n; ++t)
        for (int s = 0; s < t; ++s) {
          double kk = 0.0;
          for (int j = 0; j < dk; ++j) kk += KT(t)[j] * KT(s)[j];
          A[t * C + s] = be[t] * exp(G[t] - G[s]) * kk;
        }
      for (int t = 0; t < n; ++t)
        for (int j = 0; j < n; ++j) {
          double acc = (t == j) ? 1.0 : 0.0;
          for (int m = 0; m < t; ++m) acc -= A[t * C + m] * T[m * C + j];
          T[t * C + j] = acc;
        }
      /* W = T diag(beta e^G) K ;  U = T diag(beta) V - W S_c^T */
      for (int t = 0; t < n; ++t) {
        for (int j = 0; j < dk; ++j) {
          double acc = 0.0;
          for (int m = 0; m <= t; ++m) acc += T[t * C + m] * be[m] * exp(G[m]) * KT(m)[j];
          W[t * dk + j] = acc;
        }
        for (int i = 0; i < dv; ++i) {
          double acc = 0.0;
          for (int m = 0; m <= t; ++m) acc += T[t * C + m] * be[m] * VT(m)[i];
          double ws = 0.0;
          for (int j = 0; j < dk; ++j) ws += W[t * dk + j] * S[i * dk + j];
          U[t * dv + i] = acc - ws;
        }
      }
      /* O = diag(e^G) Q S_c^T + (Gamma o Q K^T) U */
      for (int t = 0; t < n; ++t) {
        double *ot = o + ((tok0 + t) * Hv + h) * dv;
        const double eg = exp(G[t]);
        for (int i = 0; i < dv; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dk; ++j) acc += S[i * dk + j] * QT(t)[j];
          ot[i] = eg * acc;
        }
        for (int s = 0; s <= t; ++s) {
          double qk = 0.0;
          for (int j = 0; j < dk; ++j) qk += QT(t)[j] * KT(s)[j];
          const double coef = exp(G[t] - G[s]) * qk;
          for (int i = 0; i < dv; ++i) ot[i] += coef * U[s * dv + i];
        }
      }
      /* checkpoints that fall in this chunk: S_t = e^{G_t} S_c + sum_{s<=t} e^{G_t-G_s} u_s k_s^T */
      for (int t = 0; t < n; ++t) {
        const int slot = (c0 + t) - (L[r] - nt);
        if (slot < 0) continue;
        double *dst = ckpt + (((long)r * n_slot + slot) * Hv + h) * unit_sz;
        for (int i = 0; i < dv; ++i)
          for (int j = 0; j < dk; ++j) {
            double acc = exp(G[t]) * S[i * dk + j];
            for (int s = 0; s <= t; ++s) acc += exp(G[t] - G[s]) * U[s * dv + i] * KT(s)[j];
            dst[i * dk + j] = acc;
          }
      }
      /* S_{c+1} = e^{G_n} S_c + U^T diag(e^{G_n - G}) K */
      for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j) {
          double acc = exp(G[n - 1]) * S[i * dk + j];
          for (int s = 0; s < n; ++s) acc += exp(G[n - 1] - G[s]) * U[s * dv + i] * KT(s)[j];
          Sn[i * dk + j] = acc;
        }
      memcpy(S, Sn, sizeof(double) * unit_sz);
#undef KT
#undef QT
#undef VT
    }
    if (S_final) memcpy(S_final + unit * unit_sz, S, sizeof(double) * unit_sz);
    free(S); free(Sn); free(G); free(be); free(A); free(T); free(W); free(U);
  }
  free(cu);
  return 0;
}
