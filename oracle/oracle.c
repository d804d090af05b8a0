/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY. A plain, slow, fp64 CPU oracle of the
 * SketchSSM windowed linear-attention decode. Nothing in the product path may
 * load it: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no code, header or constant with the HIP library.
 *
 * Sources (the SketchSSM pages):
 *   [P1] readsearch.ai listing of arXiv 2609.33051, "SketchSSM: Write to the
 *        Full State, Read from a Compact Sketch", Abstract.
 *   [P2] agihunt.info news summary of SketchSSM, "Confirmed" bullets
 *        ("Mechanism details", "Error control").
 * The pages name the three recurrences (Mamba-2, Gated DeltaNet, KDA; [P1]
 * Abstract) but print no formula. Used here, as those model families define
 * them: Mamba-2 S <- a S + k v^T (scalar decay a); Gated DeltaNet
 * S <- alpha (I - beta k k^T) S + beta k v^T; KDA, the channel-wise gated
 * delta rule, read as S <- (I - beta k k^T) Diag(alpha) S + beta k v^T
 * (decay first, then the delta write). Within a window the state is not
 * written and only the queries change ([P2] "Mechanism details"), so the
 * state after tau buffered tokens is S_tau = A S_win + R with A the product of
 * the tokens' transition matrices; the query is carried back to the window
 * start as q~ = A^T q and projected on the basis, c = B q~ ([P1] Abstract:
 * outputs for fixed basis vectors are stored once per update, each step
 * combines them with query-dependent coefficients).
 *
 * What it computes, per (sequence, head) unit, independently:
 *   every token t:  M_t  = the token's transition matrix (d_k x d_k, dense)
 *                   S    <- M_t S + b_t k_t v_t^T          (b = beta, or 1 for Mamba-2)
 *                   A    <- M_t A,  R <- M_t R + b_t k_t v_t^T   (A = I, R = 0 at window start)
 *                   y_exact  = S^T q_t                       (full state after the token)
 *                   q~       = A^T q_t
 *                   c        = B q~                          (B holds the r basis rows)
 *                   y_sketch = Sk^T c + R^T q_t              (Sk = B S_win: the stored sketch)
 *                   y_replay = S_win^T q~ + R^T q_t          (exact read of the window-start state)
 *   every W tokens: S_win <- S, Sk <- B S_win, A <- I, R <- 0.
 * "R" is the additive part of the window decomposition (often written B_t);
 * it is renamed so that it does not clash with the basis B.
 *
 * Sketch storage. The pages do not fix the sketch's precision. With
 * sketch_bf16 set, every stored sketch element is rounded as a bf16 store
 * would round it: first to fp32 (the precision the sketch is computed in),
 * then to the nearest bf16 (8 significant bits), ties to the even neighbour.
 * y_sketch then reads the rounded sketch; nothing else changes.
 *
 * Every matrix is formed densely and multiplied with plain loops, in fp64.
 * Parity is pinned by tests/test_oracle_pins.py (closed forms, invariants and
 * brute force on tiny inputs).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_MAMBA2 = 0, ORACLE_GDN = 1, ORACLE_KDA = 2 };

/* M_t, the linear part of the token's state update S <- M_t S + b_t k v^T.
 *   Mamba-2: M = a I                         (scalar decay a)
 *   GDN:     M = alpha (I - beta k k^T)      (scalar gate alpha)
 *   KDA:     M = (I - beta k k^T) Diag(alpha) (per-channel gate alpha[d_k]) */
static void transition_matrix(int rule, int dk, const double* k, const double* decay,
                              double beta, double* M) {
  for (int i = 0; i < dk; ++i) {
    for (int j = 0; j < dk; ++j) {
      double eye = (i == j) ? 1.0 : 0.0;
      double m;
      if (rule == ORACLE_MAMBA2) {
        m = decay[0] * eye;
      } else if (rule == ORACLE_GDN) {
        m = decay[0] * (eye - beta * k[i] * k[j]);
      } else {
        m = (eye - beta * k[i] * k[j]) * decay[j];
      }
      M[i * dk + j] = m;
    }
  }
}

/* Weight of the rank-1 write k v^T: beta for the delta rules, 1 for Mamba-2. */
static double write_weight(int rule, double beta) {
  return rule == ORACLE_MAMBA2 ? 1.0 : beta;
}

/* out (n x p) = X (n x m) Y (m x p); out must not alias X or Y. */
static void matmul(int n, int m, int p, const double* X, const double* Y, double* out) {
  for (int i = 0; i < n; ++i) {
    for (int j = 0; j < p; ++j) out[i * p + j] = 0.0;
    for (int l = 0; l < m; ++l) {
      double x = X[i * m + l];
      for (int j = 0; j < p; ++j) out[i * p + j] += x * Y[l * p + j];
    }
  }
}

/* X (dk x ncols) <- M X + w k v^T  (v may be NULL: no additive term) */
static void apply_token(int dk, int ncols, const double* M, double* X, double* tmp,
                        double w, const double* k, const double* v) {
  matmul(dk, dk, ncols, M, X, tmp);
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < ncols; ++j)
      X[i * ncols + j] = tmp[i * ncols + j] + (v ? w * k[i] * v[j] : 0.0);
}

/* out[j] = sum_i X[i][j] q[i]   (X is n x p, so out = X^T q) */
static void transpose_times(int n, int p, const double* X, const double* q, double* out) {
  for (int j = 0; j < p; ++j) out[j] = 0.0;
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < p; ++j) out[j] += X[i * p + j] * q[i];
}

/* ------------------------------------------------------------------------- */
/* Exported helpers for the tests                                            */
/* ------------------------------------------------------------------------- */

/* M_t for one token; M is dk x dk row-major. */
void oracle_transition_matrix(int rule, int dk, const double* k, const double* decay,
                              double beta, double* M) {
  transition_matrix(rule, dk, k, decay, beta, M);
}

/* One token's state update, in place: S (dk x dv) <- M_t S + b_t k v^T. Returns 0. */
int oracle_rule_step(int rule, int dk, int dv, double* S, const double* k, const double* v,
                     const double* decay, double beta) {
  double* M = (double*)malloc(sizeof(double) * (size_t)dk * dk);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)dk * dv);
  if (!M || !tmp) { free(M); free(tmp); return 1; }
  transition_matrix(rule, dk, k, decay, beta, M);
  apply_token(dk, dv, M, S, tmp, write_weight(rule, beta), k, v);
  free(M);
  free(tmp);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* The windowed decode run                                                   */
/* x as a bf16 store keeps it: rounded to fp32, then to the nearest value with
 * 8 significant bits. Of the fp32 pattern, the high 16 bits are kept; the low
 * 16 decide: above half of the kept unit rounds up, below rounds down, exactly
 * half rounds to the neighbour whose kept pattern is even. Infinities stay;
 * a NaN stays a NaN. */
double oracle_round_bf16(double x) {
  float f = (float)x;
  if (isnan(f)) return x;
  uint32_t u;
  memcpy(&u, &f, sizeof(u));
  uint32_t kept = u >> 16, dropped = u & 0xFFFFu;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
  u = kept << 16;
  memcpy(&f, &u, sizeof(f));
  return (double)f;
}

static void round_sketch(size_t n, double* Sk) {
  for (size_t i = 0; i < n; ++i) Sk[i] = oracle_round_bf16(Sk[i]);
}

/* ------------------------------------------------------------------------- */
/*
 * rule      0 Mamba-2, 1 GDN, 2 KDA
 * U         number of independent units (sequence, head)
 * dk, dv    state is dk x dv; r = number of basis rows; W = window length
 * T         number of decode steps (tokens); a trailing partial window is not refreshed
 * S0        [U][dk][dv]          initial state (the state at the first window start)
 * basis     [U][r][dk]           the unit's basis rows b_m (orthonormal)
 * q, k      [T][U][dk]
 * v         [T][U][dv]
 * decay     [T][U] (Mamba-2 a, GDN alpha) or [T][U][dk] (KDA alpha)
 * beta      [T][U] (GDN, KDA); ignored (may be NULL) for Mamba-2
 * outputs (any may be NULL):
 * y_exact, y_replay, y_sketch   [T][U][dv]
 * S_out     [T/W + 1][U][dk][dv]  window-start states: S0, then the state after each full window
 * Sk_out    [T/W + 1][U][r][dv]   the sketch B S_win stored at each window start
 * A_out     [T][U][dk][dk]        A after each token (tiny shapes only)
 * R_out     [T][U][dk][dv]        R after each token (tiny shapes only)
 * qt_out    [T][U][dk]            q~ = A^T q of each step (the carried-back query)
 * sketch_bf16  non-zero: the stored sketch is rounded as a bf16 store rounds it
 * nthreads  OpenMP threads (<= 0: runtime default)
 * Returns 0, or 1 on allocation failure / bad arguments.
 */
int oracle_run(int rule, int U, int dk, int dv, int r, int W, int T,
               const double* S0, const double* basis,
               const double* q, const double* k, const double* v,
               const double* decay, const double* beta,
               double* y_exact, double* y_replay, double* y_sketch,
               double* S_out, double* Sk_out, double* A_out, double* R_out,
               double* qt_out, int sketch_bf16, int nthreads) {
  if (rule < 0 || rule > 2 || U < 0 || dk < 1 || dv < 1 || r < 1 || W < 1 || T < 0) return 1;
  if (rule != ORACLE_MAMBA2 && beta == NULL) return 1;
  const int dstride = (rule == ORACLE_KDA) ? dk : 1;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
  for (int u = 0; u < U; ++u) {
    size_t sz_s = (size_t)dk * dv, sz_a = (size_t)dk * dk, sz_k = (size_t)r * dv;
    double* S = (double*)malloc(sizeof(double) * sz_s);
    double* Swin = (double*)malloc(sizeof(double) * sz_s);
    double* A = (double*)malloc(sizeof(double) * sz_a);
    double* R = (double*)malloc(sizeof(double) * sz_s);
    double* M = (double*)malloc(sizeof(double) * sz_a);
    double* tmp = (double*)malloc(sizeof(double) * (sz_s > sz_a ? sz_s : sz_a));
    double* Sk = (double*)malloc(sizeof(double) * sz_k);
    double* qt = (double*)malloc(sizeof(double) * dk);
    double* c = (double*)malloc(sizeof(double) * r);
    double* y1 = (double*)malloc(sizeof(double) * dv);
    double* y2 = (double*)malloc(sizeof(double) * dv);
    if (!S || !Swin || !A || !R || !M || !tmp || !Sk || !qt || !c || !y1 || !y2) {
      failed = 1;
    } else {
      const double* Bu = basis + (size_t)u * r * dk;
      memcpy(S, S0 + (size_t)u * sz_s, sizeof(double) * sz_s);
      memcpy(Swin, S, sizeof(double) * sz_s);
      /* window start: A = I, R = 0, Sk = B S_win */
      for (size_t i = 0; i < sz_a; ++i) A[i] = 0.0;
      for (int i = 0; i < dk; ++i) A[i * dk + i] = 1.0;
      for (size_t i = 0; i < sz_s; ++i) R[i] = 0.0;
      matmul(r, dk, dv, Bu, Swin, Sk);
      if (sketch_bf16) round_sketch(sz_k, Sk);
      if (S_out) memcpy(S_out + (size_t)u * sz_s, Swin, sizeof(double) * sz_s);
      if (Sk_out) memcpy(Sk_out + (size_t)u * sz_k, Sk, sizeof(double) * sz_k);
      int tau = 0, win = 0;
      for (int t = 0; t < T; ++t) {
        size_t tu = (size_t)t * U + u;
        const double* qv = q + tu * dk;
        const double* kv = k + tu * dk;
        const double* vv = v + tu * dv;
        const double* dv_ = decay + tu * dstride;
        double b = (rule == ORACLE_MAMBA2) ? 0.0 : beta[tu];
        double w = write_weight(rule, b);
        transition_matrix(rule, dk, kv, dv_, b, M);
        apply_token(dk, dv, M, S, tmp, w, kv, vv);   /* sequential recurrence */
        apply_token(dk, dk, M, A, tmp, w, kv, NULL); /* A <- M A */
        apply_token(dk, dv, M, R, tmp, w, kv, vv);   /* R <- M R + w k v^T */
        tau += 1;
        if (A_out) memcpy(A_out + tu * sz_a, A, sizeof(double) * sz_a);
        if (R_out) memcpy(R_out + tu * sz_s, R, sizeof(double) * sz_s);
        /* exact read of the full state */
        if (y_exact) transpose_times(dk, dv, S, qv, y_exact + tu * dv);
        /* q~ = A^T q ; c = B q~ ; intra = R^T q */
        transpose_times(dk, dk, A, qv, qt);
        if (qt_out) memcpy(qt_out + tu * dk, qt, sizeof(double) * dk);
        for (int m = 0; m < r; ++m) {
          double acc = 0.0;
          for (int i = 0; i < dk; ++i) acc += Bu[(size_t)m * dk + i] * qt[i];
          c[m] = acc;
        }
        transpose_times(dk, dv, R, qv, y1);
        if (y_sketch) {
          transpose_times(r, dv, Sk, c, y2);
          for (int j = 0; j < dv; ++j) y_sketch[tu * dv + j] = y2[j] + y1[j];
        }
        if (y_replay) {
          transpose_times(dk, dv, Swin, qt, y2);
          for (int j = 0; j < dv; ++j) y_replay[tu * dv + j] = y2[j] + y1[j];
        }
        if (tau == W) { /* window end: write-back point of the full state, refresh */
          memcpy(Swin, S, sizeof(double) * sz_s);
          matmul(r, dk, dv, Bu, Swin, Sk);
          if (sketch_bf16) round_sketch(sz_k, Sk);
          for (size_t i = 0; i < sz_a; ++i) A[i] = 0.0;
          for (int i = 0; i < dk; ++i) A[i * dk + i] = 1.0;
          for (size_t i = 0; i < sz_s; ++i) R[i] = 0.0;
          tau = 0;
          win += 1;
          if (S_out) memcpy(S_out + ((size_t)win * U + u) * sz_s, Swin, sizeof(double) * sz_s);
          if (Sk_out) memcpy(Sk_out + ((size_t)win * U + u) * sz_k, Sk, sizeof(double) * sz_k);
        }
      }
    }
    free(S); free(Swin); free(A); free(R); free(M); free(tmp); free(Sk);
    free(qt); free(c); free(y1); free(y2);
  }
  return failed ? 1 : 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
