/*
 * ckda_oracle.c -- plain sequential fp64 CPU oracle for the (Complex) Kimi
 * Delta Attention recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg load it.  It shares no source, header,
 * table or helper with the GPU library, and the GPU library never calls it.
 *
 * What it computes (one head, one sequence; heads are independent states that
 * receive the same layer input -- "Complex KDA" paper, App. B.2, paragraph
 * "Heads and layers"):
 *
 *   H_t = (I - beta_t k_t k_t^T) Diag(alpha_t) H_{t-1} + beta_t k_t v_t^T
 *   o_t = H_t^T q_t                       (read-out of the post-update state)
 *
 * ("Complex KDA" discussion slides, frame "CKDA keeps the original
 * gate--delta--readout structure", Eq. (1) of the paper; App. B.2, Eq. (9).)
 *
 * It is evaluated in the gate / read / compare / correct order of the KDA
 * course lesson (session 17, "Mechanism map" and "Worked case -- full trace",
 * part B):
 *
 *   Hbar = Diag(alpha_t) H_{t-1}          row i (key channel i) times alpha_t[i]
 *   s    = Hbar^T k_t                     the state's current prediction for k_t
 *   H_t  = Hbar + beta_t k_t (v_t - s)^T  delta correction
 *
 * which is the same matrix as the first form: (I - b k k^T) Hbar + b k v^T
 * = Hbar + b k (v - Hbar^T k)^T.  The state is n x d_v with row i = key
 * channel i.  No log-space, no sign handling, no chunking: alpha is applied
 * as the signed real number it is (negative and zero gates included: App. B.2
 * admits the closed ranges, their endpoints and zero gates among them).  No
 * query scaling and no key normalisation are applied; inputs are used exactly
 * as given (bf16 and fp32 inputs are widened exactly to fp64).
 *
 * Parallel only across the independent (batch, head) recurrences (OpenMP).
 *
 * Layouts (C order): q, k, alpha [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T];
 * h0 [B,H,dk,dv]; o [B,H,T,dv]; hT [B,H,dk,dv].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* Widen element i of a raw buffer of the given dtype to double (exact). */
static double widen(const void* base, long long i, int dtype) {
  if (dtype == ORACLE_F64) return ((const double*)base)[i];
  if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
  /* bf16: the upper 16 bits of an IEEE binary32 */
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int valid_dtype(int d) { return d == ORACLE_F32 || d == ORACLE_BF16 || d == ORACLE_F64; }

/* One recurrence step on a dk x dv fp64 state S (row-major, row = key channel).
 * a, kk, qq: length dk; vv: length dv; s: scratch length dv; out: length dv. */
static void step(double* S, const double* a, const double* kk, const double* qq,
                 const double* vv, double b, double* s, double* out, int dk, int dv) {
  /* gate: Hbar = Diag(alpha) H */
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(long)i * dv + j] *= a[i];
  /* read: s = Hbar^T k */
  for (int j = 0; j < dv; ++j) s[j] = 0.0;
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) s[j] += S[(long)i * dv + j] * kk[i];
  /* correct: H = Hbar + beta k (v - s)^T */
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += b * kk[i] * (vv[j] - s[j]);
  /* query the updated state: o = H^T q */
  if (out) {
    for (int j = 0; j < dv; ++j) out[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) out[j] += S[(long)i * dv + j] * qq[i];
  }
}

/* Full-sequence forward.  h0 may be NULL (zero initial state); its dtype is
 * h0_dtype (F32 or F64).  o may be NULL (outputs not wanted); hT may be NULL.
 * Returns 0 on success, nonzero on bad arguments or allocation failure. */
int ckda_oracle_fwd(const void* q, const void* k, const void* v, const void* alpha,
                    const void* beta, int dtype, const void* h0, int h0_dtype,
                    double* o, double* hT, int B, int H, int T, int dk, int dv,
                    int nthreads) {
  if (!q || !k || !v || !alpha || !beta) return 1;
  if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return 2;
  if (!valid_dtype(dtype) || (h0 && !valid_dtype(h0_dtype))) return 3;
  long long BH = (long long)B * H;
  int failed = 0;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed) num_threads(nt)
#else
  (void)nthreads;
#endif
  for (long long bh = 0; bh < BH; ++bh) {
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* buf = (double*)malloc(sizeof(double) * (size_t)(3 * dk + 3 * dv));
    if (!S || !buf) { free(S); free(buf); failed |= 1; continue; }
    double *a = buf, *kk = a + dk, *qq = kk + dk, *vv = qq + dk, *s = vv + dv, *ot = s + dv;
    long long sbase = bh * (long long)dk * dv;
    for (long long e = 0; e < (long long)dk * dv; ++e)
      S[e] = h0 ? widen(h0, sbase + e, h0_dtype) : 0.0;
    for (int t = 0; t < T; ++t) {
      long long tk = (bh * T + t) * (long long)dk, tv = (bh * T + t) * (long long)dv;
      for (int i = 0; i < dk; ++i) {
        a[i] = widen(alpha, tk + i, dtype);
        kk[i] = widen(k, tk + i, dtype);
        qq[i] = widen(q, tk + i, dtype);
      }
      for (int j = 0; j < dv; ++j) vv[j] = widen(v, tv + j, dtype);
      double b = widen(beta, bh * T + t, dtype);
      step(S, a, kk, qq, vv, b, s, o ? ot : NULL, dk, dv);
      if (o) memcpy(o + tv, ot, sizeof(double) * dv);
    }
    if (hT) memcpy(hT + sbase, S, sizeof(double) * (size_t)dk * dv);
    free(S);
    free(buf);
  }
  return failed ? 4 : 0;
}

/* Single-token step for N sequences x H heads, state updated in place.
 * q, k, alpha [N,H,dk]; v [N,H,dv]; beta [N,H]; S_inout [N,H,dk,dv] fp64;
 * o [N,H,dv] fp64 (may be NULL).  Applies exactly the step above. */
int ckda_oracle_decode(const void* q, const void* k, const void* v, const void* alpha,
                       const void* beta, int dtype, double* S_inout, double* o,
                       int N, int H, int dk, int dv, int nthreads) {
  if (!q || !k || !v || !alpha || !beta || !S_inout) return 1;
  if (N < 0 || H < 0 || dk <= 0 || dv <= 0) return 2;
  if (!valid_dtype(dtype)) return 3;
  long long NH = (long long)N * H;
  int failed = 0;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(static) reduction(| : failed) num_threads(nt)
#else
  (void)nthreads;
#endif
  for (long long nh = 0; nh < NH; ++nh) {
    double* buf = (double*)malloc(sizeof(double) * (size_t)(3 * dk + 3 * dv));
    if (!buf) { failed |= 1; continue; }
    double *a = buf, *kk = a + dk, *qq = kk + dk, *vv = qq + dk, *s = vv + dv, *ot = s + dv;
    for (int i = 0; i < dk; ++i) {
      a[i] = widen(alpha, nh * dk + i, dtype);
      kk[i] = widen(k, nh * dk + i, dtype);
      qq[i] = widen(q, nh * dk + i, dtype);
    }
    for (int j = 0; j < dv; ++j) vv[j] = widen(v, nh * dv + j, dtype);
    double b = widen(beta, nh, dtype);
    step(S_inout + nh * (long long)dk * dv, a, kk, qq, vv, b, s, o ? ot : NULL, dk, dv);
    if (o) memcpy(o + nh * dv, ot, sizeof(double) * dv);
    free(buf);
  }
  return failed ? 4 : 0;
}

int ckda_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------- prologue
 *
 * The practical gate and key parameterisation of the "Complex KDA" discussion
 * slides (frame "Backup: practical gates differ from exact theoretical
 * endpoints"; paper App. E--G.1), applied per token before the recurrence:
 *
 *   r = tanh(a / 2),  s = +1 if r >= 0 else -1,
 *   alpha = s (eps + (1 - eps) |r|),  eps = e^-5,       so log|alpha| in [-5, 0]
 *   beta  = 2 sigma(b),
 *
 * and keys (optionally queries) scaled to unit Euclidean norm per token (the
 * recurrence assumes ||k_t|| = 1; slides, frame "Absorb cumulative signs into
 * keys and queries", fuses the sign application with this normalisation).
 * The pages give no guard for a zero vector; here x / sqrt(sum x^2 + 1e-6),
 * which maps a zero vector to zero and changes a unit vector by 5e-7.
 *
 * Flags: 1 = alpha and beta arguments are the logits a and b; 2 = normalise k;
 * 4 = normalise q.  A step whose flag is off copies its input (widened).
 * Layouts: a, k, q [ntok, dk]; b [ntok]; outputs fp64 of the same shapes.
 * Returns 0, or 1 for invalid arguments. */
#define PRO_GATES 1
#define PRO_NORM_K 2
#define PRO_NORM_Q 4

static double practical_alpha(double a) {
  const double eps = exp(-5.0);
  const double r = tanh(0.5 * a);
  const double s = r >= 0.0 ? 1.0 : -1.0;
  return s * (eps + (1.0 - eps) * fabs(r));
}

static double practical_beta(double b) { return 2.0 / (1.0 + exp(-b)); }

static void unit_rows(const void* x, int dtype, long long ntok, int dk, int on, double* out) {
  for (long long t = 0; t < ntok; ++t) {
    double ss = 0.0;
    for (int i = 0; i < dk; ++i) {
      const double e = widen(x, t * dk + i, dtype);
      out[t * dk + i] = e;
      ss += e * e;
    }
    if (on) {
      const double inv = 1.0 / sqrt(ss + 1e-6);
      for (int i = 0; i < dk; ++i) out[t * dk + i] *= inv;
    }
  }
}

int ckda_oracle_prologue(const void* a, const void* b, const void* k, const void* q, int dtype, int flags,
                         long long ntok, int dk, double* alpha, double* beta, double* kk, double* qq) {
  if (!valid_dtype(dtype) || ntok < 0 || dk <= 0 || (flags & ~7) != 0) return 1;
  for (long long i = 0; i < ntok * dk; ++i) {
    const double e = widen(a, i, dtype);
    alpha[i] = (flags & PRO_GATES) ? practical_alpha(e) : e;
  }
  for (long long t = 0; t < ntok; ++t) {
    const double e = widen(b, t, dtype);
    beta[t] = (flags & PRO_GATES) ? practical_beta(e) : e;
  }
  unit_rows(k, dtype, ntok, dk, flags & PRO_NORM_K, kk);
  unit_rows(q, dtype, ntok, dk, flags & PRO_NORM_Q, qq);
  return 0;
}

/* Reverse mode of the prologue: given the gradients of a loss with respect
 * to its outputs (dalpha, dkk, dqq [ntok, dk] and dbeta [ntok], fp64), the
 * gradients with respect to its inputs (da, dk_raw, dq_raw [ntok, dk] and
 * db [ntok], fp64).  The gate follows the backward convention of the same
 * slide frame ("Backup: practical gates differ from exact theoretical
 * endpoints"): the sign s is held constant and |r| takes the zero subgradient
 * at r = 0, so
 *   d alpha / d a = s (1 - eps) d|r|/da,   d|r|/da = sign(r) (1 - r^2) / 2 for r != 0, 0 at r = 0;
 *   d beta / d b = 2 sigma(b) (1 - sigma(b));
 * a normalised row y = x n, n = (sum x^2 + 1e-6)^-1/2, passes back
 *   dx = n dy - n^3 x (x . dy)
 * (the Jacobian of y is n I - n^3 x x^T).  A step whose flag is off passes its
 * gradient through.  Returns 0, or 1 for invalid arguments. */
static double practical_alpha_slope(double a) {
  const double eps = exp(-5.0);
  const double r = tanh(0.5 * a);
  const double s = r >= 0.0 ? 1.0 : -1.0;   /* held constant */
  const double dabs = r > 0.0 ? 0.5 * (1.0 - r * r) : r < 0.0 ? -0.5 * (1.0 - r * r) : 0.0;
  return s * (1.0 - eps) * dabs;
}

static double practical_beta_slope(double b) {
  const double sg = 1.0 / (1.0 + exp(-b));
  return 2.0 * sg * (1.0 - sg);
}

static void unit_rows_bwd(const void* x, int dtype, long long ntok, int dk, int on, const double* dy, double* dx) {
  for (long long t = 0; t < ntok; ++t) {
    if (!on) {
      for (int i = 0; i < dk; ++i) dx[t * dk + i] = dy[t * dk + i];
      continue;
    }
    double ss = 0.0, xdy = 0.0;
    for (int i = 0; i < dk; ++i) {
      const double e = widen(x, t * dk + i, dtype);
      ss += e * e;
      xdy += e * dy[t * dk + i];
    }
    const double n = 1.0 / sqrt(ss + 1e-6);
    for (int i = 0; i < dk; ++i) dx[t * dk + i] = n * dy[t * dk + i] - n * n * n * widen(x, t * dk + i, dtype) * xdy;
  }
}

int ckda_oracle_prologue_bwd(const void* a, const void* b, const void* k, const void* q, int dtype, int flags,
                             long long ntok, int dk, const double* dalpha, const double* dbeta, const double* dkk,
                             const double* dqq, double* da, double* db, double* dk_raw, double* dq_raw) {
  if (!valid_dtype(dtype) || ntok < 0 || dk <= 0 || (flags & ~7) != 0) return 1;
  for (long long i = 0; i < ntok * dk; ++i)
    da[i] = (flags & PRO_GATES) ? dalpha[i] * practical_alpha_slope(widen(a, i, dtype)) : dalpha[i];
  for (long long t = 0; t < ntok; ++t)
    db[t] = (flags & PRO_GATES) ? dbeta[t] * practical_beta_slope(widen(b, t, dtype)) : dbeta[t];
  unit_rows_bwd(k, dtype, ntok, dk, flags & PRO_NORM_K, dkk, dk_raw);
  unit_rows_bwd(q, dtype, ntok, dk, flags & PRO_NORM_Q, dqq, dq_raw);
  return 0;
}

/* ---------------------------------------------------------------- DeltaProduct_2
 *
 * The DeltaProduct_2 comparator of the "Complex KDA" paper (Fig. 5 and the
 * implementation paragraph of Sec. 6: two delta-rule updates per token,
 * ungated there; App. C, "Consequences for CKDA and Gated DeltaProduct": the
 * gated form scales the product of the per-token Householder factors
 * (I - beta_j k_j k_j^T), j = 1, 2, by one scalar gate alpha_t).  Per token:
 *
 *   H <- alpha_t H                                  (omitted when ungated)
 *   for j = 1, 2:  H <- (I - beta_tj k_tj k_tj^T) H + beta_tj k_tj v_tj^T
 *   o_t = H^T q_t
 *
 * The additive term of each sub-step follows its own Householder factor, as
 * in a delta-rule update (the reading of "two delta-rule updates per token").
 * Layouts: q [B,H,T,dk]; k [B,H,T,2,dk]; v [B,H,T,2,dv]; beta [B,H,T,2];
 * alpha [B,H,T] or NULL; h0/hT [B,H,dk,dv]; o [B,H,T,dv]. */

/* H <- (I - b k k^T) H + b k v^T, with the Householder factor applied as
 * H - b k (k^T H).  w: scratch of length dv. */
static void householder_write(double* S, const double* kk, const double* vv, double b, double* w, int dk, int dv) {
  for (int j = 0; j < dv; ++j) w[j] = 0.0;
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) w[j] += kk[i] * S[(long)i * dv + j];
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += b * kk[i] * (vv[j] - w[j]);
}

static void dp2_token(double* S, const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                      int dtype, long long tok, int dk, int dv, double* buf, double* out) {
  double *kk = buf, *qq = kk + dk, *vv = qq + dk, *w = vv + dv;
  if (alpha) {
    const double a = widen(alpha, tok, dtype);
    for (long long e = 0; e < (long long)dk * dv; ++e) S[e] *= a;
  }
  for (int j = 0; j < 2; ++j) {
    for (int i = 0; i < dk; ++i) kk[i] = widen(k, (tok * 2 + j) * dk + i, dtype);
    for (int c = 0; c < dv; ++c) vv[c] = widen(v, (tok * 2 + j) * dv + c, dtype);
    householder_write(S, kk, vv, widen(beta, tok * 2 + j, dtype), w, dk, dv);
  }
  if (out) {
    for (int i = 0; i < dk; ++i) qq[i] = widen(q, tok * dk + i, dtype);
    for (int c = 0; c < dv; ++c) out[c] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int c = 0; c < dv; ++c) out[c] += S[(long)i * dv + c] * qq[i];
  }
}

int ckda_oracle_deltaproduct2(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                              int dtype, const void* h0, int h0_dtype, double* o, double* hT, int B, int H, int T,
                              int dk, int dv, int nthreads) {
  if (!q || !k || !v || !beta) return 1;
  if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return 2;
  if (!valid_dtype(dtype) || (h0 && !valid_dtype(h0_dtype))) return 3;
  long long BH = (long long)B * H;
  int failed = 0;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed) num_threads(nt)
#else
  (void)nthreads;
#endif
  for (long long bh = 0; bh < BH; ++bh) {
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* buf = (double*)malloc(sizeof(double) * (size_t)(2 * dk + 3 * dv));
    if (!S || !buf) { free(S); free(buf); failed |= 1; continue; }
    long long sbase = bh * (long long)dk * dv;
    for (long long e = 0; e < (long long)dk * dv; ++e) S[e] = h0 ? widen(h0, sbase + e, h0_dtype) : 0.0;
    for (int t = 0; t < T; ++t) {
      const long long tok = bh * T + t;
      dp2_token(S, q, k, v, alpha, beta, dtype, tok, dk, dv, buf, o ? o + tok * dv : NULL);
    }
    if (hT) memcpy(hT + sbase, S, sizeof(double) * (size_t)dk * dv);
    free(S);
    free(buf);
  }
  return failed ? 4 : 0;
}

/* One DeltaProduct_2 token for N sequences x H heads, fp64 state in place.
 * q [N,H,dk]; k [N,H,2,dk]; v [N,H,2,dv]; beta [N,H,2]; alpha [N,H] or NULL. */
int ckda_oracle_deltaproduct2_decode(const void* q, const void* k, const void* v, const void* alpha,
                                     const void* beta, int dtype, double* S_inout, double* o, int N, int H, int dk,
                                     int dv) {
  if (!q || !k || !v || !beta || !S_inout) return 1;
  if (N < 0 || H < 0 || dk <= 0 || dv <= 0) return 2;
  if (!valid_dtype(dtype)) return 3;
  double* buf = (double*)malloc(sizeof(double) * (size_t)(2 * dk + 3 * dv));
  if (!buf) return 4;
  for (long long nh = 0; nh < (long long)N * H; ++nh)
    dp2_token(S_inout + nh * (long long)dk * dv, q, k, v, alpha, beta, dtype, nh, dk, dv, buf,
              o ? o + nh * dv : NULL);
  free(buf);
  return 0;
}

/* ---------------------------------------------------------------- backward
 *
 * Reverse-mode derivative of the forward above for a loss L whose gradients
 * with respect to the outputs are do = dL/do_t and dhT = dL/dH_T: returns
 * dq, dk, dv, dalpha, dbeta (all per token, like their inputs) and dh0.
 * Written from the step itself (paper Eq. (1), in the course's order:
 * Hbar = Diag(alpha) H_{t-1}, s = Hbar^T k, u = beta (v - s),
 * H_t = Hbar + k u^T, o_t = H_t^T q), differentiated line by line in
 * reverse, with G = dL/dH_t carried from the end of the sequence:
 *
 *   G    += q do^T          dq = H_t do
 *   dk    = G u             du = G^T k
 *   dbeta = du . (v - s)    dv = beta du       ds = -beta du
 *   dHbar = G + k ds^T      dk += Hbar ds
 *   dalpha_i = sum_j dHbar_ij H_{t-1,ij}       G <- Diag(alpha) dHbar
 *
 * and dh0 = G after the first token.  The gate enters as the signed number
 * it is: dalpha is the plain partial derivative (no log space, no sign
 * convention, exact at zero gates).  States are kept at checkpoints every
 * `seg` tokens and recomputed one segment at a time in reverse.
 * Layouts as ckda_oracle_fwd; do [B,H,T,dv] (may be NULL: zero), dhT
 * [B,H,dk,dv] (may be NULL: zero); all outputs fp64. */
int ckda_oracle_bwd(const void* q, const void* k, const void* v, const void* alpha, const void* beta, int dtype,
                    const void* h0, int h0_dtype, const void* dout, const void* dhT, int g_dtype, double* dq,
                    double* dk, double* dv_, double* dalpha, double* dbeta, double* dh0, int B, int H, int T, int dk_,
                    int dv, int nthreads) {
  if (!q || !k || !v || !alpha || !beta || !dq || !dk || !dv_ || !dalpha || !dbeta || !dh0) return 1;
  if (B < 0 || H < 0 || T < 0 || dk_ <= 0 || dv <= 0) return 2;
  if (!valid_dtype(dtype) || (h0 && !valid_dtype(h0_dtype)) || !valid_dtype(g_dtype)) return 3;
  const int n = dk_, seg = 64;
  const long long NS = (long long)n * dv;
  long long BH = (long long)B * H;
  int failed = 0;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed) num_threads(nt)
#else
  (void)nthreads;
#endif
  for (long long bh = 0; bh < BH; ++bh) {
    const int nseg = (T + seg - 1) / seg;
    double* ck = (double*)malloc(sizeof(double) * (size_t)NS * (nseg + 1));   /* state at each segment start */
    double* st = (double*)malloc(sizeof(double) * (size_t)NS * (seg + 1));    /* states inside one segment */
    double* G = (double*)malloc(sizeof(double) * (size_t)NS);
    double* Hb = (double*)malloc(sizeof(double) * (size_t)NS);
    double* buf = (double*)malloc(sizeof(double) * (size_t)(3 * n + 6 * dv));
    if (!ck || !st || !G || !Hb || !buf) {
      free(ck); free(st); free(G); free(Hb); free(buf);
      failed |= 1;
      continue;
    }
    double *a = buf, *kk = a + n, *qq = kk + n, *vv = qq + n, *s = vv + dv, *u = s + dv, *gd = u + dv, *du = gd + dv,
           *ds = du + dv;
    const long long sbase = bh * NS;
    /* forward: checkpoints */
    for (long long e = 0; e < NS; ++e) ck[e] = h0 ? widen(h0, sbase + e, h0_dtype) : 0.0;
    for (int g = 0; g < nseg; ++g) {
      double* S = ck + (long long)(g + 1) * NS;
      memcpy(S, ck + (long long)g * NS, sizeof(double) * NS);
      for (int t = g * seg; t < T && t < (g + 1) * seg; ++t) {
        const long long tk = (bh * T + t) * (long long)n, tv = (bh * T + t) * (long long)dv;
        for (int i = 0; i < n; ++i) { a[i] = widen(alpha, tk + i, dtype); kk[i] = widen(k, tk + i, dtype); }
        for (int j = 0; j < dv; ++j) vv[j] = widen(v, tv + j, dtype);
        step(S, a, kk, kk, vv, widen(beta, bh * T + t, dtype), s, NULL, n, dv);
      }
    }
    /* reverse */
    for (long long e = 0; e < NS; ++e) G[e] = dhT ? widen(dhT, sbase + e, g_dtype) : 0.0;
    for (int g = nseg - 1; g >= 0; --g) {
      const int t0 = g * seg, t1 = (t0 + seg < T) ? t0 + seg : T;
      memcpy(st, ck + (long long)g * NS, sizeof(double) * NS);   /* st[0] = H_{t0-1} */
      for (int t = t0; t < t1; ++t) {
        const long long tk = (bh * T + t) * (long long)n, tv = (bh * T + t) * (long long)dv;
        double* S = st + (long long)(t - t0 + 1) * NS;
        memcpy(S, S - NS, sizeof(double) * NS);
        for (int i = 0; i < n; ++i) { a[i] = widen(alpha, tk + i, dtype); kk[i] = widen(k, tk + i, dtype); }
        for (int j = 0; j < dv; ++j) vv[j] = widen(v, tv + j, dtype);
        step(S, a, kk, kk, vv, widen(beta, bh * T + t, dtype), s, NULL, n, dv);
      }
      for (int t = t1 - 1; t >= t0; --t) {
        const long long tk = (bh * T + t) * (long long)n, tv = (bh * T + t) * (long long)dv;
        const double* Hp = st + (long long)(t - t0) * NS;       /* H_{t-1} */
        const double* Ht = Hp + NS;                             /* H_t */
        for (int i = 0; i < n; ++i) {
          a[i] = widen(alpha, tk + i, dtype);
          kk[i] = widen(k, tk + i, dtype);
          qq[i] = widen(q, tk + i, dtype);
        }
        for (int j = 0; j < dv; ++j) { vv[j] = widen(v, tv + j, dtype); gd[j] = dout ? widen(dout, tv + j, g_dtype) : 0.0; }
        const double b = widen(beta, bh * T + t, dtype);
        /* recompute Hbar, s, u */
        for (int i = 0; i < n; ++i)
          for (int j = 0; j < dv; ++j) Hb[(long)i * dv + j] = a[i] * Hp[(long)i * dv + j];
        for (int j = 0; j < dv; ++j) s[j] = 0.0;
        for (int i = 0; i < n; ++i)
          for (int j = 0; j < dv; ++j) s[j] += Hb[(long)i * dv + j] * kk[i];
        for (int j = 0; j < dv; ++j) u[j] = b * (vv[j] - s[j]);
        /* o_t = H_t^T q */
        for (int i = 0; i < n; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += Ht[(long)i * dv + j] * gd[j];
          dq[tk + i] = acc;
          for (int j = 0; j < dv; ++j) G[(long)i * dv + j] += qq[i] * gd[j];
        }
        /* H_t = Hbar + k u^T */
        for (int j = 0; j < dv; ++j) du[j] = 0.0;
        for (int i = 0; i < n; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) { acc += G[(long)i * dv + j] * u[j]; du[j] += G[(long)i * dv + j] * kk[i]; }
          dk[tk + i] = acc;
        }
        /* u = beta (v - s) */
        double db = 0.0;
        for (int j = 0; j < dv; ++j) {
          db += du[j] * (vv[j] - s[j]);
          dv_[tv + j] = b * du[j];
          ds[j] = -b * du[j];
        }
        dbeta[bh * T + t] = db;
        /* s = Hbar^T k;  Hbar = Diag(alpha) H_{t-1} */
        for (int i = 0; i < n; ++i) {
          double acc = 0.0, ga = 0.0;
          for (int j = 0; j < dv; ++j) {
            acc += Hb[(long)i * dv + j] * ds[j];
            const double dhb = G[(long)i * dv + j] + kk[i] * ds[j];
            ga += dhb * Hp[(long)i * dv + j];
            G[(long)i * dv + j] = a[i] * dhb;
          }
          dk[tk + i] += acc;
          dalpha[tk + i] = ga;
        }
      }
    }
    memcpy(dh0 + sbase, G, sizeof(double) * NS);
    free(ck); free(st); free(G); free(Hb); free(buf);
  }
  return failed ? 4 : 0;
}

/* ---------------------------------------------------------------- DeltaProduct_2 backward
 *
 * Reverse-mode derivative of ckda_oracle_deltaproduct2 for a loss L with
 * dL/do_t = do and dL/dH_T = dhT, written from the token step itself (not by
 * way of the delta-rule backward above).  Per token, forward:
 *
 *   Hb = alpha_t H_{t-1}                        (Hb = H_{t-1} when ungated)
 *   e1 = v_t1 - Hb^T k_t1,   Hm = Hb + beta_t1 k_t1 e1^T
 *   e2 = v_t2 - Hm^T k_t2,   H_t = Hm + beta_t2 k_t2 e2^T
 *   o_t = H_t^T q_t
 *
 * and in reverse, with G = dL/dH_t carried from the end of the sequence:
 *
 *   dq = H_t do                    G += q do^T
 *   de2 = beta2 G^T k2             dbeta2 = k2^T G e2      dv2 = de2
 *   dk2 = beta2 G e2 - Hm de2      dHm = G - k2 de2^T
 *   de1 = beta1 dHm^T k1           dbeta1 = k1^T dHm e1    dv1 = de1
 *   dk1 = beta1 dHm e1 - Hb de1    dHb = dHm - k1 de1^T
 *   dalpha = <dHb, H_{t-1}>        G <- alpha dHb
 *
 * States are kept at checkpoints every 64 tokens and recomputed one segment
 * at a time.  Layouts as the forward: q, dq [B,H,T,dk]; k, dk [B,H,T,2,dk];
 * v, dv [B,H,T,2,dv]; beta, dbeta [B,H,T,2]; alpha, dalpha [B,H,T] (alpha
 * NULL: ungated, dalpha not written); do [B,H,T,dv] and dhT [B,H,dk,dv] in
 * g_dtype (either may be NULL: zero); dh0 [B,H,dk,dv]. */
int ckda_oracle_deltaproduct2_bwd(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                                  int dtype, const void* h0, int h0_dtype, const void* dout, const void* dhT,
                                  int g_dtype, double* dq, double* dk, double* dv_, double* dalpha, double* dbeta,
                                  double* dh0, int B, int H, int T, int dk_, int dv, int nthreads) {
  if (!q || !k || !v || !beta || !dq || !dk || !dv_ || !dbeta || !dh0 || (alpha && !dalpha)) return 1;
  if (B < 0 || H < 0 || T < 0 || dk_ <= 0 || dv <= 0) return 2;
  if (!valid_dtype(dtype) || (h0 && !valid_dtype(h0_dtype)) || !valid_dtype(g_dtype)) return 3;
  const int n = dk_, seg = 64;
  const long long NS = (long long)n * dv;
  const long long BH = (long long)B * H;
  int failed = 0;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed) num_threads(nt)
#else
  (void)nthreads;
#endif
  for (long long bh = 0; bh < BH; ++bh) {
    const int nseg = (T + seg - 1) / seg;
    double* ck = (double*)malloc(sizeof(double) * (size_t)NS * (nseg + 1));   /* state at each segment start */
    double* st = (double*)malloc(sizeof(double) * (size_t)NS * (seg + 1));    /* states inside one segment */
    double* work = (double*)malloc(sizeof(double) * (size_t)NS * 4);          /* G, Hb, Hm, Ht */
    /* k1, k2, q, (3 n spare), v1, v2, e1, e2, do, de1, de2, then the forward step's scratch (2 n + 3 dv) */
    double* buf = (double*)malloc(sizeof(double) * (size_t)(8 * n + 12 * dv));
    if (!ck || !st || !work || !buf) {
      free(ck); free(st); free(work); free(buf);
      failed |= 1;
      continue;
    }
    double *G = work, *Hb = G + NS, *Hm = Hb + NS, *Ht = Hm + NS;
    double *k1 = buf, *k2 = k1 + n, *qq = k2 + n, *tmp = qq + n;
    double *v1 = tmp + 3 * n, *v2 = v1 + dv, *e1 = v2 + dv, *e2 = e1 + dv, *gd = e2 + dv, *de1 = gd + dv,
           *de2 = de1 + dv, *w = de2 + dv;
    const long long sbase = bh * NS;
    /* forward: checkpoints */
    for (long long e = 0; e < NS; ++e) ck[e] = h0 ? widen(h0, sbase + e, h0_dtype) : 0.0;
    for (int g = 0; g < nseg; ++g) {
      double* S = ck + (long long)(g + 1) * NS;
      memcpy(S, ck + (long long)g * NS, sizeof(double) * NS);
      for (int t = g * seg; t < T && t < (g + 1) * seg; ++t) dp2_token(S, q, k, v, alpha, beta, dtype, bh * T + t, n, dv, w, NULL);
    }
    /* reverse */
    for (long long e = 0; e < NS; ++e) G[e] = dhT ? widen(dhT, sbase + e, g_dtype) : 0.0;
    for (int g = nseg - 1; g >= 0; --g) {
      const int t0 = g * seg, t1 = (t0 + seg < T) ? t0 + seg : T;
      memcpy(st, ck + (long long)g * NS, sizeof(double) * NS);
      for (int t = t0; t < t1; ++t) {
        double* S = st + (long long)(t - t0 + 1) * NS;
        memcpy(S, S - NS, sizeof(double) * NS);
        dp2_token(S, q, k, v, alpha, beta, dtype, bh * T + t, n, dv, w, NULL);
      }
      for (int t = t1 - 1; t >= t0; --t) {
        const long long tok = bh * T + t;
        const double* Hp = st + (long long)(t - t0) * NS;   /* H_{t-1} */
        const double a = alpha ? widen(alpha, tok, dtype) : 1.0;
        const double b1 = widen(beta, tok * 2, dtype), b2 = widen(beta, tok * 2 + 1, dtype);
        for (int i = 0; i < n; ++i) {
          k1[i] = widen(k, (tok * 2) * n + i, dtype);
          k2[i] = widen(k, (tok * 2 + 1) * n + i, dtype);
          qq[i] = widen(q, tok * n + i, dtype);
        }
        for (int j = 0; j < dv; ++j) {
          v1[j] = widen(v, (tok * 2) * dv + j, dtype);
          v2[j] = widen(v, (tok * 2 + 1) * dv + j, dtype);
          gd[j] = dout ? widen(dout, tok * dv + j, g_dtype) : 0.0;
        }
        /* recompute Hb, e1, Hm, e2, H_t */
        for (long long e = 0; e < NS; ++e) Hb[e] = a * Hp[e];
        for (int j = 0; j < dv; ++j) {
          double s = 0.0;
          for (int i = 0; i < n; ++i) s += Hb[(long)i * dv + j] * k1[i];
          e1[j] = v1[j] - s;
        }
        for (int i = 0; i < n; ++i)
          for (int j = 0; j < dv; ++j) Hm[(long)i * dv + j] = Hb[(long)i * dv + j] + b1 * k1[i] * e1[j];
        for (int j = 0; j < dv; ++j) {
          double s = 0.0;
          for (int i = 0; i < n; ++i) s += Hm[(long)i * dv + j] * k2[i];
          e2[j] = v2[j] - s;
        }
        for (int i = 0; i < n; ++i)
          for (int j = 0; j < dv; ++j) Ht[(long)i * dv + j] = Hm[(long)i * dv + j] + b2 * k2[i] * e2[j];
        /* o_t = H_t^T q */
        for (int i = 0; i < n; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += Ht[(long)i * dv + j] * gd[j];
          dq[tok * n + i] = acc;
          for (int j = 0; j < dv; ++j) G[(long)i * dv + j] += qq[i] * gd[j];
        }
        /* second write: H_t = Hm + beta2 k2 e2^T */
        double db2 = 0.0;
        for (int j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (int i = 0; i < n; ++i) acc += G[(long)i * dv + j] * k2[i];
          de2[j] = b2 * acc;
          db2 += acc * e2[j];
          dv_[(tok * 2 + 1) * dv + j] = de2[j];
        }
        for (int i = 0; i < n; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += b2 * G[(long)i * dv + j] * e2[j] - Hm[(long)i * dv + j] * de2[j];
          dk[(tok * 2 + 1) * n + i] = acc;
        }
        for (int i = 0; i < n; ++i)
          for (int j = 0; j < dv; ++j) G[(long)i * dv + j] -= k2[i] * de2[j];   /* now dHm */
        /* first write: Hm = Hb + beta1 k1 e1^T */
        double db1 = 0.0;
        for (int j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (int i = 0; i < n; ++i) acc += G[(long)i * dv + j] * k1[i];
          de1[j] = b1 * acc;
          db1 += acc * e1[j];
          dv_[(tok * 2) * dv + j] = de1[j];
        }
        for (int i = 0; i < n; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += b1 * G[(long)i * dv + j] * e1[j] - Hb[(long)i * dv + j] * de1[j];
          dk[(tok * 2) * n + i] = acc;
        }
        dbeta[tok * 2] = db1;
        dbeta[tok * 2 + 1] = db2;
        for (int i = 0; i < n; ++i)
          for (int j = 0; j < dv; ++j) G[(long)i * dv + j] -= k1[i] * de1[j];   /* now dHb */
        /* gate: Hb = alpha H_{t-1} */
        double ga = 0.0;
        for (long long e = 0; e < NS; ++e) {
          ga += G[e] * Hp[e];
          G[e] *= a;
        }
        if (alpha) dalpha[tok] = ga;
      }
    }
    memcpy(dh0 + sbase, G, sizeof(double) * NS);
    free(ck); free(st); free(work); free(buf);
  }
  return failed ? 4 : 0;
}
