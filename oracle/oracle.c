/*
 * Float64 CPU reference for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the oracle that the GPU kernels are
 * checked against. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it. It shares no code, header, table or helper
 * with the HIP library, and the HIP library never calls it.
 *
 * What it computes is the plain definition, written out with no tiling, no
 * running statistics and no reordering (and, further down, the gradients of
 * that definition for a backward pass):
 *
 *   S = Q K^T * scale (+ mask)      P = softmax(S) row by row      O = P V
 *
 *   - Definition of S, P and O: "Flash Attention Optimization", section
 *     "Attention is not slow because of arithmetic" (the three-line display),
 *     and "Explain FlashAttention ...", section "Keep only the state needed
 *     for the final weighted average" (scores are scaled, then the mask or
 *     bias is added before the softmax).
 *   - Max subtraction before exponentiating (the standard stable softmax):
 *     "Flash Attention Optimization", section "Worked example: online
 *     softmax by hand" (the direct softmax subtracts the global max 5).
 *   - Causal mask on absolute positions, not tile-local ones: "Explain
 *     FlashAttention ...", section "Executable recurrence, with an
 *     empty-state policy" (last paragraph) and section "Common mistakes".
 *     Reading taken where the pages are silent: when Nq != Nk the query rows
 *     are the LAST Nq positions of the key sequence (bottom-right
 *     alignment, causal = 1), so query i sits at absolute position
 *     i + (Nk - Nq) and sees key j iff j <= i + (Nk - Nq). The other reading,
 *     queries at the FIRST Nq positions (top-left, causal = 2: query i sees
 *     key j iff j <= i), is offered as an option. For Nq == Nk both are j <= i.
 *   - A row with no visible key returns O = 0: same page and section (the
 *     explicit empty-row policy). Its log-sum-exp is -inf (the log of an
 *     empty sum).
 *   - An additive bias (optional, oracle_attention_bias) is added to the
 *     scaled score of every visible pair before the softmax: same page,
 *     section "Keep only the state needed for the final weighted average"
 *     (scores are scaled, then the intended mask or bias is added). Reading
 *     taken where the pages are silent: the bias is not multiplied by the
 *     scale, a key hidden by the causal mask stays hidden whatever its bias,
 *     and a bias of -inf hides a key like the mask does (so a row whose keys
 *     all carry -inf is an empty row).
 *   - The per-row statistic saved for a backward pass is reported as
 *     LSE = m + ln(l), in natural-log units of the scaled, masked scores:
 *     "Flash Attention Optimization", section "Sizing a tile, and why the
 *     backward pass recomputes instead of storing" (only m and l are kept).
 *
 * Precision: every input element (IEEE float32, bfloat16 bit pattern or float64) is
 * widened exactly to double; all arithmetic is double with libm exp/log.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 1
#define ORACLE_BF16 0
#define ORACLE_F64 2

/* Widen element idx of a float32, bfloat16 or float64 array to double (exact). */
static double widen(const void* base, int dtype, size_t idx) {
  if (dtype == ORACLE_F64) return ((const double*)base)[idx];
  if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Key position of query row 0 under the causal mask: bottom-right (causal = 1)
 * places the queries at the end of the key sequence, top-left (causal = 2) at its
 * start. */
static long long query_offset(int causal, int Nq, int Nk) {
  return causal == 2 ? 0 : (long long)Nk - (long long)Nq;
}

/* Optional additive bias: element (b, h, i, j) sits at index
 * b*sb + h*sh + i*sq + j of p (a stride of 0 repeats the same values along that
 * dimension). p == NULL means no bias. */
typedef struct {
  const void* p;
  int dtype;
  long long sb, sh, sq;
} bias_view;

/*
 * One query row: row id r = (b*H + h)*Nq + i.
 * s   : scratch of Nk doubles (scores, then unnormalised weights)
 * o   : d doubles out;  lse : 1 double out;  p : Nk doubles out or NULL.
 */
static void one_row(const void* q, const void* k, const void* v, int dtype,
                    int H, int Nq, int Nk, int d, double scale, int causal,
                    const bias_view* bias,
                    long long r, double* s, double* o, double* lse, double* p) {
  long long bh = r / Nq;
  int i = (int)(r % Nq);
  size_t qoff = (size_t)r * (size_t)d;
  size_t kvbase = (size_t)bh * (size_t)Nk * (size_t)d;
  long long last_visible = causal ? (long long)i + query_offset(causal, Nq, Nk) : (long long)Nk - 1;
  size_t brow = 0; /* index of bias element (b, h, i, 0) */
  if (bias && bias->p)
    brow = (size_t)((bh / H) * bias->sb + (bh % H) * bias->sh + (long long)i * bias->sq);

  /* scores of visible keys; masked keys are -inf */
  double m = -INFINITY;
  for (int j = 0; j < Nk; ++j) {
    if ((long long)j > last_visible) { s[j] = -INFINITY; continue; }
    double dot = 0.0;
    for (int t = 0; t < d; ++t)
      dot += widen(q, dtype, qoff + t) * widen(k, dtype, kvbase + (size_t)j * d + t);
    s[j] = scale * dot;
    if (bias && bias->p) s[j] += widen(bias->p, bias->dtype, brow + (size_t)j);
    if (s[j] > m) m = s[j];
  }

  if (m == -INFINITY) { /* no visible key: empty-row policy */
    for (int t = 0; t < d; ++t) o[t] = 0.0;
    *lse = -INFINITY;
    if (p) for (int j = 0; j < Nk; ++j) p[j] = 0.0;
    return;
  }

  /* stable softmax: exponentiate relative to the row max, then normalise */
  double l = 0.0;
  for (int j = 0; j < Nk; ++j) {
    s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
    l += s[j];
  }
  for (int t = 0; t < d; ++t) o[t] = 0.0;
  for (int j = 0; j < Nk; ++j) {
    if (s[j] == 0.0) continue;
    double w = s[j] / l;
    for (int t = 0; t < d; ++t) o[t] += w * widen(v, dtype, kvbase + (size_t)j * d + t);
  }
  *lse = m + log(l);
  if (p) for (int j = 0; j < Nk; ++j) p[j] = s[j] / l;
}

/* Shared checks and row loop of oracle_attention and oracle_attention_bias. */
static int attention_rows(const void* q, const void* k, const void* v, int dtype,
                          int B, int H, int Nq, int Nk, int d, double scale, int causal,
                          const bias_view* bias,
                          const long long* rows, long long nrows, int nthreads,
                          double* scratch, double* o, double* lse, double* p) {
  if (!q || !k || !v || !o || !lse || !scratch) return -1;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || nthreads < 1) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
  if (causal < 0 || causal > 2) return -1;
  if (bias && bias->p) {
    if (bias->dtype != ORACLE_F32 && bias->dtype != ORACLE_BF16 && bias->dtype != ORACLE_F64) return -1;
    if (bias->sb < 0 || bias->sh < 0 || bias->sq < 0) return -1;
  }
  long long total = (long long)B * H * Nq;
  if (!rows) nrows = total;
  for (long long n = 0; rows && n < nrows; ++n)
    if (rows[n] < 0 || rows[n] >= total) return -1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (long long n = 0; n < nrows; ++n) {
    int tid = 0;
#ifdef _OPENMP
    extern int omp_get_thread_num(void);
    tid = omp_get_thread_num();
#endif
    long long r = rows ? rows[n] : n;
    one_row(q, k, v, dtype, H, Nq, Nk, d, scale, causal, bias, r,
            scratch + (size_t)tid * (size_t)Nk, o + (size_t)n * d, lse + n,
            p ? p + (size_t)n * Nk : NULL);
  }
  return 0;
}

/*
 * oracle_attention
 *   q [B][H][Nq][d], k and v [B][H][Nk][d], contiguous, dtype ORACLE_F32,
 *   ORACLE_BF16 (raw bfloat16 bit patterns) or ORACLE_F64.
 *   rows   : list of nrows flat row ids (b*H + h)*Nq + i, or NULL for all
 *            B*H*Nq rows in order.
 *   o      : [nrows][d] doubles;  lse : [nrows] doubles;
 *   p      : [nrows][Nk] doubles or NULL (the probability rows, small cases).
 *   scratch: caller-owned, nthreads_max * Nk doubles (one score row per
 *            thread); nthreads_max is the value the caller passes as nthreads.
 * Returns 0, or -1 for an invalid argument.
 */
int oracle_attention(const void* q, const void* k, const void* v, int dtype,
                     int B, int H, int Nq, int Nk, int d, double scale, int causal,
                     const long long* rows, long long nrows, int nthreads,
                     double* scratch, double* o, double* lse, double* p) {
  return attention_rows(q, k, v, dtype, B, H, Nq, Nk, d, scale, causal, NULL,
                        rows, nrows, nthreads, scratch, o, lse, p);
}

/*
 * oracle_attention_bias: as oracle_attention, with the additive bias
 *   S[b][h][i][j] = scale * q_i . k_j + bias[b*sb + h*sh + i*sq + j]
 * (bias of dtype bdtype, strides in elements, each >= 0; 0 repeats a dimension).
 */
int oracle_attention_bias(const void* q, const void* k, const void* v, int dtype,
                          const void* bias, int bdtype, long long sb, long long sh, long long sq,
                          int B, int H, int Nq, int Nk, int d, double scale, int causal,
                          const long long* rows, long long nrows, int nthreads,
                          double* scratch, double* o, double* lse, double* p) {
  if (!bias) return -1;
  bias_view bv = {bias, bdtype, sb, sh, sq};
  return attention_rows(q, k, v, dtype, B, H, Nq, Nk, d, scale, causal, &bv,
                        rows, nrows, nthreads, scratch, o, lse, p);
}

/*
 * Backward pass: gradients of the loss sum(O * dO) with respect to Q, K and V,
 * for the same attention as above. The pages say only that a backward pass
 * recomputes the probability tiles from the saved per-row statistics instead
 * of storing P ("Flash Attention Optimization", section "Sizing a tile, and
 * why the backward pass recomputes instead of storing"; "Explain
 * FlashAttention ...", section "Exact attention, finite precision and
 * backward"); the gradients themselves follow from the definition
 * O = P V, P = softmax(S) row by row, S = scale * Q K^T (+ mask) by the chain
 * rule, written out here in double precision:
 *
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   dS_ij = P_ij (dP_ij - sum_t P_it dP_it)          (softmax Jacobian)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 *
 * with P_ij = exp(s_ij - LSE_i) (the identity exp(s - m) / l = exp(s - (m + ln l)))
 * and sum_t P_it dP_it = dO_i . O_i. Masked pairs have P = 0 and contribute
 * nothing; a row with no visible key has P = 0 everywhere.
 *
 * Row statistics pass: for every query row of a head, LSE_i and
 * Dsum_i = dO_i . O_i from the definition above (one_row). dQ rows need only
 * their own row; dK and dV rows need the statistics of every query row of the
 * head, which are computed for each head that a requested key row belongs to.
 */
static void row_stats(const void* q, const void* k, const void* v, const void* dout,
                      int dtype, int H, int Nq, int Nk, int d, double scale, int causal,
                      const bias_view* bias,
                      long long r, double* s, double* o, double* lse, double* dsum) {
  one_row(q, k, v, dtype, H, Nq, Nk, d, scale, causal, bias, r, s, o, lse, NULL);
  double acc = 0.0;
  for (int t = 0; t < d; ++t) acc += widen(dout, dtype, (size_t)r * d + t) * o[t];
  *dsum = acc;
}

/* score of (query row r, key j of the same head), plus the bias element of the pair if
 * there is a bias, or -inf when masked */
static double score(const void* q, const void* k, int dtype, int H, int Nq, int Nk, int d,
                    double scale, int causal, const bias_view* bias, long long r, int j) {
  long long bh = r / Nq;
  int i = (int)(r % Nq);
  if (causal && (long long)j - query_offset(causal, Nq, Nk) > (long long)i) return -INFINITY;
  size_t qoff = (size_t)r * d, koff = ((size_t)bh * Nk + j) * d;
  double dot = 0.0;
  for (int t = 0; t < d; ++t) dot += widen(q, dtype, qoff + t) * widen(k, dtype, koff + t);
  double sc = scale * dot;
  if (bias && bias->p)
    sc += widen(bias->p, bias->dtype,
                (size_t)((bh / H) * bias->sb + (bh % H) * bias->sh + (long long)i * bias->sq + j));
  return sc;
}

/* dP_ij = dO_i . v_j */
static double dprob(const void* dout, const void* v, int dtype, int Nq, int Nk, int d,
                    long long r, int j) {
  long long bh = r / Nq;
  size_t ooff = (size_t)r * d, voff = ((size_t)bh * Nk + j) * d;
  double dot = 0.0;
  for (int t = 0; t < d; ++t) dot += widen(dout, dtype, ooff + t) * widen(v, dtype, voff + t);
  return dot;
}

/*
 * oracle_attention_bwd (bwd_rows below, with no bias; oracle_attention_bwd_bias at the end
 * of the file adds one)
 *   q [B][H][Nq][d], k, v [B][H][Nk][d], dout [B][H][Nq][d], one dtype.
 *   qrows : flat query rows (b*H + h)*Nq + i whose dQ is wanted (nq of them),
 *           or NULL for all;  dq : [nq][d] doubles (may be NULL if nq == 0).
 *   krows : flat key rows (b*H + h)*Nk + j whose dK and dV are wanted (nk of
 *           them), or NULL for all;  dk, dv : [nk][d] doubles.
 *   nthreads : OpenMP threads. Returns 0, or -1 for an invalid argument or a
 *   failed allocation.
 */
static int bwd_rows(const void* q, const void* k, const void* v, const void* dout,
                    int dtype, int B, int H, int Nq, int Nk, int d, double scale,
                    int causal, const bias_view* bias, const long long* qrows, long long nq,
                    const long long* krows, long long nk, int nthreads,
                    double* dq, double* dk, double* dv, double* dbias) {
  if (!q || !k || !v || !dout) return -1;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || nthreads < 1) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
  if (causal < 0 || causal > 2) return -1;
  if (bias && bias->p) {
    if (bias->dtype != ORACLE_F32 && bias->dtype != ORACLE_BF16 && bias->dtype != ORACLE_F64) return -1;
    if (bias->sb < 0 || bias->sh < 0 || bias->sq < 0) return -1;
  }
  /* the bias gradient is the full dS of every query row */
  if (dbias && qrows) return -1;
  const long long BH = (long long)B * H;
  if (!qrows) nq = BH * Nq;
  if (!krows) nk = BH * Nk;
  if ((nq > 0 && !dq) || (nk > 0 && (!dk || !dv))) return -1;
  for (long long n = 0; qrows && n < nq; ++n)
    if (qrows[n] < 0 || qrows[n] >= BH * Nq) return -1;
  for (long long n = 0; krows && n < nk; ++n)
    if (krows[n] < 0 || krows[n] >= BH * Nk) return -1;

  int failed = 0;
  /* dQ rows: each needs only its own row statistics */
#pragma omp parallel num_threads(nthreads)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    if (!s || !o) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (long long n = 0; n < nq; ++n) {
      long long r = qrows ? qrows[n] : n;
      long long bh = r / Nq;
      double lse, dsum;
      double* out = dq + (size_t)n * d;
      for (int t = 0; t < d; ++t) out[t] = 0.0;
      if (!s || !o) continue;
      double* grow = dbias ? dbias + (size_t)n * Nk : NULL;
      if (grow) for (int j = 0; j < Nk; ++j) grow[j] = 0.0;
      row_stats(q, k, v, dout, dtype, H, Nq, Nk, d, scale, causal, bias, r, s, o, &lse, &dsum);
      if (lse == -INFINITY) continue; /* empty row: P = 0 */
      for (int j = 0; j < Nk; ++j) {
        double sc = score(q, k, dtype, H, Nq, Nk, d, scale, causal, bias, r, j);
        if (sc == -INFINITY) continue;
        double p = exp(sc - lse);
        double ds = p * (dprob(dout, v, dtype, Nq, Nk, d, r, j) - dsum);
        /* the bias enters S with weight 1, so dL/dbias_ij = dS_ij */
        if (grow) grow[j] = ds;
        size_t koff = ((size_t)bh * Nk + j) * d;
        for (int t = 0; t < d; ++t) out[t] += scale * ds * widen(k, dtype, koff + t);
      }
    }
    free(s);
    free(o);
  }

  if (failed) return -1;
  if (nk == 0) return 0;
  /* row statistics of every query row of the heads that requested key rows belong to */
  char* need = (char*)calloc((size_t)BH, 1);
  double* lse_all = (double*)malloc(sizeof(double) * (size_t)(BH * Nq));
  double* dsum_all = (double*)malloc(sizeof(double) * (size_t)(BH * Nq));
  if (!need || !lse_all || !dsum_all) {
    free(need); free(lse_all); free(dsum_all);
    return -1;
  }
  for (long long n = 0; n < nk; ++n) need[(krows ? krows[n] : n) / Nk] = 1;
#pragma omp parallel num_threads(nthreads)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    if (!s || !o) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (long long r = 0; r < BH * Nq; ++r) {
      if (!need[r / Nq] || !s || !o) continue;
      row_stats(q, k, v, dout, dtype, H, Nq, Nk, d, scale, causal, bias, r, s, o,
                lse_all + r, dsum_all + r);
    }
    free(s);
    free(o);
  }
  if (failed) {
    free(need); free(lse_all); free(dsum_all);
    return -1;
  }

  /* dK and dV rows: sum over the query rows of the key's head */
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (long long n = 0; n < nk; ++n) {
    long long kr = krows ? krows[n] : n;
    long long bh = kr / Nk;
    int j = (int)(kr % Nk);
    double* gk = dk + (size_t)n * d;
    double* gv = dv + (size_t)n * d;
    for (int t = 0; t < d; ++t) gk[t] = gv[t] = 0.0;
    for (int i = 0; i < Nq; ++i) {
      long long r = bh * Nq + i;
      if (lse_all[r] == -INFINITY) continue;
      double sc = score(q, k, dtype, H, Nq, Nk, d, scale, causal, bias, r, j);
      if (sc == -INFINITY) continue;
      double p = exp(sc - lse_all[r]);
      double ds = p * (dprob(dout, v, dtype, Nq, Nk, d, r, j) - dsum_all[r]);
      size_t off = (size_t)r * d;
      for (int t = 0; t < d; ++t) {
        gv[t] += p * widen(dout, dtype, off + t);
        gk[t] += scale * ds * widen(q, dtype, off + t);
      }
    }
  }
  free(need); free(lse_all); free(dsum_all);
  return 0;
}

int oracle_attention_bwd(const void* q, const void* k, const void* v, const void* dout,
                         int dtype, int B, int H, int Nq, int Nk, int d, double scale,
                         int causal, const long long* qrows, long long nq,
                         const long long* krows, long long nk, int nthreads,
                         double* dq, double* dk, double* dv) {
  return bwd_rows(q, k, v, dout, dtype, B, H, Nq, Nk, d, scale, causal, NULL, qrows, nq,
                  krows, nk, nthreads, dq, dk, dv, NULL);
}

/*
 * oracle_attention_bwd_bias: oracle_attention_bwd for the attention with the additive
 * bias of oracle_attention_bias (S = scale * Q K^T + bias, the same strides and dtypes),
 * and optionally the gradient with respect to a full bias:
 *   dbias : [B*H*Nq][Nk] doubles or NULL. The bias enters each score with weight 1, so
 *           dL/dbias_ij = dS_ij (0 for pairs the mask hides and rows that see no key).
 *           A broadcast bias's gradient is this summed over its broadcast dimensions.
 *           Requires qrows == NULL (every query row).
 */
int oracle_attention_bwd_bias(const void* q, const void* k, const void* v, const void* dout,
                              int dtype, const void* bias, int bdtype, long long sb,
                              long long sh, long long sq, int B, int H, int Nq, int Nk, int d,
                              double scale, int causal, const long long* qrows, long long nq,
                              const long long* krows, long long nk, int nthreads,
                              double* dq, double* dk, double* dv, double* dbias) {
  if (!bias) return -1;
  bias_view bv = {bias, bdtype, sb, sh, sq};
  return bwd_rows(q, k, v, dout, dtype, B, H, Nq, Nk, d, scale, causal, &bv, qrows, nq,
                  krows, nk, nthreads, dq, dk, dv, dbias);
}
