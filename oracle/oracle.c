/*
 * Float64 CPU reference for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the oracle that the GPU kernels are
 * checked against. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it. It shares no code, header, table or helper
 * with the HIP library, and the HIP library never calls it.
 *
 * What it computes is the plain definition, written out with no tiling, no
 * running statistics and no reordering:
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
 *     alignment), so query i sits at absolute position i + (Nk - Nq) and sees
 *     key j iff j <= i + (Nk - Nq).
 *   - A row with no visible key returns O = 0: same page and section (the
 *     explicit empty-row policy). Its log-sum-exp is -inf (the log of an
 *     empty sum).
 *   - The per-row statistic saved for a backward pass is reported as
 *     LSE = m + ln(l), in natural-log units of the scaled, masked scores:
 *     "Flash Attention Optimization", section "Sizing a tile, and why the
 *     backward pass recomputes instead of storing" (only m and l are kept).
 *
 * Precision: every input element (IEEE float32 or bfloat16 bit pattern) is
 * widened exactly to double; all arithmetic is double with libm exp/log.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_F32 1
#define ORACLE_BF16 0

/* Widen element idx of a float32 or bfloat16 array to double (exact). */
static double widen(const void* base, int dtype, size_t idx) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/*
 * One query row: row id r = (b*H + h)*Nq + i.
 * s   : scratch of Nk doubles (scores, then unnormalised weights)
 * o   : d doubles out;  lse : 1 double out;  p : Nk doubles out or NULL.
 */
static void one_row(const void* q, const void* k, const void* v, int dtype,
                    int H, int Nq, int Nk, int d, double scale, int causal,
                    long long r, double* s, double* o, double* lse, double* p) {
  long long bh = r / Nq;
  int i = (int)(r % Nq);
  size_t qoff = (size_t)r * (size_t)d;
  size_t kvbase = (size_t)bh * (size_t)Nk * (size_t)d;
  long long last_visible = causal ? (long long)i + (long long)(Nk - Nq) : (long long)Nk - 1;
  (void)H;

  /* scores of visible keys; masked keys are -inf */
  double m = -INFINITY;
  for (int j = 0; j < Nk; ++j) {
    if ((long long)j > last_visible) { s[j] = -INFINITY; continue; }
    double dot = 0.0;
    for (int t = 0; t < d; ++t)
      dot += widen(q, dtype, qoff + t) * widen(k, dtype, kvbase + (size_t)j * d + t);
    s[j] = scale * dot;
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

/*
 * oracle_attention
 *   q [B][H][Nq][d], k and v [B][H][Nk][d], contiguous, dtype ORACLE_F32 or
 *   ORACLE_BF16 (raw bfloat16 bit patterns).
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
  if (!q || !k || !v || !o || !lse || !scratch) return -1;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || nthreads < 1) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
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
    one_row(q, k, v, dtype, H, Nq, Nk, d, scale, causal, r,
            scratch + (size_t)tid * (size_t)Nk, o + (size_t)n * d, lse + n,
            p ? p + (size_t)n * Nk : NULL);
  }
  return 0;
}
