/*
 * Plain fp64 CPU attention: the test oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg use it.  It shares no code,
 * header, table or helper with the GPU library.
 *
 * What it computes (and why this is the whole definition):
 *   "FlashAttention (NL)", section "Problemen met standaard attention":
 *   attention is softmax(Q K^T / sqrt(d_k)) V over the full N x N score
 *   matrix S.  The same page ("Online berekening van Softmax") and the
 *   Czech copy of it say the tiled method reaches this result exactly, and
 *   "Memory-Optimized Flash Attention AI", section "How it compares", says it
 *   computes the full attention matrix without approximation.  So the oracle
 *   is the definition itself, evaluated one query row at a time in double
 *   precision with no tiling, no online rescaling and no reordering:
 *
 *     s_ij   = scale * sum_c q_ic k_jc            for every visible j
 *     m_i    = max_j s_ij
 *     l_i    = sum_j exp(s_ij - m_i)
 *     o_i    = (sum_j exp(s_ij - m_i) v_j) / l_i
 *     lse_i  = m_i + ln(l_i)                      (natural logarithm)
 *
 *   The page's 1/sqrt(d_k) is the caller's `scale`.  Masking ("maskering",
 *   listed among the fused operations in section "Samensmelting van
 *   bewerkingen in één CUDA-kernel") is read as a visibility predicate: a
 *   masked key gets logit -inf, i.e. weight exactly 0, so summing only over
 *   visible keys IS the definition.  lse is the pair of running values the
 *   online-softmax section names (current maximum, sum of exponentials)
 *   folded into one number.
 *
 *   Visibility of key j to query i (0-based positions):
 *     mask 0 (none)    : every j in [0, N)
 *     mask 1 (causal)  : j <= i
 *     mask 2 (sliding) : i - window < j <= i   ("Sparse Attention" glossary,
 *                        "Abgrenzung & Vergleiche": sliding-window attention
 *                        attends to a local window only; read here as the
 *                        `window` most recent keys including key i)
 *
 * Layout: contiguous row-major [BH][N][d] for q, k, v, o; [BH][N] for lse.
 * A row with no visible key (only reachable with window < 1) gets o = 0 and
 * lse = -inf.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MASK_NONE 0
#define ORACLE_MASK_CAUSAL 1
#define ORACLE_MASK_SLIDING 2

/* Visible key range [lo, hi) of query position i. */
static void visible_range(long long i, long long N, int mask_kind,
                          long long window, long long *lo, long long *hi) {
  if (mask_kind == ORACLE_MASK_NONE) {
    *lo = 0;
    *hi = N;
  } else if (mask_kind == ORACLE_MASK_CAUSAL) {
    *lo = 0;
    *hi = i + 1 < N ? i + 1 : N;
  } else {
    long long first = i - window + 1; /* i - window < j  <=>  j >= i-window+1 */
    *lo = first > 0 ? first : 0;
    *hi = i + 1 < N ? i + 1 : N;
  }
}

/* One query row: the definition written out, two passes over the row. */
static void attend_row(const double *qi, long long i, const double *k,
                       const double *v, long long N, long long d, double scale,
                       int mask_kind, long long window, double *s_row,
                       double *oi, double *lse_i) {
  long long lo, hi, j, c;
  visible_range(i, N, mask_kind, window, &lo, &hi);
  for (c = 0; c < d; ++c) oi[c] = 0.0;
  if (hi <= lo) {
    *lse_i = -INFINITY;
    return;
  }
  /* score row s_ij = scale * <q_i, k_j> */
  for (j = lo; j < hi; ++j) {
    const double *kj = k + j * d;
    double dot = 0.0;
    for (c = 0; c < d; ++c) dot += qi[c] * kj[c];
    s_row[j] = scale * dot;
  }
  /* m_i = max_j s_ij */
  double m = s_row[lo];
  for (j = lo + 1; j < hi; ++j)
    if (s_row[j] > m) m = s_row[j];
  /* e_ij = exp(s_ij - m_i), l_i = sum_j e_ij, o_i = sum_j e_ij v_j */
  double l = 0.0;
  for (j = lo; j < hi; ++j) {
    double e = exp(s_row[j] - m);
    const double *vj = v + j * d;
    l += e;
    for (c = 0; c < d; ++c) oi[c] += e * vj[c];
  }
  for (c = 0; c < d; ++c) oi[c] /= l;
  *lse_i = m + log(l);
}

/*
 * Every row of every (batch, head) slice.
 * Returns 0 on success, -1 on a bad argument, -2 if scratch allocation fails.
 */
int oracle_attn_f64(const double *q, const double *k, const double *v,
                    long long BH, long long N, long long d, double scale,
                    int mask_kind, long long window, double *o, double *lse) {
  if (!q || !k || !v || !o || !lse || BH < 0 || N < 0 || d <= 0) return -1;
  if (mask_kind < 0 || mask_kind > 2) return -1;
  int failed = 0;
#pragma omp parallel
  {
    /* every thread reaches the worksharing loop, even if its scratch row
       could not be allocated (it then only records the failure) */
    double *s_row = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    long long r;
#pragma omp for schedule(dynamic, 16)
    for (r = 0; r < BH * N; ++r) {
      if (!s_row) {
#pragma omp atomic write
        failed = 1;
        continue;
      }
      long long bh = r / N, i = r % N;
      const double *kb = k + bh * N * d, *vb = v + bh * N * d;
      attend_row(q + r * d, i, kb, vb, N, d, scale, mask_kind, window, s_row,
                 o + r * d, lse + r);
    }
    free(s_row);
  }
  return failed ? -2 : 0;
}

/*
 * Selected query rows of one (batch, head) slice: q_rows[R][d] holds the
 * query vectors, pos[R] their positions in the sequence, k and v are the
 * slice's [N][d] keys and values.  Output o[R][d], lse[R].  Used to check
 * sampled rows of inputs too large to evaluate whole.
 */
int oracle_attn_rows_f64(const double *q_rows, const long long *pos,
                         long long R, const double *k, const double *v,
                         long long N, long long d, double scale, int mask_kind,
                         long long window, double *o, double *lse) {
  if (!q_rows || !pos || !k || !v || !o || !lse || R < 0 || N < 0 || d <= 0)
    return -1;
  if (mask_kind < 0 || mask_kind > 2) return -1;
  long long r;
  for (r = 0; r < R; ++r)
    if (pos[r] < 0 || pos[r] >= N) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double *s_row = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    long long t;
#pragma omp for schedule(dynamic, 4)
    for (t = 0; t < R; ++t) {
      if (!s_row) {
#pragma omp atomic write
        failed = 1;
        continue;
      }
      attend_row(q_rows + t * d, pos[t], k, v, N, d, scale, mask_kind, window,
                 s_row, o + t * d, lse + t);
    }
    free(s_row);
  }
  return failed ? -2 : 0;
}

/* Number of threads an OpenMP parallel region would use here. */
#ifdef _OPENMP
#include <omp.h>
#endif
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
