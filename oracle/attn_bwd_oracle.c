/*
 * Plain fp64 CPU gradients of attention: the backward-pass test oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the tests and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the GPU library (nor with attn_oracle.c).
 *
 * What it computes.  The forward definition is that of attn_oracle.c
 * ("FlashAttention (NL)", section "Problemen met standaard attention"):
 *
 *   s_ij = scale * <q_i, k_j>   over the keys j visible to query i
 *   P_ij = exp(s_ij) / sum_k exp(s_ik)
 *   o_i  = sum_j P_ij v_j
 *
 * Given the gradient do_i of a loss with respect to o_i, the gradients with
 * respect to q, k and v follow from the chain rule, written out here with no
 * tiling and no reordering:
 *
 *   dP_ij = <do_i, v_j>                      (o_i is linear in P_i.)
 *   D_i   = sum_j P_ij dP_ij                 (softmax Jacobian:
 *   dS_ij = P_ij (dP_ij - D_i)                dP_i. -> dS_i.)
 *   dq_i  = scale * sum_j dS_ij k_j
 *   dk_j  = scale * sum_i dS_ij q_i
 *   dv_j  = sum_i P_ij do_i
 *
 * P is recomputed from q and k wherever it is needed, never stored whole:
 * the recomputation of intermediate results that "Memory-Optimized Flash
 * Attention AI", section "How it works", describes.  Masked pairs have
 * P_ij = 0 and contribute nothing.  Visibility of key j to query i as in
 * attn_oracle.c: none (all j), causal (j <= i), sliding (i - window < j <= i).
 *
 * Layout: contiguous row-major [N][d] per (batch, head) slice.
 */
#include <math.h>
#include <stdlib.h>

static int visible(long long i, long long j, int mask_kind, long long window) {
  if (mask_kind == 0) return 1;
  if (mask_kind == 1) return j <= i;
  return j <= i && j > i - window;
}

/*
 * Row statistics of query row i of one slice: the maximum m and exponent
 * sum l of its visible scores (so P_ij = exp(s_ij - m) / l) and D_i.
 * s_row is N doubles of scratch.  Returns 0 if the row sees no key.
 */
static int row_stats(const double *qi, long long i, const double *k,
                     const double *v, const double *doi, long long N,
                     long long d, double scale, int mask_kind, long long window,
                     double *s_row, double *m_out, double *l_out,
                     double *D_out) {
  long long j, c;
  double m = -INFINITY;
  int any = 0;
  for (j = 0; j < N; ++j) {
    if (!visible(i, j, mask_kind, window)) continue;
    double dot = 0.0;
    for (c = 0; c < d; ++c) dot += qi[c] * k[j * d + c];
    s_row[j] = scale * dot;
    if (!any || s_row[j] > m) m = s_row[j];
    any = 1;
  }
  if (!any) return 0;
  double l = 0.0;
  for (j = 0; j < N; ++j)
    if (visible(i, j, mask_kind, window)) l += exp(s_row[j] - m);
  double D = 0.0;
  for (j = 0; j < N; ++j) {
    if (!visible(i, j, mask_kind, window)) continue;
    double p = exp(s_row[j] - m) / l;
    double dp = 0.0;
    for (c = 0; c < d; ++c) dp += doi[c] * v[j * d + c];
    D += p * dp;
  }
  *m_out = m;
  *l_out = l;
  *D_out = D;
  return 1;
}

/* dq_i of one query row (s_row: N doubles of scratch). */
static void dq_row(const double *qi, long long i, const double *k,
                   const double *v, const double *doi, long long N, long long d,
                   double scale, int mask_kind, long long window, double *s_row,
                   double *dqi) {
  long long j, c;
  double m, l, D;
  for (c = 0; c < d; ++c) dqi[c] = 0.0;
  if (!row_stats(qi, i, k, v, doi, N, d, scale, mask_kind, window, s_row, &m, &l, &D))
    return;
  for (j = 0; j < N; ++j) {
    if (!visible(i, j, mask_kind, window)) continue;
    double p = exp(s_row[j] - m) / l;
    double dp = 0.0;
    for (c = 0; c < d; ++c) dp += doi[c] * v[j * d + c];
    double ds = p * (dp - D);
    for (c = 0; c < d; ++c) dqi[c] += scale * ds * k[j * d + c];
  }
}

/*
 * dk_j and dv_j of one key, given every row's statistics (m, l, D; ok[i] = 0
 * for a row that sees no key).
 */
static void dkv_key(long long j, const double *q, const double *k,
                    const double *v, const double *dout, long long N,
                    long long d, double scale, int mask_kind, long long window,
                    const double *m, const double *l, const double *D,
                    const int *ok, double *dkj, double *dvj) {
  long long i, c;
  for (c = 0; c < d; ++c) dkj[c] = dvj[c] = 0.0;
  for (i = 0; i < N; ++i) {
    if (!ok[i] || !visible(i, j, mask_kind, window)) continue;
    double dot = 0.0, dp = 0.0;
    for (c = 0; c < d; ++c) {
      dot += q[i * d + c] * k[j * d + c];
      dp += dout[i * d + c] * v[j * d + c];
    }
    double p = exp(scale * dot - m[i]) / l[i];
    double ds = p * (dp - D[i]);
    for (c = 0; c < d; ++c) {
      dvj[c] += p * dout[i * d + c];
      dkj[c] += scale * ds * q[i * d + c];
    }
  }
}

/* Row statistics of every row of one slice (parallel over rows). */
static int all_row_stats(const double *q, const double *k, const double *v,
                         const double *dout, long long N, long long d,
                         double scale, int mask_kind, long long window,
                         double *m, double *l, double *D, int *ok) {
  int failed = 0;
#pragma omp parallel
  {
    double *s_row = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    long long i;
#pragma omp for schedule(dynamic, 8)
    for (i = 0; i < N; ++i) {
      if (!s_row) {
#pragma omp atomic write
        failed = 1;
        continue;
      }
      ok[i] = row_stats(q + i * d, i, k, v, dout + i * d, N, d, scale, mask_kind,
                        window, s_row, &m[i], &l[i], &D[i]);
    }
    free(s_row);
  }
  return failed;
}

static int bad_args(long long N, long long d, int mask_kind) {
  return N < 0 || d <= 0 || mask_kind < 0 || mask_kind > 2;
}

/*
 * dq, dk, dv of every slice: q, k, v, dout, dq, dk, dv are [BH][N][d].
 * Returns 0, -1 on a bad argument, -2 if scratch allocation fails.
 */
int oracle_attn_bwd_f64(const double *q, const double *k, const double *v,
                        const double *dout, long long BH, long long N,
                        long long d, double scale, int mask_kind,
                        long long window, double *dq, double *dk, double *dv) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv || BH < 0 || bad_args(N, d, mask_kind))
    return -1;
  double *m = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  double *l = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  double *D = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  int *ok = (int *)malloc(sizeof(int) * (size_t)(N > 0 ? N : 1));
  int failed = !m || !l || !D || !ok;
  long long bh;
  for (bh = 0; bh < BH && !failed; ++bh) {
    const long long off = bh * N * d;
    const double *qs = q + off, *ks = k + off, *vs = v + off, *dos = dout + off;
    failed = all_row_stats(qs, ks, vs, dos, N, d, scale, mask_kind, window, m, l, D, ok);
    if (failed) break;
#pragma omp parallel
    {
      double *s_row = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
      long long t;
#pragma omp for schedule(dynamic, 8)
      for (t = 0; t < N; ++t) {
        if (!s_row) {
#pragma omp atomic write
          failed = 1;
          continue;
        }
        dq_row(qs + t * d, t, ks, vs, dos + t * d, N, d, scale, mask_kind, window, s_row,
               dq + off + t * d);
        dkv_key(t, qs, ks, vs, dos, N, d, scale, mask_kind, window, m, l, D, ok,
                dk + off + t * d, dv + off + t * d);
      }
      free(s_row);
    }
  }
  free(m);
  free(l);
  free(D);
  free(ok);
  return failed ? -2 : 0;
}

/*
 * dq of selected query rows of one slice: rows[R] are positions, q, k, v,
 * dout are the slice's [N][d].  Output dq[R][d].
 */
int oracle_attn_bwd_rows_f64(const double *q, const double *k, const double *v,
                             const double *dout, long long N, long long d,
                             double scale, int mask_kind, long long window,
                             const long long *rows, long long R, double *dq) {
  if (!q || !k || !v || !dout || !rows || !dq || R < 0 || bad_args(N, d, mask_kind))
    return -1;
  long long t;
  for (t = 0; t < R; ++t)
    if (rows[t] < 0 || rows[t] >= N) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double *s_row = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    long long u;
#pragma omp for schedule(dynamic, 4)
    for (u = 0; u < R; ++u) {
      if (!s_row) {
#pragma omp atomic write
        failed = 1;
        continue;
      }
      const long long i = rows[u];
      dq_row(q + i * d, i, k, v, dout + i * d, N, d, scale, mask_kind, window, s_row,
             dq + u * d);
    }
    free(s_row);
  }
  return failed ? -2 : 0;
}

/*
 * dk and dv of selected keys of one slice: keys[K] are positions.  Output
 * dk[K][d], dv[K][d].  Every row's statistics are computed first.
 */
int oracle_attn_bwd_keys_f64(const double *q, const double *k, const double *v,
                             const double *dout, long long N, long long d,
                             double scale, int mask_kind, long long window,
                             const long long *keys, long long K, double *dk,
                             double *dv) {
  if (!q || !k || !v || !dout || !keys || !dk || !dv || K < 0 || bad_args(N, d, mask_kind))
    return -1;
  long long t;
  for (t = 0; t < K; ++t)
    if (keys[t] < 0 || keys[t] >= N) return -1;
  double *m = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  double *l = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  double *D = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  int *ok = (int *)malloc(sizeof(int) * (size_t)(N > 0 ? N : 1));
  int failed = !m || !l || !D || !ok;
  if (!failed) failed = all_row_stats(q, k, v, dout, N, d, scale, mask_kind, window, m, l, D, ok);
  if (!failed) {
    long long u;
#pragma omp parallel for schedule(dynamic, 4)
    for (u = 0; u < K; ++u)
      dkv_key(keys[u], q, k, v, dout, N, d, scale, mask_kind, window, m, l, D, ok,
              dk + u * d, dv + u * d);
  }
  free(m);
  free(l);
  free(D);
  free(ok);
  return failed ? -2 : 0;
}
