/*
 * saf_oracle.c -- plain, slow, fp64 CPU oracle for the mixed-head SAF attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this file's library.  The GPU product path never calls it, links it or falls
 * back to it, and this file shares no code, header, table or helper with the GPU path.
 *
 * Citations name the page and the section / equation / table on it:
 *   [Notes]      the page "When Can Attention Heads Be Statically Defined?：中文精读笔记"
 *                (close-reading notes on arXiv 2609.34650v1).
 *   [Paper page] the page "When Can Attention Heads Be Statically Defined?" (abstract, figure
 *                captions and appendix tables of the same paper).
 *
 * Every function works on ONE (batch, head) slice, row-major, in fp64:
 *   q, k, v, dout : [T][d]          a, r : [T]  (a = alpha, r = rho, 0-based)
 * and on an explicit list of rows (queries) or columns (keys), so that a caller can ask for every
 * row (full compare) or for a sample of rows (spot checks at large sizes).
 *
 * What is computed is the plain definition, written out:
 *   ordinary head   A = softmax_causal(s * Q K^T),  O = A V               [Notes §一]
 *   replaced head   P(i,j) = exp(a(j) + r(i-j)) / Z(i) for j <= i, 0 for j > i,
 *                   Z(i) = sum_{k<=i} exp(a(k) + r(i-k)),  O = P V          [Notes §二.3, Eq.(3)]
 *   backward        ordinary: the softmax chain rule (dq, dk, dv);
 *                   replaced: dV = P^T dO only, alpha and rho are frozen      [Notes §二.4]
 *   calibration     Ahat = (1/N) sum_n A^(n);  s_var = sum_n ||A^(n) - Ahat||_F^2 / ((N-1) T^2)
 *                                                                             [Notes §二.1, Eq.(1)]
 *   KL score        mean over sequences and rows of KL(A^(n)_i || Ahat_i)     [Notes §二.1]
 *   pattern grad    dL/da, dL/dr of a replaced head whose pattern is trained  [Paper page] Table 14
 *   compact fit     a, r minimising the row-wise cross-entropy to Ahat by Adam [Notes §二.3]
 * A row's softmax is evaluated as exp(t_j - m) / sum_k exp(t_k - m) with m the row maximum, which is
 * the same quantity as exp(t_j) / sum_k exp(t_k) (the common factor exp(-m) cancels) but cannot
 * overflow.  The log normaliser is reported as m + log(sum_k exp(t_k - m)) = log sum_k exp(t_k).
 *
 * Readings where the pages leave a step open (each also listed in the design notes):
 *   - Eq. (3) is 1-based; here a[j] is alpha at key position j and r[delta] is rho at distance
 *     delta = i - j, both 0-based, r[0] the self-distance.
 *   - alpha and rho are logits as they stand: no 1/sqrt(d) on replaced heads.
 *   - key j is visible to query i iff j <= i (self included) for both head kinds.
 *   - -inf in a or r is allowed and gives weight 0; a row whose entries are all -inf is undefined.
 *   - Eq. (1) counts all T^2 entries (the upper triangle is 0 in every map and in the mean).
 *   - the "row-wise forward KL" selector is KL(A^(n)_i || Ahat_i), averaged over n and rows.
 *   - the compact fit starts from a = r = 0 with Adam step size lr (the pages give neither).
 *
 * Return value of every entry point: 0 on success, -1 on an invalid argument (nothing written).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_EXPORT __attribute__((visibility("default")))

/* ---- one causal row of an ordinary head: logits t[0..i] = s * q_i . k_j ------------------------ */
static void ordinary_logits(int d, const double* q, const double* k, double scale, int i,
                            double* t) {
  const double* qi = q + (size_t)i * d;
  for (int j = 0; j <= i; ++j) {
    const double* kj = k + (size_t)j * d;
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += qi[c] * kj[c];
    t[j] = scale * acc;
  }
}

/* ---- one causal row of a replaced head: logits t[0..i] = a(j) + r(i-j)   [Notes Eq.(3)] -------- */
static void replaced_logits(const double* a, const double* r, int i, double* t) {
  for (int j = 0; j <= i; ++j) t[j] = a[j] + r[i - j];
}

/* ---- turn logits t[0..i] into probabilities p[0..i]; returns log sum_j exp(t_j) -------------- */
static double softmax_row(int i, const double* t, double* p) {
  double m = -INFINITY;
  for (int j = 0; j <= i; ++j)
    if (t[j] > m) m = t[j];
  double l = 0.0;
  for (int j = 0; j <= i; ++j) {
    p[j] = exp(t[j] - m);
    l += p[j];
  }
  for (int j = 0; j <= i; ++j) p[j] /= l;
  return m + log(l);
}

/* row i of the causal pattern of either head kind: p[0..i], returns the row's log normaliser */
static double pattern_row(int kind, int d, const double* q, const double* k, const double* a,
                          const double* r, double scale, int i, double* t, double* p) {
  if (kind == 0)
    ordinary_logits(d, q, k, scale, i, t);
  else
    replaced_logits(a, r, i, t);
  return softmax_row(i, t, p);
}

static int rows_ok(int T, int n, const int* rows) {
  if (n < 0 || (n > 0 && !rows)) return 0;
  for (int x = 0; x < n; ++x)
    if (rows[x] < 0 || rows[x] >= T) return 0;
  return 1;
}

/*
 * Forward for one head.  kind 0 = ordinary (uses q, k, scale), kind 1 = replaced (uses a, r).
 * For each listed row i:  o[x][:] = sum_{j<=i} P(i,j) v[j][:],  lse[x] = log of the row normaliser
 * (ordinary: log sum_j exp(s q_i.k_j); replaced: log Z(i)).
 */
ORC_EXPORT int orc_head_fwd(int kind, int T, int d, const double* q, const double* k,
                            const double* v, const double* a, const double* r, double scale,
                            int nrows, const int* rows, double* o, double* lse) {
  if (T < 1 || d < 1 || !v || !o || !rows_ok(T, nrows, rows)) return -1;
  if (kind == 0 && (!q || !k)) return -1;
  if (kind == 1 && (!a || !r)) return -1;
  if (kind != 0 && kind != 1) return -1;
#pragma omp parallel
  {
    double* t = (double*)malloc(sizeof(double) * (size_t)T);
    double* p = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(dynamic, 4)
    for (int x = 0; x < nrows; ++x) {
      const int i = rows[x];
      const double lz = pattern_row(kind, d, q, k, a, r, scale, i, t, p);
      double* oi = o + (size_t)x * d;
      for (int c = 0; c < d; ++c) oi[c] = 0.0;
      for (int j = 0; j <= i; ++j) {
        const double* vj = v + (size_t)j * d;
        for (int c = 0; c < d; ++c) oi[c] += p[j] * vj[c];
      }
      if (lse) lse[x] = lz;
    }
    free(t);
    free(p);
  }
  return 0;
}

/*
 * Dense pattern of one head (tiny T only): P[i][j] for all i, j (zeros above the diagonal).
 */
ORC_EXPORT int orc_head_pattern(int kind, int T, int d, const double* q, const double* k,
                                const double* a, const double* r, double scale, double* P) {
  if (T < 1 || !P) return -1;
  if (kind == 0 && (!q || !k || d < 1)) return -1;
  if (kind == 1 && (!a || !r)) return -1;
  double* t = (double*)malloc(sizeof(double) * (size_t)T);
  for (int i = 0; i < T; ++i) {
    double* Pi = P + (size_t)i * T;
    pattern_row(kind, d, q, k, a, r, scale, i, t, Pi);
    for (int j = i + 1; j < T; ++j) Pi[j] = 0.0;
  }
  free(t);
  return 0;
}

/*
 * Backward for one head, loss gradient dout = dL/dO.
 *   ordinary (kind 0), with P the causal softmax, dP(i,j) = dO_i . v_j,
 *     delta_i = sum_j P(i,j) dP(i,j),  dS(i,j) = P(i,j) (dP(i,j) - delta_i):
 *       dq_i = s sum_{j<=i} dS(i,j) k_j,  dk_j = s sum_{i>=j} dS(i,j) q_i,  dv_j = sum_{i>=j} P(i,j) dO_i
 *   replaced (kind 1): dv_j = sum_{i>=j} P(i,j) dO_i; dq = dk = 0 (outputs do not depend on q, k;
 *     alpha and rho are frozen buffers)                                    [Notes §二.4]
 * dq is produced for the listed query rows (qrows), dk / dv for the listed key rows (krows).
 * Any of dq / dk may be NULL when not wanted (their row count is then ignored).
 */
ORC_EXPORT int orc_head_bwd(int kind, int T, int d, const double* q, const double* k,
                            const double* v, const double* dout, const double* a,
                            const double* r, double scale, int nq, const int* qrows, double* dq,
                            int nk, const int* krows, double* dk, double* dv) {
  if (T < 1 || d < 1 || !v || !dout) return -1;
  if (kind != 0 && kind != 1) return -1;
  if (kind == 0 && (!q || !k)) return -1;
  if (kind == 1 && (!a || !r)) return -1;
  if (dq && !rows_ok(T, nq, qrows)) return -1;
  if ((dk || dv) && !rows_ok(T, nk, krows)) return -1;

  /* query-side outputs: dq rows (zero for a replaced head) */
  if (dq) {
    if (kind == 1) {
      memset(dq, 0, sizeof(double) * (size_t)nq * d);
    } else {
#pragma omp parallel
      {
        double* t = (double*)malloc(sizeof(double) * (size_t)T);
        double* p = (double*)malloc(sizeof(double) * (size_t)T);
        double* dp = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(dynamic, 4)
        for (int x = 0; x < nq; ++x) {
          const int i = qrows[x];
          pattern_row(0, d, q, k, a, r, scale, i, t, p);
          const double* doi = dout + (size_t)i * d;
          double delta = 0.0;
          for (int j = 0; j <= i; ++j) {
            const double* vj = v + (size_t)j * d;
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += doi[c] * vj[c];
            dp[j] = acc;
            delta += p[j] * acc;
          }
          double* dqi = dq + (size_t)x * d;
          for (int c = 0; c < d; ++c) dqi[c] = 0.0;
          for (int j = 0; j <= i; ++j) {
            const double ds = p[j] * (dp[j] - delta);
            const double* kj = k + (size_t)j * d;
            for (int c = 0; c < d; ++c) dqi[c] += scale * ds * kj[c];
          }
        }
        free(t);
        free(p);
        free(dp);
      }
    }
  }
  if (kind == 1 && dk) memset(dk, 0, sizeof(double) * (size_t)nk * d);
  if (!dk && !dv) return 0;

  /* key-side outputs need, for every query row i >= j, the row's normaliser and (ordinary) delta_i.
   * First pass: log normaliser of every row and delta_i of every row. */
  double* lz = (double*)malloc(sizeof(double) * (size_t)T);
  double* dl = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp parallel
  {
    double* t = (double*)malloc(sizeof(double) * (size_t)T);
    double* p = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(dynamic, 8)
    for (int i = 0; i < T; ++i) {
      lz[i] = pattern_row(kind, d, q, k, a, r, scale, i, t, p);
      dl[i] = 0.0;
      if (kind == 0) {
        const double* doi = dout + (size_t)i * d;
        double delta = 0.0;
        for (int j = 0; j <= i; ++j) {
          const double* vj = v + (size_t)j * d;
          double acc = 0.0;
          for (int c = 0; c < d; ++c) acc += doi[c] * vj[c];
          delta += p[j] * acc;
        }
        dl[i] = delta;
      }
    }
    free(t);
    free(p);
  }
  /* Second pass: for each listed key j, sum over the query rows i >= j that see it.
   * P(i,j) = exp(t(i,j) - log normaliser of row i), the same probability as in the forward. */
#pragma omp parallel for schedule(dynamic, 4)
  for (int x = 0; x < nk; ++x) {
    const int j = krows[x];
    double* dkj = dk ? dk + (size_t)x * d : NULL;
    double* dvj = dv ? dv + (size_t)x * d : NULL;
    for (int c = 0; c < d; ++c) {
      if (dkj && kind == 0) dkj[c] = 0.0;
      if (dvj) dvj[c] = 0.0;
    }
    const double* vj = v + (size_t)j * d;
    const double* kj = kind == 0 ? k + (size_t)j * d : NULL;
    for (int i = j; i < T; ++i) {
      double tij;
      if (kind == 0) {
        const double* qi = q + (size_t)i * d;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += qi[c] * kj[c];
        tij = scale * acc;
      } else {
        tij = a[j] + r[i - j];
      }
      const double pij = exp(tij - lz[i]);
      const double* doi = dout + (size_t)i * d;
      if (dvj)
        for (int c = 0; c < d; ++c) dvj[c] += pij * doi[c];
      if (kind == 0 && dkj) {
        double dpij = 0.0;
        for (int c = 0; c < d; ++c) dpij += doi[c] * vj[c];
        const double ds = pij * (dpij - dl[i]);
        const double* qi = q + (size_t)i * d;
        for (int c = 0; c < d; ++c) dkj[c] += scale * ds * qi[c];
      }
    }
  }
  free(lz);
  free(dl);
  return 0;
}

/*
 * Calibration statistics for one head over N sequences, from their queries and keys
 * (q, k: [N][T][d]): the maps A^(n) = softmax_causal(s Q^(n) K^(n)T) are formed row by row and
 * never stored whole.  For each listed row i:
 *   ahat[x][j] = (1/N) sum_n A^(n)(i,j)  (j <= i),  0 for j > i              [Notes §二.1]
 *   dev[x]     = sum_n sum_j (A^(n)(i,j) - ahat(i,j))^2
 * so that, when every row is listed, s_var = sum_x dev[x] / ((N-1) T^2)     [Notes Eq.(1)].
 * ahat may be NULL (deviations only).
 */
ORC_EXPORT int orc_head_calibrate(int N, int T, int d, const double* q, const double* k,
                                  double scale, int nrows, const int* rows, double* ahat,
                                  double* dev) {
  if (N < 2 || T < 1 || d < 1 || !q || !k || !dev || !rows_ok(T, nrows, rows)) return -1;
#pragma omp parallel
  {
    double* t = (double*)malloc(sizeof(double) * (size_t)T);
    double* A = (double*)malloc(sizeof(double) * (size_t)N * T);
    double* mean = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(dynamic, 4)
    for (int x = 0; x < nrows; ++x) {
      const int i = rows[x];
      for (int n = 0; n < N; ++n) {
        const double* qn = q + (size_t)n * T * d;
        const double* kn = k + (size_t)n * T * d;
        ordinary_logits(d, qn, kn, scale, i, t);
        softmax_row(i, t, A + (size_t)n * T);
      }
      for (int j = 0; j <= i; ++j) {
        double s = 0.0;
        for (int n = 0; n < N; ++n) s += A[(size_t)n * T + j];
        mean[j] = s / N;
      }
      double acc = 0.0;
      for (int n = 0; n < N; ++n)
        for (int j = 0; j <= i; ++j) {
          const double e = A[(size_t)n * T + j] - mean[j];
          acc += e * e;
        }
      dev[x] = acc;
      if (ahat) {
        double* ar = ahat + (size_t)x * T;
        for (int j = 0; j < T; ++j) ar[j] = j <= i ? mean[j] : 0.0;
      }
    }
    free(t);
    free(A);
    free(mean);
  }
  return 0;
}

/*
 * Eq. (1) from N dense maps (tiny T only): maps [N][T][T] -> ahat [T][T], *svar.
 * Every one of the T^2 entries counts, as the equation is written.          [Notes §二.1, Eq.(1)]
 */
ORC_EXPORT int orc_calibrate_maps(int N, int T, const double* maps, double* ahat, double* svar) {
  if (N < 2 || T < 1 || !maps || !ahat || !svar) return -1;
  const size_t TT = (size_t)T * T;
  for (size_t e = 0; e < TT; ++e) {
    double s = 0.0;
    for (int n = 0; n < N; ++n) s += maps[(size_t)n * TT + e];
    ahat[e] = s / N;
  }
  double acc = 0.0;
  for (int n = 0; n < N; ++n)
    for (size_t e = 0; e < TT; ++e) {
      const double x = maps[(size_t)n * TT + e] - ahat[e];
      acc += x * x;
    }
  *svar = acc / ((double)(N - 1) * (double)T * (double)T);
  return 0;
}

/*
 * Row-wise forward-KL score of one head (the alternative selector of [Notes §二.1]; the pages name
 * it but print no formula, so the plainest reading is taken: the KL divergence of each sequence's
 * row from the mean row, summed).  For each listed row i:
 *   kl[x] = sum_n sum_{j<=i} A^(n)(i,j) * ln(A^(n)(i,j) / Ahat(i,j)),   Ahat = mean_n A^(n),
 * a term with A^(n)(i,j) = 0 counting 0.  The score of the head is sum_x kl[x] / (N T) over all rows.
 */
ORC_EXPORT int orc_head_kl_score(int N, int T, int d, const double* q, const double* k,
                                 double scale, int nrows, const int* rows, double* kl) {
  if (N < 2 || T < 1 || d < 1 || !q || !k || !kl || !rows_ok(T, nrows, rows)) return -1;
#pragma omp parallel
  {
    double* t = (double*)malloc(sizeof(double) * (size_t)T);
    double* A = (double*)malloc(sizeof(double) * (size_t)N * T);
    double* mean = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(dynamic, 4)
    for (int x = 0; x < nrows; ++x) {
      const int i = rows[x];
      for (int n = 0; n < N; ++n) {
        ordinary_logits(d, q + (size_t)n * T * d, k + (size_t)n * T * d, scale, i, t);
        softmax_row(i, t, A + (size_t)n * T);
      }
      for (int j = 0; j <= i; ++j) {
        double s = 0.0;
        for (int n = 0; n < N; ++n) s += A[(size_t)n * T + j];
        mean[j] = s / N;
      }
      double acc = 0.0;
      for (int n = 0; n < N; ++n)
        for (int j = 0; j <= i; ++j) {
          const double an = A[(size_t)n * T + j];
          if (an > 0.0) acc += an * log(an / mean[j]);
        }
      kl[x] = acc;
    }
    free(t);
    free(A);
    free(mean);
  }
  return 0;
}

/* The same score from N dense maps [N][T][T] (tiny T only): *skl = sum_n sum_i KL / (N T). */
ORC_EXPORT int orc_kl_maps(int N, int T, const double* maps, double* skl) {
  if (N < 2 || T < 1 || !maps || !skl) return -1;
  const size_t TT = (size_t)T * T;
  double acc = 0.0;
  for (size_t e = 0; e < TT; ++e) {
    double s = 0.0;
    for (int n = 0; n < N; ++n) s += maps[(size_t)n * TT + e];
    const double mean = s / N;
    for (int n = 0; n < N; ++n) {
      const double an = maps[(size_t)n * TT + e];
      if (an > 0.0) acc += an * log(an / mean);
    }
  }
  *skl = acc / ((double)N * (double)T);
  return 0;
}

/*
 * Gradient of the loss with respect to a replaced head's pattern logits, one (batch, head) slice
 * (the trainable-pattern variant of [Paper page] Table 14, where a and r are trained instead of
 * frozen).  The pattern row is p_i = softmax over j <= i of t(i,j) = a(j) + r(i-j) ([Notes Eq.(3)])
 * and o_i = sum_j p_i(j) v_j.  With g(i,j) = dL/dp_i(j) = dout_i . v_j the softmax chain rule gives
 *   dL/dt(i,j) = p_i(j) * (g(i,j) - sum_k p_i(k) g(i,k)),
 * and t(i,j) depends on a(j) and r(i-j) with coefficient 1, so
 *   da[j] += sum_{i>=j} dL/dt(i,j),   dr[delta] += sum_i dL/dt(i, i-delta).
 * ACCUMULATES into da[0..T-1] and dr[0..T-1] (the caller sums slices of the same head over batch).
 * Rows are split into contiguous per-thread ranges and the per-thread sums are added in thread
 * order, so a fixed thread count gives the same bits on every run.
 */
ORC_EXPORT int orc_head_pattern_grad(int T, int d, const double* v, const double* dout,
                                     const double* a, const double* r, double* da, double* dr) {
  if (T < 1 || d < 1 || !v || !dout || !a || !r || !da || !dr) return -1;
  int nth = 1;
#ifdef _OPENMP
  nth = omp_get_max_threads();
#endif
  double* part = (double*)calloc((size_t)nth * 2 * T, sizeof(double));
#pragma omp parallel num_threads(nth)
  {
    int th = 0;
#ifdef _OPENMP
    th = omp_get_thread_num();
#endif
    double* pa = part + (size_t)th * 2 * T;
    double* pr = pa + T;
    double* t = (double*)malloc(sizeof(double) * (size_t)T);
    double* p = (double*)malloc(sizeof(double) * (size_t)T);
    double* g = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(static)
    for (int i = 0; i < T; ++i) {
      replaced_logits(a, r, i, t);
      softmax_row(i, t, p);
      const double* gi = dout + (size_t)i * d;
      double pg = 0.0;
      for (int j = 0; j <= i; ++j) {
        const double* vj = v + (size_t)j * d;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += gi[c] * vj[c];
        g[j] = acc;
        pg += p[j] * acc;
      }
      for (int j = 0; j <= i; ++j) {
        const double dt = p[j] * (g[j] - pg);
        pa[j] += dt;
        pr[i - j] += dt;
      }
    }
    free(t);
    free(p);
    free(g);
  }
  for (int th = 0; th < nth; ++th)
    for (int x = 0; x < T; ++x) {
      da[x] += part[(size_t)th * 2 * T + x];
      dr[x] += part[(size_t)th * 2 * T + T + x];
    }
  free(part);
  return 0;
}

/*
 * Compact fit of one head's target pattern Ahat [T][T] by a, r ([Notes §二.3]: the row-wise
 * cross-entropy against the target pattern is minimised; [Notes §二.3] / Appendix A.2: 400 Adam
 * steps, mean row KL at most 0.2 nat to accept).  The loss, averaged over rows, is
 *   L(a, r) = -(1/T) sum_i sum_{j<=i} Ahat(i,j) ln p_i(j),   p_i = softmax_j (a(j) + r(i-j)),
 * and its gradient by the chain rule of the log-softmax is
 *   dL/dt(i,j) = (1/T) (p_i(j) * sum_k Ahat(i,k) - Ahat(i,j)),
 *   dL/da(j) = sum_{i>=j} dL/dt(i,j),   dL/dr(delta) = sum_i dL/dt(i, i-delta).
 * orc_fit_loss_grad evaluates L and (if ga, gr are not NULL) the gradient at (a, r).
 */
ORC_EXPORT int orc_fit_loss_grad(int T, const double* ahat, const double* a, const double* r,
                                 double* loss, double* ga, double* gr) {
  if (T < 1 || !ahat || !a || !r || !loss) return -1;
  double* t = (double*)malloc(sizeof(double) * (size_t)T);
  double* p = (double*)malloc(sizeof(double) * (size_t)T);
  if (ga) memset(ga, 0, sizeof(double) * (size_t)T);
  if (gr) memset(gr, 0, sizeof(double) * (size_t)T);
  double L = 0.0;
  for (int i = 0; i < T; ++i) {
    const double* ai = ahat + (size_t)i * T;
    replaced_logits(a, r, i, t);
    const double lz = softmax_row(i, t, p);
    double rowsum = 0.0;
    for (int j = 0; j <= i; ++j) {
      rowsum += ai[j];
      if (ai[j] != 0.0) L -= ai[j] * (t[j] - lz);  /* ln p_i(j) = t(i,j) - ln Z(i) */
    }
    if (ga || gr)
      for (int j = 0; j <= i; ++j) {
        const double g = (p[j] * rowsum - ai[j]) / T;
        if (ga) ga[j] += g;
        if (gr) gr[i - j] += g;
      }
  }
  *loss = L / T;
  free(t);
  free(p);
  return 0;
}

/*
 * The fit itself: a = r = 0 (the uniform causal pattern), then `steps` Adam updates of (a, r) on L
 * with step size lr and the usual moment rates (beta1 = 0.9, beta2 = 0.999, eps = 1e-8, bias
 * correction on both moments).  On return a, r hold the fitted logits, *loss the final L and *kl
 * the mean row KL(Ahat_i || p_i) = L + (1/T) sum Ahat ln Ahat (the acceptance measure).
 */
ORC_EXPORT int orc_fit_pattern(int T, const double* ahat, int steps, double lr, double* a,
                               double* r, double* loss, double* kl) {
  if (T < 1 || steps < 0 || !(lr > 0.0) || !ahat || !a || !r || !loss || !kl) return -1;
  const double b1 = 0.9, b2 = 0.999, eps = 1e-8;
  double* g = (double*)malloc(sizeof(double) * 2 * (size_t)T);
  double* m = (double*)calloc(2 * (size_t)T, sizeof(double));
  double* v = (double*)calloc(2 * (size_t)T, sizeof(double));
  memset(a, 0, sizeof(double) * (size_t)T);
  memset(r, 0, sizeof(double) * (size_t)T);
  double L = 0.0;
  for (int s = 1; s <= steps; ++s) {
    orc_fit_loss_grad(T, ahat, a, r, &L, g, g + T);
    const double c1 = 1.0 - pow(b1, s), c2 = 1.0 - pow(b2, s);
    for (int x = 0; x < 2 * T; ++x) {
      m[x] = b1 * m[x] + (1.0 - b1) * g[x];
      v[x] = b2 * v[x] + (1.0 - b2) * g[x] * g[x];
      double* w = x < T ? &a[x] : &r[x - T];
      *w -= lr * (m[x] / c1) / (sqrt(v[x] / c2) + eps);
    }
  }
  orc_fit_loss_grad(T, ahat, a, r, &L, NULL, NULL);
  double ent = 0.0;
  for (size_t e = 0; e < (size_t)T * T; ++e)
    if (ahat[e] > 0.0) ent += ahat[e] * log(ahat[e]);
  *loss = L;
  *kl = L + ent / T;
  free(g);
  free(m);
  free(v);
  return 0;
}

/* Number of threads the parallel loops above use (for reporting the CPU baseline). */
ORC_EXPORT int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
