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

/* Number of threads the parallel loops above use (for reporting the CPU baseline). */
ORC_EXPORT int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
