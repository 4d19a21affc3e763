/*
 * attn_bwd_oracle.c -- plain, slow, fp64 CPU oracle for the gradient of the exact
 * attention forward pass.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this file. The product path (the HIP library)
 * never links, imports or falls back to it, and this file shares no code, header,
 * table or helper with that library.
 *
 * What it computes. The pages report training speed-ups (abstract of "FlashAttention-2:
 * Faster Attention with Better Parallelism and Work Partitioning"; abstract of
 * "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"), so a
 * backward pass exists, but they print no algorithm for it. This oracle is therefore the
 * analytic gradient of the forward definition (S = scale Q K^T with the mask,
 * P = softmax(S) row by row, O = P V), for a loss L whose gradient with respect to O is
 * dO, taking no gradient through lse:
 *     dV_j  = sum_i P_ij dO_i
 *     dP_ij = <dO_i, v_j>,   D_i = sum_j P_ij dP_ij  (= <dO_i, O_i>)
 *     dS_ij = P_ij (dP_ij - D_i)
 *     dQ_i  = scale sum_j dS_ij k_j
 *     dK_j  = scale sum_i dS_ij q_i
 * With grouped-query attention, dK and dV of a key/value head sum over the query heads
 * h with h / (H / Hkv) equal to it. Masking and key windows as in attn_oracle.c: masked
 * pairs have P_ij = 0 and contribute nothing.
 *
 * Layouts: q, o, dout, dq [B][N][H][d]; k, v, dk, dv [B][N][Hkv][d].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void visible_keys(int i, int N, int causal, int left, int right, int* jlo, int* jhi) {
  int lo = 0, hi = causal ? i : N - 1;
  if (left >= 0 && i - left > lo) lo = i - left;
  if (right >= 0 && i + right < hi) hi = i + right;
  *jlo = lo;
  *jhi = hi;
}

/* Returns 0, 1 on bad arguments, 2 if scratch allocation failed. dq, dk, dv are
 * overwritten. Serial over (b, kv head), so that dK and dV sum in a fixed order. */
int oracle_attn_bwd_f64(const double* q, const double* k, const double* v, const double* dout,
                        double* dq, double* dk, double* dv, int B, int H, int Hkv, int N, int d,
                        int causal, int left, int right, double scale) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1 || d < 1 || Hkv > H || H % Hkv) return 1;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return 1;
  const int group = H / Hkv;
  double* p = (double*)malloc(sizeof(double) * (size_t)N);
  double* dp = (double*)malloc(sizeof(double) * (size_t)N);
  if (!p || !dp) {
    free(p);
    free(dp);
    return 2;
  }
  memset(dk, 0, sizeof(double) * (size_t)B * N * Hkv * d);
  memset(dv, 0, sizeof(double) * (size_t)B * N * Hkv * d);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const int hk = h / group;
      for (int i = 0; i < N; ++i) {
        const double* qi = q + (((size_t)b * N + i) * H + h) * d;
        const double* gi = dout + (((size_t)b * N + i) * H + h) * d;
        double* dqi = dq + (((size_t)b * N + i) * H + h) * d;
        int jlo, jhi;
        visible_keys(i, N, causal, left, right, &jlo, &jhi);
        /* P row: scores, max, exponentials, normalisation */
        double m = -INFINITY;
        for (int j = jlo; j <= jhi; ++j) {
          const double* kj = k + (((size_t)b * N + j) * Hkv + hk) * d;
          double s = 0.0;
          for (int t = 0; t < d; ++t) s += qi[t] * kj[t];
          p[j] = scale * s;
          if (p[j] > m) m = p[j];
        }
        double l = 0.0;
        for (int j = jlo; j <= jhi; ++j) {
          p[j] = exp(p[j] - m);
          l += p[j];
        }
        for (int j = jlo; j <= jhi; ++j) p[j] /= l;
        /* dP_ij = <dO_i, v_j> and D_i = sum_j P_ij dP_ij */
        double D = 0.0;
        for (int j = jlo; j <= jhi; ++j) {
          const double* vj = v + (((size_t)b * N + j) * Hkv + hk) * d;
          double s = 0.0;
          for (int t = 0; t < d; ++t) s += gi[t] * vj[t];
          dp[j] = s;
          D += p[j] * s;
        }
        for (int t = 0; t < d; ++t) dqi[t] = 0.0;
        for (int j = jlo; j <= jhi; ++j) {
          const double ds = p[j] * (dp[j] - D);
          const double* kj = k + (((size_t)b * N + j) * Hkv + hk) * d;
          double* dkj = dk + (((size_t)b * N + j) * Hkv + hk) * d;
          double* dvj = dv + (((size_t)b * N + j) * Hkv + hk) * d;
          for (int t = 0; t < d; ++t) {
            dqi[t] += scale * ds * kj[t];
            dkj[t] += scale * ds * qi[t];
            dvj[t] += p[j] * gi[t];
          }
        }
      }
    }
  free(p);
  free(dp);
  return 0;
}

/* dQ of selected query rows only (rows[3r..3r+2] = (b, h, i)), for checking large problems:
 * row i of dQ needs only row i of P and dP. dq_rows is [nrows][d]. mag, when not NULL, is
 * [nrows][2][d]: sum_j |dS_ij| |k_j| and sum_j P_ij |k_j| (elementwise absolute values), the
 * sizes that bound the rounding error of a computed dQ row. */
int oracle_attn_bwd_dq_rows_f64(const double* q, const double* k, const double* v,
                                const double* dout, int B, int H, int Hkv, int N, int d,
                                int causal, double scale, int64_t nrows, const int64_t* rows,
                                double* dq_rows, double* mag) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1 || d < 1 || Hkv > H || H % Hkv) return 1;
  if (!q || !k || !v || !dout || !rows || !dq_rows) return 1;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= H ||
        rows[3 * r + 2] < 0 || rows[3 * r + 2] >= N)
      return 1;
  const int group = H / Hkv;
  int failed = 0;
#pragma omp parallel reduction(| : failed)
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)N);
    double* dp = (double*)malloc(sizeof(double) * (size_t)N);
    if (!p || !dp) failed = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!p || !dp) continue;
      const int b = (int)rows[3 * r], h = (int)rows[3 * r + 1], i = (int)rows[3 * r + 2];
      const int hk = h / group;
      const double* qi = q + (((size_t)b * N + i) * H + h) * d;
      const double* gi = dout + (((size_t)b * N + i) * H + h) * d;
      double* dqi = dq_rows + (size_t)r * d;
      int jlo, jhi;
      visible_keys(i, N, causal, -1, -1, &jlo, &jhi);
      double m = -INFINITY;
      for (int j = jlo; j <= jhi; ++j) {
        const double* kj = k + (((size_t)b * N + j) * Hkv + hk) * d;
        double s = 0.0;
        for (int t = 0; t < d; ++t) s += qi[t] * kj[t];
        p[j] = scale * s;
        if (p[j] > m) m = p[j];
      }
      double l = 0.0;
      for (int j = jlo; j <= jhi; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
      }
      for (int j = jlo; j <= jhi; ++j) p[j] /= l;
      double D = 0.0;
      for (int j = jlo; j <= jhi; ++j) {
        const double* vj = v + (((size_t)b * N + j) * Hkv + hk) * d;
        double s = 0.0;
        for (int t = 0; t < d; ++t) s += gi[t] * vj[t];
        dp[j] = s;
        D += p[j] * s;
      }
      for (int t = 0; t < d; ++t) dqi[t] = 0.0;
      for (int j = jlo; j <= jhi; ++j) {
        const double ds = p[j] * (dp[j] - D);
        const double* kj = k + (((size_t)b * N + j) * Hkv + hk) * d;
        for (int t = 0; t < d; ++t) dqi[t] += scale * ds * kj[t];
      }
      if (mag) {
        double* m1 = mag + (size_t)r * 2 * d;
        double* m2 = m1 + d;
        for (int t = 0; t < d; ++t) m1[t] = m2[t] = 0.0;
        for (int j = jlo; j <= jhi; ++j) {
          const double ads = fabs(p[j] * (dp[j] - D));
          const double* kj = k + (((size_t)b * N + j) * Hkv + hk) * d;
          for (int t = 0; t < d; ++t) {
            m1[t] += ads * fabs(kj[t]);
            m2[t] += p[j] * fabs(kj[t]);
          }
        }
      }
    }
    free(p);
    free(dp);
  }
  return failed ? 2 : 0;
}

/* dK and dV of selected key rows only (rows[3r..3r+2] = (b, hk, j), hk a key/value head),
 * for checking large problems. Key j's gradient sums over every query row i that sees it
 * (i >= j under the causal mask, every i otherwise) in every query head h of its group, in
 * ascending (h, i) order. The probabilities come from the forward's lse,
 * P_ij = exp(s_ij - lse_i), and D_i = <dO_i, O_i> from the forward's O: both are the values
 * oracle_attn_fwd_f64 returns for the same inputs (passed in, [B][H][N] and [B][N][H][d]),
 * and both equal what oracle_attn_bwd_f64 forms row by row, in real arithmetic.
 * dk_rows, dv_rows: [nrows][d]. mag, when not NULL, is [nrows][3][d]: sum_i |dS_ij| |q_i|,
 * sum_i P_ij w_i |q_i| with w_i = sum_t |dO_it O_it|, and sum_i P_ij |dO_i|, the sizes that
 * bound the rounding error of computed dK and dV rows. Returns 0, 1 on bad arguments,
 * 2 if scratch allocation failed. */
int oracle_attn_bwd_dkdv_rows_f64(const double* q, const double* k, const double* v,
                                  const double* dout, const double* o, const double* lse,
                                  int B, int H, int Hkv, int N, int d, int causal, double scale,
                                  int64_t nrows, const int64_t* rows, double* dk_rows,
                                  double* dv_rows, double* mag) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1 || d < 1 || Hkv > H || H % Hkv) return 1;
  if (!q || !k || !v || !dout || !o || !lse || !rows || !dk_rows || !dv_rows) return 1;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= Hkv ||
        rows[3 * r + 2] < 0 || rows[3 * r + 2] >= N)
      return 1;
  const int group = H / Hkv;
  const size_t nq = (size_t)B * H * N;           /* D and w per (b, h, i), [B][H][N] */
  double* D = (double*)malloc(sizeof(double) * nq);
  double* w = (double*)malloc(sizeof(double) * nq);
  if (!D || !w) {
    free(D);
    free(w);
    return 2;
  }
#pragma omp parallel for schedule(static)
  for (int64_t x = 0; x < (int64_t)nq; ++x) {
    const int i = (int)(x % N), h = (int)((x / N) % H), b = (int)(x / ((int64_t)N * H));
    const double* gi = dout + (((size_t)b * N + i) * H + h) * d;
    const double* oi = o + (((size_t)b * N + i) * H + h) * d;
    double s = 0.0, a = 0.0;
    for (int t = 0; t < d; ++t) {
      s += gi[t] * oi[t];
      a += fabs(gi[t] * oi[t]);
    }
    D[x] = s;
    w[x] = a;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int b = (int)rows[3 * r], hk = (int)rows[3 * r + 1], j = (int)rows[3 * r + 2];
    const double* kj = k + (((size_t)b * N + j) * Hkv + hk) * d;
    const double* vj = v + (((size_t)b * N + j) * Hkv + hk) * d;
    double* dkj = dk_rows + (size_t)r * d;
    double* dvj = dv_rows + (size_t)r * d;
    double* m1 = mag ? mag + (size_t)r * 3 * d : NULL;
    for (int t = 0; t < d; ++t) dkj[t] = dvj[t] = 0.0;
    if (m1)
      for (int t = 0; t < 3 * d; ++t) m1[t] = 0.0;
    for (int h = hk * group; h < (hk + 1) * group; ++h)
      for (int i = causal ? j : 0; i < N; ++i) {
        const double* qi = q + (((size_t)b * N + i) * H + h) * d;
        const double* gi = dout + (((size_t)b * N + i) * H + h) * d;
        const size_t row = ((size_t)b * H + h) * N + i;
        double s = 0.0, dp = 0.0;
        for (int t = 0; t < d; ++t) {
          s += qi[t] * kj[t];
          dp += gi[t] * vj[t];
        }
        const double p = exp(scale * s - lse[row]);
        const double ds = p * (dp - D[row]);
        for (int t = 0; t < d; ++t) {
          dkj[t] += scale * ds * qi[t];
          dvj[t] += p * gi[t];
        }
        if (m1)
          for (int t = 0; t < d; ++t) {
            m1[t] += fabs(ds) * fabs(qi[t]);
            m1[d + t] += p * w[row] * fabs(qi[t]);
            m1[2 * d + t] += p * fabs(gi[t]);
          }
      }
  }
  free(D);
  free(w);
  return 0;
}
