/*
 * attn_oracle.c -- plain, slow, fp64 CPU oracle for the exact attention forward pass.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this file. The product path (the HIP library)
 * never links, imports or falls back to it, and this file shares no code, header,
 * table or helper with that library.
 *
 * What it computes. Standard attention as written out on the page "FlashAttention:
 * The Algorithm That Made Long-Context AI Possible" (section "The quadratic
 * bottleneck in standard attention"): a score matrix S = Q K^T and the output
 * O = softmax(S) V. The tiled method of the FlashAttention pages (abstract of
 * "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness";
 * section "What tiling changes" of the page above) reaches exactly this result in
 * real arithmetic, so the oracle is the definition itself: no tiling, no online
 * softmax, two passes per query row, everything in IEEE double.
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *   - scores are multiplied by `scale` before the softmax;
 *   - causal masking keeps key j for query i iff j <= i (square, no offset);
 *   - a key window (the sliding-window patterns that the section "Why context lengths
 *     exploded after 2022" of the long-context page above names without defining) keeps
 *     i - left <= j <= i + right on top of the mask, a negative bound meaning no limit
 *     on that side; every query keeps at least its own key, so no row is empty;
 *   - grouped-query attention maps query head h to key/value head h / (H / Hkv);
 *   - lse is the natural log of the softmax denominator over the scaled scores,
 *     lse = m + ln(sum_j exp(s_j - m)), so that P_ij = exp(s_ij - lse_i);
 *   - the inputs are the exact values of the bf16 / f16 / e4m3 elements handed to
 *     the GPU library; an e4m3 element is multiplied by its tensor's descale.
 *
 * Layouts (row-major, contiguous): q, o [B][N][H][d]; k, v [B][N][Hkv][d];
 * lse [B][H][N].
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math: the order of every sum is
 * the ascending index order written below).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element decoders (exact conversion of a storage format to double) ---- */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 0x1f, f = h & 0x3ff;
  double mag;
  if (e == 0) mag = ldexp((double)f, -24);                  /* subnormal: f * 2^-14 * 2^-10 */
  else if (e == 31) mag = f ? NAN : INFINITY;
  else mag = ldexp((double)(1024 + f), e - 25);              /* (1 + f/1024) * 2^(e-15) */
  return sign ? -mag : mag;
}

/* bfloat16: the upper half of an IEEE binary32. */
double oracle_decode_bf16(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 7) & 0xff, f = h & 0x7f;
  double mag;
  if (e == 0) mag = ldexp((double)f, -133);                 /* f * 2^-126 * 2^-7 */
  else if (e == 255) mag = f ? NAN : INFINITY;
  else mag = ldexp((double)(128 + f), e - 134);              /* (1 + f/128) * 2^(e-127) */
  return sign ? -mag : mag;
}

/* OCP 8-bit E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits, no
 * infinities, S.1111.111 is NaN, largest finite magnitude 448. */
double oracle_decode_e4m3(uint8_t x) {
  int sign = (x >> 7) & 1, e = (x >> 3) & 0xf, f = x & 7;
  double mag;
  if (e == 15 && f == 7) mag = NAN;
  else if (e == 0) mag = ldexp((double)f, -9);              /* f/8 * 2^-6 */
  else mag = ldexp((double)(8 + f), e - 10);                 /* (1 + f/8) * 2^(e-7) */
  return sign ? -mag : mag;
}

/* dtype codes: 0 = f16, 1 = bf16, 2 = e4m3. Writes n doubles: decode(src[i]) * mult. */
int oracle_decode(int dtype, const void* src, int64_t n, double mult, double* dst) {
  if (n < 0 || (n > 0 && (!src || !dst))) return 1;
  for (int64_t i = 0; i < n; ++i) {
    double x;
    if (dtype == 0) x = oracle_decode_f16(((const uint16_t*)src)[i]);
    else if (dtype == 1) x = oracle_decode_bf16(((const uint16_t*)src)[i]);
    else if (dtype == 2) x = oracle_decode_e4m3(((const uint8_t*)src)[i]);
    else return 1;
    dst[i] = x * mult;
  }
  return 0;
}

/* ---- one query row ---- */

/* Scores, max, exponentials, denominator and output for one query row `qi` of batch b
 * against key/value head hk over the visible keys jlo <= j <= jhi (a non-empty range).
 * `s` is caller scratch of N doubles. Writes o_row[0..d) and *lse. */
static void attn_row(const double* qi, const double* k, const double* v, int Hkv, int N, int d,
                     int jlo, int jhi, double scale, int b, int hk, double* s, double* o_row,
                     double* lse) {
  /* pass 1: s_j = scale * <q_i, k_j>, and the row maximum */
  double m = -INFINITY;
  for (int j = jlo; j <= jhi; ++j) {
    const double* kj = k + (((size_t)b * N + j) * Hkv + hk) * d;
    double dot = 0.0;
    for (int t = 0; t < d; ++t) dot += qi[t] * kj[t];
    s[j] = scale * dot;
    if (s[j] > m) m = s[j];
  }
  /* pass 2: e_j = exp(s_j - m), l = sum_j e_j, o = sum_j e_j v_j / l */
  for (int t = 0; t < d; ++t) o_row[t] = 0.0;
  double l = 0.0;
  for (int j = jlo; j <= jhi; ++j) {
    const double e = exp(s[j] - m);
    const double* vj = v + (((size_t)b * N + j) * Hkv + hk) * d;
    l += e;
    for (int t = 0; t < d; ++t) o_row[t] += e * vj[t];
  }
  for (int t = 0; t < d; ++t) o_row[t] /= l;
  *lse = m + log(l);
}

/* Visible keys of query i: causal keeps j <= i; a key window keeps i - left <= j <= i + right
 * (a negative bound means no limit on that side). */
static void key_range(int i, int N, int causal, int left, int right, int* jlo, int* jhi) {
  int lo = 0, hi = causal ? i : N - 1;
  if (left >= 0 && i - left > lo) lo = i - left;
  if (right >= 0 && i + right < hi) hi = i + right;
  *jlo = lo;
  *jhi = hi;
}

static int check_shape(int B, int H, int Hkv, int N, int d) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1 || d < 1) return 1;
  if (Hkv > H || H % Hkv != 0) return 1;
  return 0;
}

/* Full forward over every (b, h, i). Returns 0 on success, 1 on bad arguments,
 * 2 if scratch allocation failed. */
int oracle_attn_fwd_local_f64(const double* q, const double* k, const double* v, double* o,
                              double* lse, int B, int H, int Hkv, int N, int d, int causal,
                              int left, int right, double scale) {
  if (check_shape(B, H, Hkv, N, d) || !q || !k || !v || !o || !lse) return 1;
  const int64_t rows = (int64_t)B * H * N;
  const int group = H / Hkv;                                 /* grouped-query head map h -> h / group */
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    if (!s) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 8)
    for (int64_t r = 0; r < rows; ++r) {
      if (!s) continue;
      const int i = (int)(r % N), h = (int)((r / N) % H), b = (int)(r / ((int64_t)N * H));
      const size_t qo = (((size_t)b * N + i) * H + h) * d;
      int jlo, jhi;
      key_range(i, N, causal, left, right, &jlo, &jhi);
      attn_row(q + qo, k, v, Hkv, N, d, jlo, jhi, scale, b, h / group, s, o + qo,
               lse + ((size_t)b * H + h) * N + i);
    }
    free(s);
  }
  return failed ? 2 : 0;
}

/* Full forward without a key window. */
int oracle_attn_fwd_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                        int B, int H, int Hkv, int N, int d, int causal, double scale) {
  return oracle_attn_fwd_local_f64(q, k, v, o, lse, B, H, Hkv, N, d, causal, -1, -1, scale);
}

/* Selected rows only: rows[3r], rows[3r+1], rows[3r+2] = (b, h, i). o_rows is
 * [nrows][d], lse_rows [nrows]. q is either a full [B][N][H][d] tensor
 * (q_is_rows = 0) or the selected query rows gathered as [nrows][d] (q_is_rows = 1),
 * so that a caller need not decode a whole large Q to check a sample. */
int oracle_attn_rows_local_f64(const double* q, int q_is_rows, const double* k, const double* v,
                               int B, int H, int Hkv, int N, int d, int causal, int left,
                               int right, double scale, int64_t nrows, const int64_t* rows,
                               double* o_rows, double* lse_rows) {
  if (check_shape(B, H, Hkv, N, d) || !q || !k || !v || !rows || !o_rows || !lse_rows) return 1;
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
    if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N) return 1;
  }
  const int group = H / Hkv;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    if (!s) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!s) continue;
      const int b = (int)rows[3 * r], h = (int)rows[3 * r + 1], i = (int)rows[3 * r + 2];
      const double* qi = q_is_rows ? q + (size_t)r * d : q + (((size_t)b * N + i) * H + h) * d;
      int jlo, jhi;
      key_range(i, N, causal, left, right, &jlo, &jhi);
      attn_row(qi, k, v, Hkv, N, d, jlo, jhi, scale, b, h / group, s, o_rows + (size_t)r * d,
               lse_rows + r);
    }
    free(s);
  }
  return failed ? 2 : 0;
}

int oracle_attn_rows_f64(const double* q, int q_is_rows, const double* k, const double* v,
                         int B, int H, int Hkv, int N, int d, int causal, double scale,
                         int64_t nrows, const int64_t* rows, double* o_rows, double* lse_rows) {
  return oracle_attn_rows_local_f64(q, q_is_rows, k, v, B, H, Hkv, N, d, causal, -1, -1, scale,
                                    nrows, rows, o_rows, lse_rows);
}

/* Softmax probabilities of one (b, h) as an N x N matrix (row i, key j), zero where
 * masked. For small N only: used to check that rows sum to one. */
int oracle_attn_probs_local_f64(const double* q, const double* k, int B, int H, int Hkv, int N,
                                int d, int causal, int left, int right, double scale, int b, int h,
                                double* p) {
  if (check_shape(B, H, Hkv, N, d) || !q || !k || !p || b < 0 || b >= B || h < 0 || h >= H)
    return 1;
  const int hk = h / (H / Hkv);
  for (int i = 0; i < N; ++i) {
    const double* qi = q + (((size_t)b * N + i) * H + h) * d;
    double* pi = p + (size_t)i * N;
    int jlo, jhi;
    key_range(i, N, causal, left, right, &jlo, &jhi);
    double m = -INFINITY, l = 0.0;
    for (int j = 0; j < N; ++j) pi[j] = 0.0;
    for (int j = jlo; j <= jhi; ++j) {
      const double* kj = k + (((size_t)b * N + j) * Hkv + hk) * d;
      double dot = 0.0;
      for (int t = 0; t < d; ++t) dot += qi[t] * kj[t];
      pi[j] = scale * dot;
      if (pi[j] > m) m = pi[j];
    }
    for (int j = jlo; j <= jhi; ++j) {
      pi[j] = exp(pi[j] - m);
      l += pi[j];
    }
    for (int j = jlo; j <= jhi; ++j) pi[j] /= l;
  }
  return 0;
}

int oracle_attn_probs_f64(const double* q, const double* k, int B, int H, int Hkv, int N, int d,
                          int causal, double scale, int b, int h, double* p) {
  return oracle_attn_probs_local_f64(q, k, B, H, Hkv, N, d, causal, -1, -1, scale, b, h, p);
}

/* Rectangular forward: Nq queries against Nk keys (q, o [B][Nq][H][d]; k, v [B][Nk][Hkv][d];
 * lse [B][H][Nq]). Query i sits at sequence position Nk - Nq + i, the queries being the last
 * Nq positions of a sequence whose keys are all Nk positions (decode); under the causal mask
 * it sees keys j <= Nk - Nq + i. Nq <= Nk. With Nq = Nk this is oracle_attn_fwd_f64. */
int oracle_attn_fwd_kv_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                           int B, int H, int Hkv, int Nq, int Nk, int d, int causal, double scale) {
  if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < Nq || d < 1 || Hkv > H || H % Hkv) return 1;
  if (!q || !k || !v || !o || !lse) return 1;
  const int64_t rows = (int64_t)B * H * Nq;
  const int group = H / Hkv;
  int failed = 0;
#pragma omp parallel reduction(| : failed)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
    if (!s) failed = 1;
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
      if (!s) continue;
      const int i = (int)(r % Nq), h = (int)((r / Nq) % H), b = (int)(r / ((int64_t)Nq * H));
      const size_t qo = (((size_t)b * Nq + i) * H + h) * d;
      const int pos = Nk - Nq + i;                            /* the query's sequence position */
      attn_row(q + qo, k, v, Hkv, Nk, d, 0, causal ? pos : Nk - 1, scale, b, h / group, s, o + qo,
               lse + ((size_t)b * H + h) * Nq + i);
    }
    free(s);
  }
  return failed ? 2 : 0;
}

/* ---- block-sparse attention ----
 * The approximate variant named in the abstract of "FlashAttention: Fast and Memory-
 * Efficient Exact Attention with IO-Awareness" (block-sparse FlashAttention), which the
 * pages do not define further. Reading: a 0/1 mask over blocks of `block` queries x
 * `block` keys says which blocks are computed; key j is visible to query i iff
 *     mask[hm][i / block][j / block] != 0   (and j <= i when causal),
 * hm = 0 when the mask is shared by every head (mask_heads = 1), else the query head h
 * (mask_heads = H). The attention over the visible keys is then exact. A row with no
 * visible key has no softmax; its output is taken as O = 0 and lse = -inf.
 * mask is [mask_heads][nb][nb] bytes, nb = ceil(N / block). */

/* One row over the keys with keep[j] != 0 (any subset of 0..N-1). */
static void attn_row_keep(const double* qi, const double* k, const double* v, int Hkv, int N, int d,
                          const unsigned char* keep, double scale, int b, int hk, double* s,
                          double* o_row, double* lse) {
  double m = -INFINITY;
  for (int j = 0; j < N; ++j) {
    if (!keep[j]) continue;
    const double* kj = k + (((size_t)b * N + (size_t)j) * Hkv + hk) * d;
    double dot = 0.0;
    for (int t = 0; t < d; ++t) dot += qi[t] * kj[t];
    s[j] = scale * dot;
    if (s[j] > m) m = s[j];
  }
  for (int t = 0; t < d; ++t) o_row[t] = 0.0;
  if (m == -INFINITY) {                      /* no visible key */
    *lse = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int j = 0; j < N; ++j) {
    if (!keep[j]) continue;
    const double e = exp(s[j] - m);
    const double* vj = v + (((size_t)b * N + (size_t)j) * Hkv + hk) * d;
    l += e;
    for (int t = 0; t < d; ++t) o_row[t] += e * vj[t];
  }
  for (int t = 0; t < d; ++t) o_row[t] /= l;
  *lse = m + log(l);
}

static void block_keep(const unsigned char* mask, int mask_heads, int block, int N, int causal, int h,
                       int i, unsigned char* keep) {
  const int nb = (N + block - 1) / block;
  const unsigned char* row = mask + ((size_t)(mask_heads == 1 ? 0 : h) * nb + i / block) * nb;
  for (int j = 0; j < N; ++j) keep[j] = row[j / block] != 0 && (!causal || j <= i);
}

int oracle_attn_fwd_block_f64(const double* q, const double* k, const double* v, double* o,
                              double* lse, int B, int H, int Hkv, int N, int d, int causal,
                              const unsigned char* mask, int mask_heads, int block, double scale) {
  if (check_shape(B, H, Hkv, N, d) || !q || !k || !v || !o || !lse || !mask || block < 1) return 1;
  if (mask_heads != 1 && mask_heads != H) return 1;
  const int64_t rows = (int64_t)B * H * N;
  const int group = H / Hkv;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    unsigned char* keep = (unsigned char*)malloc((size_t)N);
    if (!s || !keep) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 8)
    for (int64_t r = 0; r < rows; ++r) {
      if (!s || !keep) continue;
      const int i = (int)(r % N), h = (int)((r / N) % H), b = (int)(r / ((int64_t)N * H));
      const size_t qo = (((size_t)b * N + i) * H + h) * d;
      block_keep(mask, mask_heads, block, N, causal, h, i, keep);
      attn_row_keep(q + qo, k, v, Hkv, N, d, keep, scale, b, h / group, s, o + qo,
                    lse + ((size_t)b * H + h) * N + i);
    }
    free(s);
    free(keep);
  }
  return failed ? 2 : 0;
}

/* Selected rows (as oracle_attn_rows_local_f64) under a block mask. */
int oracle_attn_rows_block_f64(const double* q, int q_is_rows, const double* k, const double* v,
                               int B, int H, int Hkv, int N, int d, int causal,
                               const unsigned char* mask, int mask_heads, int block, double scale,
                               int64_t nrows, const int64_t* rows, double* o_rows, double* lse_rows) {
  if (check_shape(B, H, Hkv, N, d) || !q || !k || !v || !rows || !o_rows || !lse_rows || !mask ||
      block < 1)
    return 1;
  if (mask_heads != 1 && mask_heads != H) return 1;
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
    if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N) return 1;
  }
  const int group = H / Hkv;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    unsigned char* keep = (unsigned char*)malloc((size_t)N);
    if (!s || !keep) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!s || !keep) continue;
      const int b = (int)rows[3 * r], h = (int)rows[3 * r + 1], i = (int)rows[3 * r + 2];
      const double* qi = q_is_rows ? q + (size_t)r * d : q + (((size_t)b * N + i) * H + h) * d;
      block_keep(mask, mask_heads, block, N, causal, h, i, keep);
      attn_row_keep(qi, k, v, Hkv, N, d, keep, scale, b, h / group, s, o_rows + (size_t)r * d,
                    lse_rows + r);
    }
    free(s);
    free(keep);
  }
  return failed ? 2 : 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
