/*
 * fp8_quant_oracle.c -- plain CPU oracle for block quantisation of attention inputs to
 * OCP E4M3 with power-of-two block scales, optionally after incoherent processing.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this file. The product path (the HIP library)
 * never links, imports or falls back to it, and this file shares no code, header,
 * table or helper with that library.
 *
 * What it computes. The abstract of "FlashAttention-3: Fast and Accurate Attention with
 * Asynchrony and Low-precision" names two techniques for its FP8 mode, block
 * quantisation and incoherent processing, and reports lower error than a baseline FP8
 * attention; the reference list of the same page names QuIP# (Hadamard incoherence).
 * The pages define neither step; this oracle takes the plainest reading:
 *   - block quantisation: every run of `block_rows` consecutive sequence positions of
 *     one (batch, head) -- a block_rows x d slab -- has its own scale; the scale is a
 *     power of two 2^e (the shared-exponent E8M0 form), with e the smallest integer such
 *     that the slab's largest magnitude times 2^-e is at most 448 (the largest E4M3
 *     value), floored at -127; an all-zero slab has e = 0;
 *   - element code = E4M3 round-to-nearest-even of x * 2^-e (saturated to +-448; exact
 *     scaling, so the scale itself adds no rounding);
 *   - incoherent processing (Q and K only): before quantising, each row x (length d) is
 *     replaced by (x * s) H, with s a vector of random signs (an input, drawn by the
 *     caller) and H the d x d Sylvester-Hadamard matrix (entries +-1, H H^T = d I), so
 *     that (q s H).(k s H) = d q.k: attention on rotated Q and K with the score scale
 *     divided by d is attention on the originals. The rotation runs in IEEE single
 *     precision with the fast Walsh-Hadamard butterfly order below -- the precision the
 *     GPU takes its rounding decisions in -- so that both sides reach the same codes.
 *
 * Layouts: x, codes [B][N][Hx][d]; scales [B][Hx][ceil(N / block_rows)], one E8M0 byte
 * each (value 2^(byte - 127)).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* E4M3 code of a finite value y (round to nearest, ties to the even code; |y| > 448 is
 * clamped to 448 first; NaN gives 0x7F). Magnitudes: subnormal m * 2^-9 (m = 1..7),
 * normal (1 + m/8) * 2^(E) for E = -6..8, except E = 8, m = 7 (NaN). Works in double, in
 * which every float input and every step below is exact. */
uint8_t oracle_e4m3_encode(float yf) {
  const double y = (double)yf;
  if (isnan(y)) return 0x7F;
  const int neg = signbit(y) ? 1 : 0;
  double a = fabs(y);
  if (a > 448.0) a = 448.0;
  uint8_t code;
  if (a < ldexp(1.0, -6)) {
    /* subnormal quantum 2^-9; m = 8 is the smallest normal, whose code is 0x08 */
    code = (uint8_t)rint(a * 512.0);
  } else {
    int e2;
    frexp(a, &e2);                       /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    double m = rint(ldexp(a, 3 - E));    /* significand in eighths, 8..16 */
    if (m == 16.0) {
      E += 1;
      m = 8.0;
    }
    code = (uint8_t)(((E + 7) << 3) | ((int)m - 8));
  }
  return neg ? (uint8_t)(code | 0x80) : code;
}

int oracle_e4m3_encode_array(const float* y, int64_t n, uint8_t* codes) {
  if (n < 0 || (n > 0 && (!y || !codes))) return 1;
  for (int64_t i = 0; i < n; ++i) codes[i] = oracle_e4m3_encode(y[i]);
  return 0;
}

/* Unnormalised fast Walsh-Hadamard transform of one row of length d (a power of two),
 * in single precision: for h = 1, 2, 4, ..., d/2 and every j with bit h clear,
 * (x_j, x_{j+h}) <- (x_j + x_{j+h}, x_j - x_{j+h}). The result is x H with H the
 * Sylvester-Hadamard matrix (H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]). */
void oracle_fwht_f32(float* x, int d) {
  for (int h = 1; h < d; h <<= 1)
    for (int j = 0; j < d; ++j)
      if ((j & h) == 0) {
        const float a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
}

int oracle_fwht_rows_f32(float* x, int64_t rows, int d) {
  if (rows < 0 || d < 1 || (d & (d - 1)) || (rows > 0 && !x)) return 1;
  for (int64_t r = 0; r < rows; ++r) oracle_fwht_f32(x + r * d, d);
  return 0;
}

/* Exponent e of a slab's power-of-two scale: the smallest integer with amax * 2^-e <=
 * 448, floored at -127 (e = 0 for amax = 0). */
int oracle_block_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e2;
  frexp((double)amax, &e2);
  const int E = e2 - 1;                               /* amax in [2^E, 2^(E+1)) */
  int e = ldexp((double)amax, 8 - E) <= 448.0 ? E - 8 : E - 7;
  if (e < -127) e = -127;
  return e;
}

/* Block quantisation of x (exact input values, float-representable) as described at the
 * top; `signs` (d floats, each +1 or -1) selects incoherent processing, NULL skips it.
 * Returns 0, 1 on bad arguments, 2 if scratch allocation failed. */
int oracle_block_quantize_e4m3(const double* x, int B, int N, int Hx, int d, int block_rows,
                               const float* signs, uint8_t* codes, uint8_t* scales) {
  if (B < 1 || N < 1 || Hx < 1 || d < 1 || block_rows < 1 || !x || !codes || !scales) return 1;
  if (signs && (d & (d - 1))) return 1;
  const int nb = (N + block_rows - 1) / block_rows;
  float* slab = (float*)malloc(sizeof(float) * (size_t)block_rows * d);
  if (!slab) return 2;
  for (int b = 0; b < B; ++b)
    for (int hx = 0; hx < Hx; ++hx)
      for (int blk = 0; blk < nb; ++blk) {
        const int r0 = blk * block_rows;
        const int nr = (N - r0) < block_rows ? (N - r0) : block_rows;
        float amax = 0.0f;
        for (int r = 0; r < nr; ++r) {
          const double* xr = x + (((size_t)b * N + r0 + r) * Hx + hx) * d;
          float* y = slab + (size_t)r * d;
          for (int t = 0; t < d; ++t) y[t] = signs ? (float)xr[t] * signs[t] : (float)xr[t];
          if (signs) oracle_fwht_f32(y, d);
          for (int t = 0; t < d; ++t)
            if (fabsf(y[t]) > amax) amax = fabsf(y[t]);
        }
        const int e = oracle_block_exponent(amax);
        scales[((size_t)b * Hx + hx) * nb + blk] = (uint8_t)(e + 127);
        for (int r = 0; r < nr; ++r) {
          uint8_t* c = codes + (((size_t)b * N + r0 + r) * Hx + hx) * d;
          const float* y = slab + (size_t)r * d;
          for (int t = 0; t < d; ++t) c[t] = oracle_e4m3_encode((float)ldexp((double)y[t], -e));
        }
      }
  free(slab);
  return 0;
}
