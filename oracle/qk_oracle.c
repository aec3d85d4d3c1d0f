/*
 * ORACLE -- TEST INFRASTRUCTURE ONLY.
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * or call this code. The product path never does, and this file shares no code,
 * header, table or helper with the HIP library.
 *
 * What it computes: the skinny quantized product y[M,N] = x[M,K] . w[N,K]^T in
 * which w is stored as 4.5-bit k-quant super-blocks, written out as its plain
 * definition: dequantize each weight, multiply, sum in ascending k, in binary64.
 *   - "sixi-asi 0.9", section "What I got wrong in 0.8": the verify pass is a
 *     batched pass over k+1 rows whose time goes to quantized matrix products,
 *     whose kernels decode the 4-bit weights.
 *   - "sixi-asi 0.9", section "Numbers": the weights are plain Q4_K_M GGUF
 *     files, i.e. the Q4_K k-quant super-block: 256 weights along K with a
 *     binary16 scale d and min dmin, eight 32-weight sub-blocks with a 6-bit
 *     scale sc and 6-bit min m each, and 4-bit quants q; the weight is
 *     w = d*sc*q - dmin*m.
 *   - "sixi-asi 0.9", section "The patch": the GPU kernels are checked
 *     against a CPU reference of the same product.
 *
 * Byte layout of one 144-byte super-block (a reading; the pages name the
 * format but do not print its bytes; this is the public Q4_K layout):
 *   [0..1] d, [2..3] dmin (little-endian binary16);
 *   [4..15] eight 6-bit scales and eight 6-bit mins, see oracle_scale_min();
 *   [16..143] 128 bytes of quants, see oracle_dequant_block().
 * A matrix is N rows of K/256 consecutive blocks, rows consecutive.
 *
 * Pins (all in tests/, marked "not gpu"): exhaustive binary16 decode against
 * numpy; hand-built literal blocks under tests/golden/ with hand-derived
 * weights; an exact rational (fractions.Fraction) evaluator with its own
 * decoder on tiny shapes; one-hot, all-ones and zero-scale closed forms; row,
 * permutation and linearity invariants. GGUF file compatibility of the byte
 * layout is parity unpinned: no GGUF file is available to compare against.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16 -> binary64, written from the format's definition: sign,
 * 5-bit biased exponent (bias 15), 10-bit fraction; exponent 0 is zero or a
 * subnormal (fraction * 2^-24), exponent 31 is inf or NaN. Exact. */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1F;
  int fr = h & 0x3FF;
  double v;
  if (ex == 0)
    v = ldexp((double)fr, -24);
  else if (ex == 31)
    v = fr ? NAN : INFINITY;
  else
    v = ldexp((double)(fr | 0x400), ex - 25);
  return sign ? -v : v;
}

/* Scale sc_j and min m_j (j = 0..7) of the 12 packed bytes s[0..11] of a
 * super-block (Q4_K packing, a reading): for j < 4 the low six bits of s[j]
 * and of s[j+4]; for j >= 4 the low nibble (scale) or high nibble (min) of
 * s[j+4] gives bits 0..3, and the top two bits of s[j-4] (scale) or of s[j]
 * (min) give bits 4..5. */
void oracle_scale_min(const uint8_t* s, int j, int* sc, int* m) {
  if (j < 4) {
    *sc = s[j] & 63;
    *m = s[j + 4] & 63;
  } else {
    *sc = (s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4);
    *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
  }
}

/* The 256 weights of one super-block, in binary64:
 * w[i] = d * sc_j * q_i - dmin * m_j with j = i / 32. Quant order (a reading,
 * the Q4_K order): weight i = 64c + r (c = 0..3, r = 0..63) sits in byte
 * 16 + 32c + (r mod 32), in its low nibble when r < 32, in its high nibble
 * otherwise. d*sc*q (at most 21 significant bits) and dmin*m (at most 17) are
 * exact in binary64; their difference is rounded once. */
void oracle_dequant_block(const uint8_t* blk, double* w) {
  double d = oracle_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
  double dmin = oracle_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
  for (int i = 0; i < 256; ++i) {
    int c = i / 64, r = i % 64, j = i / 32;
    uint8_t byte = blk[16 + 32 * c + (r % 32)];
    int q = (r < 32) ? (byte & 0x0F) : (byte >> 4);
    int sc, m;
    oracle_scale_min(blk + 4, j, &sc, &m);
    w[i] = d * (double)sc * (double)q - dmin * (double)m;
  }
}

/* Dequantized rows: wout[r][k] = w[rows[r]][k] for r = 0..nrows-1. */
int oracle_dequant_rows(const uint8_t* W, int64_t N, int64_t K, const int64_t* rows,
                        int64_t nrows, double* wout) {
  if (!W || !rows || !wout || K <= 0 || K % 256 || N < 0) return -1;
  const int64_t nb = K / 256;
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t n = rows[r];
    if (n < 0 || n >= N) return -1;
    for (int64_t b = 0; b < nb; ++b)
      oracle_dequant_block(W + (n * nb + b) * 144, wout + r * K + b * 256);
  }
  return 0;
}

/* y[m][r] = sum_k x[m][k] * w[rows[r]][k] and a[m][r] = sum_k |x[m][k] * w[rows[r]][k]|,
 * each summed in ascending k in binary64 (x is widened exactly from fp32).
 * Rows are independent; threads split the rows only, so the result does not
 * depend on the thread count. nthreads <= 0 uses the OpenMP default. */
int oracle_qmm_rows(const float* x, const uint8_t* W, int64_t M, int64_t N, int64_t K,
                    const int64_t* rows, int64_t nrows, double* y, double* a,
                    int nthreads) {
  if (!x || !W || !rows || !y || M < 1 || N < 0 || K <= 0 || K % 256) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return -1;
  const int64_t nb = K / 256;
  int bad = 0;
#ifdef _OPENMP
  /* a count for this call only (the process default stays as it was) */
  const int team = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
  (void)nthreads;
#endif
#pragma omp parallel num_threads(team)
  {
    double w[256];
    double* acc = (double*)malloc(sizeof(double) * 2 * (size_t)M);
    if (!acc) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t n = rows[r];
        for (int64_t mm = 0; mm < 2 * M; ++mm) acc[mm] = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
          oracle_dequant_block(W + (n * nb + b) * 144, w);
          for (int64_t mm = 0; mm < M; ++mm) {
            const float* xr = x + mm * K + b * 256;
            double s = acc[mm], t = acc[M + mm];
            for (int i = 0; i < 256; ++i) {
              double p = w[i] * (double)xr[i];
              s += p;
              t += fabs(p);
            }
            acc[mm] = s;
            acc[M + mm] = t;
          }
        }
        for (int64_t mm = 0; mm < M; ++mm) {
          y[mm * nrows + r] = acc[mm];
          if (a) a[mm * nrows + r] = acc[M + mm];
        }
      }
      free(acc);
    }
  }
  return bad ? -2 : 0;
}

/* The whole product: y[M][N], a[M][N]. */
int oracle_qmm(const float* x, const uint8_t* W, int64_t M, int64_t N, int64_t K,
               double* y, double* a, int nthreads) {
  if (N < 0) return -1;
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
  if (!rows) return -2;
  for (int64_t n = 0; n < N; ++n) rows[n] = n;
  int rc = oracle_qmm_rows(x, W, M, N, K, rows, N, y, a, nthreads);
  free(rows);
  return rc;
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
