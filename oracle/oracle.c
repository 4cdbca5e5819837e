/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.  A plain, slow, direct-loop CPU
 * reference of the DAC-style waveform decoder's operations.  Only the tests,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never does.  It shares no code with the HIP library.
 *
 * Built twice from this one file: REAL=double (the oracle proper, fp64
 * accumulation) and REAL=float (the "precision floor": the same loops in
 * float32, used only to show how far an honest fp32 evaluation lands from
 * the fp64 result).
 *
 * Layout of every activation: [rows][C][T] contiguous (time fastest), the
 * T-first layout the qwentts.cpp ARCHITECTURE page uses for its codec.
 * Each output is a plain sum in a fixed order (input channel, then tap),
 * so results do not depend on the number of OpenMP threads.
 *
 * Sources (page, section):
 *  - Snake: minimaxmusic.cpp ARCHITECTURE, "Flow VAE": y = x + sin^2(a x)/(a + 1e-9),
 *    alpha read verbatim.
 *  - SnakeBeta: qwentts.cpp ARCHITECTURE, "Audio tokenizer decoder" and the
 *    glossary: x + sin^2(alpha x)/beta (exp() of the stored logs folded at load;
 *    the synthetic configs give the values used in the formula directly).
 *  - Weight norm fold: minimaxmusic.cpp ARCHITECTURE, "Models": w = g v/||v||,
 *    axis 0 of the stored tensor.
 *  - Transposed conv as a scatter of kernel copies (what col2im overlap-adds):
 *    qwentts.cpp ARCHITECTURE, "Custom GGML ops" (col2im_1d, output length
 *    (T_in-1) s + K - 2 p0).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef REAL
#define REAL double
#endif

#ifdef ORACLE_FLOAT
#define SIN sinf
#define TANH tanhf
#define SQRT sqrtf
#else
#define SIN sin
#define TANH tanh
#define SQRT sqrt
#endif

#define EXPORT __attribute__((visibility("default")))

/* Size of REAL in bytes, so the loader can check it picked the right build. */
EXPORT int orc_real_size(void) { return (int)sizeof(REAL); }

/*
 * Snake / SnakeBeta, elementwise per channel:
 *   y[r][c][t] = x + sin(alpha_c x)^2 / (den_c + 1e-9),
 * with den = alpha (Snake) or beta (SnakeBeta, beta != NULL).
 */
EXPORT void orc_snake(const REAL *x, REAL *y, int64_t rows, int64_t C, int64_t T,
                      const REAL *alpha, const REAL *beta) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < C; ++c) {
      const REAL a = alpha[c];
      const REAL den = (beta ? beta[c] : alpha[c]) + (REAL)1e-9;
      const REAL *xr = x + (r * C + c) * T;
      REAL *yr = y + (r * C + c) * T;
      for (int64_t t = 0; t < T; ++t) {
        const REAL s = SIN(a * xr[t]);
        yr[t] = xr[t] + s * s / den;
      }
    }
}

/*
 * Weight-norm fold along axis 0: v is [d0][rest], g is [d0];
 *   w[i][:] = g[i] * v[i][:] / ||v[i][:]||_2.
 * Writes the norms to norms[d0] (may be NULL).
 */
EXPORT void orc_weight_norm(const REAL *v, const REAL *g, REAL *w, int64_t d0,
                            int64_t rest, REAL *norms) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < d0; ++i) {
    REAL ss = 0;
    for (int64_t j = 0; j < rest; ++j) ss += v[i * rest + j] * v[i * rest + j];
    const REAL n = SQRT(ss);
    if (norms) norms[i] = n;
    for (int64_t j = 0; j < rest; ++j) w[i * rest + j] = g[i] * v[i * rest + j] / n;
  }
}

/*
 * Conv1d with zero left padding P, output length T:
 *   y[r][o][t] = bias[o] + sum_i sum_j w[o][i][j] * x[r][i][t + j*dil - P],
 * x outside [0, T) is zero.  P = (K-1)/2 * dil is the "same" convolution,
 * P = (K-1) * dil the causal one.  w is [Cout][Cin][K]; bias may be NULL.
 */
EXPORT void orc_conv1d(const REAL *x, REAL *y, int64_t rows, int64_t Cin, int64_t T,
                       const REAL *w, const REAL *bias, int64_t Cout, int64_t K,
                       int64_t dil, int64_t P) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t o = 0; o < Cout; ++o) {
      REAL *yr = y + (r * Cout + o) * T;
      for (int64_t t = 0; t < T; ++t) yr[t] = 0;
      for (int64_t i = 0; i < Cin; ++i) {
        const REAL *xr = x + (r * Cin + i) * T;
        for (int64_t j = 0; j < K; ++j) {
          const REAL wv = w[(o * Cin + i) * K + j];
          const int64_t sh = j * dil - P; /* reads x[t + sh] */
          const int64_t t0 = sh < 0 ? -sh : 0;
          const int64_t t1 = sh > 0 ? T - sh : T;
          for (int64_t t = t0; t < t1; ++t) yr[t] += wv * xr[t + sh];
        }
      }
      if (bias)
        for (int64_t t = 0; t < T; ++t) yr[t] += bias[o];
    }
}

/*
 * Strided Conv1d (the encoder's downsampling conv): zero padding P on the
 * left, stride s, output length Tout:
 *   y[r][o][t] = bias[o] + sum_i sum_j w[o][i][j] * x[r][i][t*s + j - P],
 * x outside [0, T) is zero.  w is [Cout][Cin][K]; bias may be NULL.
 */
EXPORT void orc_conv1d_strided(const REAL *x, REAL *y, int64_t rows, int64_t Cin, int64_t T,
                               const REAL *w, const REAL *bias, int64_t Cout, int64_t K,
                               int64_t s, int64_t P, int64_t Tout) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t o = 0; o < Cout; ++o) {
      REAL *yr = y + (r * Cout + o) * Tout;
      for (int64_t t = 0; t < Tout; ++t) {
        REAL acc = 0;
        for (int64_t i = 0; i < Cin; ++i) {
          const REAL *xr = x + (r * Cin + i) * T;
          for (int64_t j = 0; j < K; ++j) {
            const int64_t src = t * s + j - P;
            if (src >= 0 && src < T) acc += w[(o * Cin + i) * K + j] * xr[src];
          }
        }
        yr[t] = acc + (bias ? bias[o] : (REAL)0);
      }
    }
}

/*
 * ConvTranspose1d with stride s, kernel K, left crop p, output length Tout:
 * every input sample x[i][m] adds w[i][o][:] * x[i][m] into the full output
 * starting at m*s; the kept output is full[n + p] for n in [0, Tout):
 *   y[r][o][n] = bias[o] + sum_i sum_m x[r][i][m] * w[i][o][n + p - m*s],
 * over 0 <= n + p - m*s < K.  w is [Cin][Cout][K].  The bias is added once
 * per output sample.
 */
EXPORT void orc_conv_transpose1d(const REAL *x, REAL *y, int64_t rows, int64_t Cin,
                                 int64_t T, const REAL *w, const REAL *bias,
                                 int64_t Cout, int64_t K, int64_t s, int64_t p,
                                 int64_t Tout) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t o = 0; o < Cout; ++o) {
      REAL *yr = y + (r * Cout + o) * Tout;
      for (int64_t n = 0; n < Tout; ++n) yr[n] = 0;
      for (int64_t i = 0; i < Cin; ++i) {
        const REAL *xr = x + (r * Cin + i) * T;
        const REAL *wr = w + (i * Cout + o) * K;
        for (int64_t m = 0; m < T; ++m)
          for (int64_t k = 0; k < K; ++k) {
            const int64_t n = m * s + k - p;
            if (n >= 0 && n < Tout) yr[n] += xr[m] * wr[k];
          }
      }
      if (bias)
        for (int64_t n = 0; n < Tout; ++n) yr[n] += bias[o];
    }
}

/* y = tanh(x) elementwise. */
EXPORT void orc_tanh(const REAL *x, REAL *y, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) y[k] = TANH(x[k]);
}

/* y = a + b elementwise (the residual add). */
EXPORT void orc_add(const REAL *a, const REAL *b, REAL *y, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) y[k] = a[k] + b[k];
}

/* Threads the parallel loops above use (OpenMP's maximum). */
#ifdef _OPENMP
#include <omp.h>
EXPORT int orc_num_threads(void) { return omp_get_max_threads(); }
#else
EXPORT int orc_num_threads(void) { return 1; }
#endif
