/*
 * SS2D forward oracle: plain, sequential, double precision.  TEST INFRASTRUCTURE
 * ONLY -- it checks the HIP path and is never part of it.  It shares no code,
 * header, table or helper with the GPU library.
 *
 * Pages followed (cited by title and section):
 *   [SS2D]   "深入解析VMamba中的SS2D模块从理论到代码实现" (omica.com.cn)
 *            §3.1 the four scan sequences, §3.2 the selective_scan call
 *            (A = -exp(A_log), delta_bias, delta_softplus), §3.3 the merge,
 *            §4 the direction table.
 *   [DAMamba] DAMamba walkthrough (lpnh.cn) §2.1 discrete SSM h_t = A h_{t-1} + B x_t,
 *            y_t = C h_t + D x_t; §3.1 the scan loop starts from a zero state.
 *   The recurrence per state n is h = exp(delta*A) * h + delta * B * u and the
 *   output is y = sum_n C_n * h_n + D * u (zero-order hold for A, Euler for B).
 *
 * Definition computed, for every batch b, direction k, channel d (c = k*D + d):
 *   direction 0 visits the H x W map row by row, left to right;
 *   direction 1 column by column, top to bottom;
 *   directions 2 and 3 visit the same pixels as 0 and 1 in reverse order.
 *   u[l]     = x[b, d, pixel visited at step l]
 *   delta[l] = softplus(dt[b, k, d, l] + dt_bias[c])      (dt is in scan order)
 *   out[l]   = Ds[c] * u[l] + sum_n Cs[b,k,n,l] * h_n[l]
 *   h_n[-1]  = 0,  h_n[l] = exp(delta[l] * -exp(A_log[c,n])) * h_n[l-1]
 *                           + delta[l] * Bs[b,k,n,l] * u[l]
 *   y[b, d, pixel visited at step l of direction k] += out[l]   (sum over k)
 * Bs and Cs are shared by all D channels of a direction.
 *
 * Parallelism: only across independent (b, d) map planes (OpenMP); inside a
 * plane the four directions are done in order k = 0..3 and each recurrence runs
 * sequentially over l, so the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(v) = log(1 + e^v), evaluated without overflow for large v. */
static double softplus_f64(double v) {
  if (v > 0.0) return v + log1p(exp(-v));
  return log1p(exp(v));
}

/* Pixel (flat index h*W + w) that direction k visits at scan step l.
 * Built from the walking order itself: rows-then-columns for k = 0,
 * columns-then-rows for k = 1, and the reversed walks for k = 2, 3. */
static int64_t visited_pixel(int k, int64_t l, int64_t H, int64_t W) {
  const int64_t L = H * W;
  const int64_t step = (k >= 2) ? (L - 1 - l) : l;
  if ((k & 1) == 0) {
    return step;                      /* row walk: step = h*W + w */
  }
  const int64_t col = step / H;       /* column walk: step = w*H + h */
  const int64_t row = step % H;
  return row * W + col;
}

int ss2d_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * All arrays are host memory, double precision, dense row-major:
 *   x (B,D,H,W), dt (B,4,D,L), A_log (4D,N), dt_bias (4D), Bs/Cs (B,4,N,L),
 *   Ds (4D), y (B,D,H,W) output (overwritten), out_k (B,4,D,L) optional
 *   per-direction outputs in scan order (NULL to skip).
 * Returns 0, or -1 for a bad argument, -2 for an allocation failure.
 */
int ss2d_oracle_f64(const double* x, const double* dt, const double* A_log,
                    const double* dt_bias, const double* Bs, const double* Cs,
                    const double* Ds, double* y, double* out_k,
                    int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                    int nthreads) {
  if (!x || !dt || !A_log || !dt_bias || !Bs || !Cs || !Ds || !y) return -1;
  if (B < 1 || D < 1 || H < 1 || W < 1 || N < 1) return -1;
  const int64_t L = H * W;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  const int nt = omp_get_max_threads();
#else
  (void)nthreads;
  const int nt = 1;
#endif
  /* per-thread scratch rows: u, delta, out */
  double* scratch = (double*)malloc(sizeof(double) * (size_t)L * 3u * (size_t)nt);
  if (!scratch) return -2;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bd = 0; bd < B * D; ++bd) {
#ifdef _OPENMP
    const int t = omp_get_thread_num();
#else
    const int t = 0;
#endif
    double* u = scratch + (size_t)L * 3u * (size_t)t;
    double* delta = u + L;
    double* out = delta + L;
    const int64_t b = bd / D, d = bd % D;
    const double* xp = x + (b * D + d) * L;
    double* yp = y + (b * D + d) * L;
    for (int64_t p = 0; p < L; ++p) yp[p] = 0.0;
    for (int k = 0; k < 4; ++k) {
      const int64_t c = (int64_t)k * D + d;
      const double* dtp = dt + ((b * 4 + k) * D + d) * L;
      for (int64_t l = 0; l < L; ++l) {
        u[l] = xp[visited_pixel(k, l, H, W)];
        delta[l] = softplus_f64(dtp[l] + dt_bias[c]);
        out[l] = Ds[c] * u[l];
      }
      for (int64_t n = 0; n < N; ++n) {
        const double A = -exp(A_log[c * N + n]);
        const double* Bp = Bs + ((b * 4 + k) * N + n) * L;
        const double* Cp = Cs + ((b * 4 + k) * N + n) * L;
        double h = 0.0;
        for (int64_t l = 0; l < L; ++l) {
          h = exp(delta[l] * A) * h + delta[l] * Bp[l] * u[l];
          out[l] += Cp[l] * h;
        }
      }
      if (out_k) memcpy(out_k + ((b * 4 + k) * D + d) * L, out, sizeof(double) * (size_t)L);
      for (int64_t l = 0; l < L; ++l) yp[visited_pixel(k, l, H, W)] += out[l];
    }
  }
  free(scratch);
  return 0;
}
