/* Runs the C oracle (oracle/ss2d_oracle.c, compiled into this program with
 * AddressSanitizer and UndefinedBehaviorSanitizer) on inputs read from a file and
 * writes y, so a test can check it against the unsanitized build.
 * File layout (native float64, then int64): B D H W N, then x, dt, A_log, dt_bias,
 * Bs, Cs, Ds in the oracle's shapes. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int ss2d_oracle_f64(const double* x, const double* dt, const double* A_log, const double* dt_bias,
                    const double* Bs, const double* Cs, const double* Ds, double* y, double* out_k,
                    int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int nthreads);

static double* read_n(FILE* f, size_t n) {
  double* p = (double*)malloc(n * sizeof(double));
  if (!p || fread(p, sizeof(double), n, f) != n) exit(3);
  return p;
}

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 2;
  int64_t s[5];
  if (fread(s, sizeof(int64_t), 5, f) != 5) return 3;
  const int64_t B = s[0], D = s[1], H = s[2], W = s[3], N = s[4], L = H * W;
  double* x = read_n(f, (size_t)(B * D * L));
  double* dt = read_n(f, (size_t)(B * 4 * D * L));
  double* A_log = read_n(f, (size_t)(4 * D * N));
  double* bias = read_n(f, (size_t)(4 * D));
  double* Bs = read_n(f, (size_t)(B * 4 * N * L));
  double* Cs = read_n(f, (size_t)(B * 4 * N * L));
  double* Ds = read_n(f, (size_t)(4 * D));
  fclose(f);
  double* y = (double*)malloc((size_t)(B * D * L) * sizeof(double));
  double* ok = (double*)malloc((size_t)(B * 4 * D * L) * sizeof(double));
  const int rc = ss2d_oracle_f64(x, dt, A_log, bias, Bs, Cs, Ds, y, ok, B, D, H, W, N, 1);
  if (rc != 0) return 4;
  FILE* g = fopen(argv[2], "wb");
  if (!g) return 2;
  fwrite(y, sizeof(double), (size_t)(B * D * L), g);
  fclose(g);
  free(x); free(dt); free(A_log); free(bias); free(Bs); free(Cs); free(Ds); free(y); free(ok);
  return 0;
}
