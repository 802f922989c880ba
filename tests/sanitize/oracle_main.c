/* Drives the oracle's C entry points on exact-size heap buffers, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer: any read or write past
 * a tensor, and any undefined arithmetic in the index computations, aborts.
 * Exits 0 when every call returned its documented status. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_conv2d(int layout, int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R, int64_t S,
                  const double *x, const double *w, const double *b, int relu, double *y, double *m);
int oracle_conv2d_points(int layout, int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R,
                         int64_t S, const double *x, const double *w, const double *b, int relu, int64_t npts,
                         const int64_t *pts, double *y, double *m);
int oracle_depth_to_space(int64_t N, int64_t H, int64_t W, int64_t f, const double *z, double *out);

static double *filled(int64_t n, unsigned seed) {
  double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  for (int64_t i = 0; i < n; ++i) {
    seed = seed * 1103515245u + 12345u;
    p[i] = (double)(seed >> 8) / 16777216.0 - 0.5;
  }
  return p;
}

static int conv_case(int layout, int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R, int64_t S,
                     int with_bias) {
  double *x = filled(N * C * H * W, 1), *w = filled(K * C * R * S, 2), *b = with_bias ? filled(K, 3) : NULL;
  double *y = filled(N * K * H * W, 4), *m = filled(N * K * H * W, 5);
  int rc = oracle_conv2d(layout, N, C, H, W, K, R, S, x, w, b, 1, y, m);
  /* a few sampled points, including the corners */
  int64_t pts[4 * 3] = {0, 0, 0, 0, N - 1, K - 1, H - 1, W - 1, N / 2, K / 2, H / 2, W / 2};
  double *yp = filled(3, 6), *mp = filled(3, 7);
  if (rc == 0) rc = oracle_conv2d_points(layout, N, C, H, W, K, R, S, x, w, b, 0, 3, pts, yp, mp);
  free(x); free(w); free(b); free(y); free(m); free(yp); free(mp);
  return rc;
}

int main(void) {
  int bad = 0;
  /* layout, N, C, H, W, K, R, S, bias */
  const int64_t cases[][9] = {{0, 1, 1, 1, 1, 1, 1, 1, 0},  {0, 2, 3, 9, 11, 4, 3, 3, 1}, {1, 2, 3, 9, 11, 4, 5, 5, 1},
                              {0, 1, 2, 7, 5, 3, 7, 1, 0},  {1, 1, 4, 3, 17, 2, 1, 7, 1}, {0, 1, 1, 2, 2, 1, 7, 7, 1},
                              {1, 3, 8, 6, 6, 16, 3, 3, 0}};
  for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i) {
    const int64_t *c = cases[i];
    if (conv_case((int)c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], (int)c[8]) != 0) {
      printf("conv case %zu failed\n", i);
      bad = 1;
    }
  }
  /* rejected shapes return an error without touching memory */
  double one = 1.0;
  if (oracle_conv2d(0, 1, 1, 4, 4, 1, 2, 3, &one, &one, NULL, 0, &one, NULL) == 0) {
    printf("even filter accepted\n");
    bad = 1;
  }
  int64_t outside[4] = {0, 0, 4, 0};
  if (oracle_conv2d_points(0, 1, 1, 4, 4, 1, 3, 3, &one, &one, NULL, 0, 1, outside, &one, NULL) == 0) {
    printf("point outside the image accepted\n");
    bad = 1;
  }
  for (int64_t f = 1; f <= 3; ++f) {
    const int64_t N = 2, H = 5, W = 7;
    double *z = filled(N * f * f * H * W, 8), *o = filled(N * f * H * f * W, 9);
    if (oracle_depth_to_space(N, H, W, f, z, o) != 0) bad = 1;
    free(z); free(o);
  }
  printf(bad ? "FAIL\n" : "OK\n");
  return bad;
}
