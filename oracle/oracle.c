/*
 * oracle.c -- plain CPU reference for direct 2D convolution with small filters.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header or constant with the HIP library.
 *
 * What it computes (all arithmetic in IEEE double, no blocking, no reordering
 * beyond the loop nest of the definition):
 *
 *   y[n,k,i,j] = act( sum_{c<C} sum_{u<R} sum_{v<S} w[k,c,u,v] * xz[n,c,i+u-R/2,j+v-S/2]  + b[k] )
 *
 * where xz is the input inside [0,H)x[0,W) and zero outside (same-size output,
 * stride 1, centred window, no filter flip).  This is the per-output-pixel loop
 * nest of "Optimizing convolution kernels - CNNs in Vulkan Part 2/3", section
 * "Where we left off" (output channel, input channel, kernel row, kernel column;
 * input pixel = output pixel + kernel offset - kernel size / 2; bias added after
 * the sum), with act = ReLU when requested (the apply_relu switch of the
 * "Vectorization" section of the same page) and identity otherwise.
 *
 * Alongside every y it returns the error scale
 *
 *   m[n,k,i,j] = sum_{c,u,v} |w[k,c,u,v] * xz[n,c,i+u-R/2,j+v-S/2]| + |b[k]|
 *
 * against which a reordered floating-point evaluation is judged.
 *
 * Precision: inputs arrive as doubles (callers widen fp32/fp16 values exactly),
 * every product and sum is a double. Build with -ffp-contract=off so that no
 * fused multiply-add changes the rounding of the plain expression.
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1

/* Index of element (n,c,i,j) of a tensor with C channels and HxW pixels. */
static inline size_t idx_nchw(int64_t n, int64_t c, int64_t i, int64_t j,
                              int64_t C, int64_t H, int64_t W) {
  return (size_t)(((n * C + c) * H + i) * W + j);
}
static inline size_t idx_nhwc(int64_t n, int64_t c, int64_t i, int64_t j,
                              int64_t C, int64_t H, int64_t W) {
  return (size_t)(((n * H + i) * W + j) * C + c);
}

/* One output element by the definition above. layout 0 = NCHW, 1 = NHWC for
 * both x and y; w is always KCRS. */
static void one_output(int layout, int64_t n, int64_t k, int64_t i, int64_t j,
                       int64_t C, int64_t H, int64_t W, int64_t R, int64_t S,
                       const double *x, const double *w, const double *b,
                       int relu, double *y_out, double *m_out) {
  const int64_t ph = (R - 1) / 2, pw = (S - 1) / 2;
  double sum = 0.0, mag = 0.0;
  for (int64_t c = 0; c < C; ++c) {
    for (int64_t u = 0; u < R; ++u) {
      for (int64_t v = 0; v < S; ++v) {
        const int64_t ii = i + u - ph;
        const int64_t jj = j + v - pw;
        if (ii < 0 || ii >= H || jj < 0 || jj >= W) continue; /* zero padding */
        const double xv = layout == 0 ? x[idx_nchw(n, c, ii, jj, C, H, W)]
                                      : x[idx_nhwc(n, c, ii, jj, C, H, W)];
        const double wv = w[(size_t)(((k * C + c) * R + u) * S + v)];
        const double p = wv * xv;
        sum += p;
        mag += fabs(p);
      }
    }
  }
  const double bias = b ? b[k] : 0.0;
  double out = sum + bias;
  if (relu && out < 0.0) out = 0.0;
  *y_out = out;
  if (m_out) *m_out = mag + fabs(bias);
}

static int shape_ok(int layout, int64_t N, int64_t C, int64_t H, int64_t W,
                    int64_t K, int64_t R, int64_t S) {
  if (layout != 0 && layout != 1) return 0;
  if (N < 0 || C < 1 || H < 0 || W < 0 || K < 1) return 0;
  if (R < 1 || S < 1 || (R % 2) == 0 || (S % 2) == 0) return 0;
  return 1;
}

/* Whole output tensor y (N,K,H,W in the given layout) and its error scale m
 * (same shape, may be NULL). Parallel over output rows only; each output is
 * still the sequential sum of the definition. */
int oracle_conv2d(int layout, int64_t N, int64_t C, int64_t H, int64_t W,
                  int64_t K, int64_t R, int64_t S, const double *x,
                  const double *w, const double *b, int relu, double *y,
                  double *m) {
  if (!shape_ok(layout, N, C, H, W, K, R, S) || !x || !w || !y)
    return ORACLE_EINVAL;
  const int64_t rows = N * K * H;
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < rows; ++row) {
    const int64_t i = row % H;
    const int64_t k = (row / H) % K;
    const int64_t n = row / (H * K);
    for (int64_t j = 0; j < W; ++j) {
      const size_t o = layout == 0 ? idx_nchw(n, k, i, j, K, H, W)
                                   : idx_nhwc(n, k, i, j, K, H, W);
      one_output(layout, n, k, i, j, C, H, W, R, S, x, w, b, relu, &y[o],
                 m ? &m[o] : NULL);
    }
  }
  return ORACLE_OK;
}

/* Selected outputs only: pts holds npts quadruples (n,k,i,j). Used to check a
 * full-size result at sampled positions. */
int oracle_conv2d_points(int layout, int64_t N, int64_t C, int64_t H,
                         int64_t W, int64_t K, int64_t R, int64_t S,
                         const double *x, const double *w, const double *b,
                         int relu, int64_t npts, const int64_t *pts, double *y,
                         double *m) {
  if (!shape_ok(layout, N, C, H, W, K, R, S) || !x || !w || !y || !pts ||
      npts < 0)
    return ORACLE_EINVAL;
  for (int64_t t = 0; t < npts; ++t) {
    const int64_t n = pts[4 * t], k = pts[4 * t + 1], i = pts[4 * t + 2],
                  j = pts[4 * t + 3];
    if (n < 0 || n >= N || k < 0 || k >= K || i < 0 || i >= H || j < 0 ||
        j >= W)
      return ORACLE_EINVAL;
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < npts; ++t) {
    one_output(layout, pts[4 * t], pts[4 * t + 1], pts[4 * t + 2],
               pts[4 * t + 3], C, H, W, R, S, x, w, b, relu, &y[t],
               m ? &m[t] : NULL);
  }
  return ORACLE_OK;
}

/* Depth-to-space by factor f: z has f*f channels of HxW, out has one channel
 * of (f*H)x(f*W) with out[n,0,f*i+dy,f*j+dx] = z[n,f*dy+dx,i,j] (channel index
 * row-offset major). A pure permutation of values. */
int oracle_depth_to_space(int64_t N, int64_t H, int64_t W, int64_t f,
                          const double *z, double *out) {
  if (N < 0 || H < 0 || W < 0 || f < 1 || !z || !out) return ORACLE_EINVAL;
  const int64_t C = f * f, Ho = H * f, Wo = W * f;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t dy = 0; dy < f; ++dy)
      for (int64_t dx = 0; dx < f; ++dx)
        for (int64_t i = 0; i < H; ++i)
          for (int64_t j = 0; j < W; ++j)
            out[(size_t)((n * Ho + (f * i + dy)) * Wo + (f * j + dx))] =
                z[idx_nchw(n, f * dy + dx, i, j, C, H, W)];
  return ORACLE_OK;
}

/* Threads the parallel loops above use (1 without OpenMP). */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
