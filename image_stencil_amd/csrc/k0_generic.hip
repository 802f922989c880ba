// k0_generic.hip -- direct convolution of any supported shape, one thread per output.
//
// The per-output-pixel loop nest of "Optimizing convolution kernels - CNNs in
// Vulkan Part 2/3" (StreamHPC), section "Where we left off", kept as the
// fallback for shapes no specialised kernel takes (filters wider than 7, channel
// counts off the register blocks, ...). fp32 accumulation, bias after the sum,
// optional ReLU; fp16 inputs are widened exactly and the fp32 result is rounded
// to nearest even on store.
#include "common.hpp"
#include "internal.hpp"

namespace is {
namespace {

__global__ __launch_bounds__(256) void is_k0_generic_nchw_f32(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ y, int N, int C, int H, int W, int K, int R, int S, int relu) {
  const long long total = (long long)N * K * H * W;
  const int P = (R - 1) / 2, Q = (S - 1) / 2;
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long long)gridDim.x * blockDim.x) {
    const int j = (int)(o % W);
    const int i = (int)((o / W) % H);
    const int k = (int)((o / ((long long)W * H)) % K);
    const long long n = o / ((long long)W * H * K);
    float acc = 0.f;
    for (int c = 0; c < C; ++c) {
      const float *xc = x + ((size_t)n * C + c) * (size_t)H * W;
      const float *wc = w + ((size_t)k * C + c) * R * S;
      for (int u = 0; u < R; ++u) {
        const int ii = i + u - P;
        if (ii < 0 || ii >= H) continue;
        for (int v = 0; v < S; ++v) {
          const int jj = j + v - Q;
          if (jj < 0 || jj >= W) continue;
          acc = __builtin_fmaf(wc[u * S + v], xc[(size_t)ii * W + jj], acc);
        }
      }
    }
    float out = acc + (bias ? bias[k] : 0.f);
    if (relu) out = fmaxf(out, 0.f);
    y[o] = out;
  }
}

__global__ __launch_bounds__(256) void is_k0_generic_nhwc_f16(
    const _Float16 *__restrict__ x, const _Float16 *__restrict__ w, const float *__restrict__ bias,
    _Float16 *__restrict__ y, int N, int C, int H, int W, int K, int R, int S, int relu) {
  const long long total = (long long)N * H * W * K;
  const int P = (R - 1) / 2, Q = (S - 1) / 2;
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long long)gridDim.x * blockDim.x) {
    const int k = (int)(o % K);
    const int j = (int)((o / K) % W);
    const int i = (int)((o / ((long long)K * W)) % H);
    const long long n = o / ((long long)K * W * H);
    float acc = 0.f;
    for (int u = 0; u < R; ++u) {
      const int ii = i + u - P;
      if (ii < 0 || ii >= H) continue;
      for (int v = 0; v < S; ++v) {
        const int jj = j + v - Q;
        if (jj < 0 || jj >= W) continue;
        const _Float16 *xp = x + (((size_t)n * H + ii) * W + jj) * C;
        for (int c = 0; c < C; ++c)
          acc = __builtin_fmaf((float)w[(((size_t)k * C + c) * R + u) * S + v], (float)xp[c], acc);
      }
    }
    float out = acc + (bias ? bias[k] : 0.f);
    if (relu) out = fmaxf(out, 0.f);
    y[o] = (_Float16)out;
  }
}

}  // namespace

bool configure_generic(Plan &p) {
  const conv2d_desc &d = p.d;
  const long long total = (long long)d.n * d.k * d.h * d.w;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  p.kid = d.layout == IS_NCHW ? kGenericNchwF32 : kGenericNhwcF16;
  p.name = d.layout == IS_NCHW ? "is_k0_generic_nchw_f32" : "is_k0_generic_nhwc_f16";
  p.grid_x = (int)blocks;
  p.grid_y = p.grid_z = 1;
  p.block = 256;
  p.lds = 0;
  p.tile_w = p.tile_h = 1;
  return true;
}

hipError_t launch_generic(const Plan &p, const void *x, const void *w, const float *b, void *y,
                          hipStream_t s) {
  const conv2d_desc &d = p.d;
  if (p.kid == kGenericNchwF32)
    return launch_kernel(is_k0_generic_nchw_f32, dim3(p.grid_x), dim3(p.block), 0, s,
                         static_cast<const float *>(x), static_cast<const float *>(w), b,
                         static_cast<float *>(y), d.n, d.c, d.h, d.w, d.k, d.r, d.s, d.relu);
  return launch_kernel(is_k0_generic_nhwc_f16, dim3(p.grid_x), dim3(p.block), 0, s,
                       static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(w), b,
                       static_cast<_Float16 *>(y), d.n, d.c, d.h, d.w, d.k, d.r, d.s, d.relu);
}

}  // namespace is
