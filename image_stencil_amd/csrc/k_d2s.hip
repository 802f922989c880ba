// k_d2s.hip -- depth-to-space for the layer-by-layer chain.
//
// out[n,0,f*i+dy,f*j+dx] = z[n,f*dy+dx,i,j]: the last layer's f*f channels
// become one channel at f times the resolution (the output step of the
// upscaling network in "Optimizing convolution kernels - CNNs in Vulkan Part
// 2/3", introduction; its own net ends in 9 channels, f = 3). A pure
// permutation, bound by HBM: each thread takes one input pixel, reads its f*f
// channels (NCHW fp32: one coalesced load per channel plane; NHWC fp16: the
// pixel's channel vector, two 16-byte loads when it holds 16 channels) and
// writes its f x f output block, f values per output row. A workgroup covers
// 256 pixels of one input row; f is a template parameter, so the only runtime
// divisions are two 32-bit ones per thread.
#include "common.hpp"
#include "internal.hpp"

namespace is {
namespace {

constexpr int kThreads = 256;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

struct Pixel {
  int n, i, j;
  bool in;
};

__device__ inline Pixel this_pixel(int H, int W, int segs) {
  const int row = blockIdx.x / segs;
  const int seg = blockIdx.x - row * segs;
  Pixel p;
  p.n = row / H;
  p.i = row - p.n * H;
  p.j = seg * kThreads + threadIdx.x;
  p.in = p.j < W;
  return p;
}

template <int F>
__global__ __launch_bounds__(kThreads) void is_d2s_nchw_f32(const float *__restrict__ z, float *__restrict__ out,
                                                           int H, int W, int segs) {
  const Pixel p = this_pixel(H, W, segs);
  if (!p.in) return;
  const size_t plane = (size_t)H * W;
  const float *zp = z + (size_t)p.n * F * F * plane + (size_t)p.i * W + p.j;
  float v[F * F];
#pragma unroll
  for (int c = 0; c < F * F; ++c) v[c] = zp[c * plane];
  const size_t wo = (size_t)W * F;
#pragma unroll
  for (int dy = 0; dy < F; ++dy) {
    float *op = out + ((size_t)p.n * H * F + (size_t)p.i * F + dy) * wo + (size_t)F * p.j;
    if constexpr (F == 2) {
      *reinterpret_cast<float2 *>(op) = make_float2(v[2 * dy], v[2 * dy + 1]);
    } else {
#pragma unroll
      for (int dx = 0; dx < F; ++dx) op[dx] = v[F * dy + dx];
    }
  }
}

template <int F>
__global__ __launch_bounds__(kThreads) void is_d2s_nhwc_f16(const _Float16 *__restrict__ z,
                                                           _Float16 *__restrict__ out, int H, int W, int segs,
                                                           int zc) {
  const Pixel p = this_pixel(H, W, segs);
  if (!p.in) return;
  const _Float16 *zp = z + (((size_t)p.n * H + p.i) * W + p.j) * zc;
  _Float16 v[F * F];
  if (zc == 16) {
    // 32-byte aligned pixel vector (the workspace is 256-byte aligned).
    const uint4v *q = reinterpret_cast<const uint4v *>(zp);
    const half8 a = __builtin_bit_cast(half8, q[0]);
    const half8 b = __builtin_bit_cast(half8, q[1]);
#pragma unroll
    for (int c = 0; c < F * F; ++c) v[c] = c < 8 ? a[c] : b[c - 8];
  } else {
#pragma unroll
    for (int c = 0; c < F * F; ++c) v[c] = zp[c];
  }
  const size_t wo = (size_t)W * F;
#pragma unroll
  for (int dy = 0; dy < F; ++dy) {
    _Float16 *op = out + ((size_t)p.n * H * F + (size_t)p.i * F + dy) * wo + (size_t)F * p.j;
#pragma unroll
    for (int dx = 0; dx < F; ++dx) op[dx] = v[F * dy + dx];
  }
}

// Grid of one workgroup per 256 pixels of each input row; false when it does
// not fit a 1-D grid.
bool grid_for(int N, int H, int W, unsigned &blocks, int &segs) {
  segs = (W + kThreads - 1) / kThreads;
  const long long b = (long long)N * H * segs;
  if (b > 0x7FFFFFFFLL) return false;
  blocks = (unsigned)b;
  return true;
}

}  // namespace

hipError_t launch_depth_to_space(const float *z, float *out, int N, int H, int W, int f, hipStream_t s) {
  if ((long long)N * H * W == 0) return hipSuccess;
  unsigned blocks;
  int segs;
  if (!grid_for(N, H, W, blocks, segs)) return hipErrorInvalidValue;
  if (f == 2) return launch_kernel(is_d2s_nchw_f32<2>, dim3(blocks), dim3(kThreads), 0, s, z, out, H, W, segs);
  if (f == 3) return launch_kernel(is_d2s_nchw_f32<3>, dim3(blocks), dim3(kThreads), 0, s, z, out, H, W, segs);
  return hipErrorInvalidValue;
}

hipError_t launch_depth_to_space_f16(const _Float16 *z, _Float16 *out, int N, int H, int W, int f, int zc,
                                     hipStream_t s) {
  if ((long long)N * H * W == 0) return hipSuccess;
  if (zc < f * f) return hipErrorInvalidValue;
  unsigned blocks;
  int segs;
  if (!grid_for(N, H, W, blocks, segs)) return hipErrorInvalidValue;
  if (f == 2)
    return launch_kernel(is_d2s_nhwc_f16<2>, dim3(blocks), dim3(kThreads), 0, s, z, out, H, W, segs, zc);
  if (f == 3)
    return launch_kernel(is_d2s_nhwc_f16<3>, dim3(blocks), dim3(kThreads), 0, s, z, out, H, W, segs, zc);
  return hipErrorInvalidValue;
}

}  // namespace is
