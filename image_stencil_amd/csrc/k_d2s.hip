// k_d2s.hip -- depth-to-space for the layer-by-layer chain.
//
// out[n,0,f*i+dy,f*j+dx] = z[n,f*dy+dx,i,j]: the last layer's f*f channels
// become one channel at f times the resolution (the output step of the
// upscaling network in "Optimizing convolution kernels - CNNs in Vulkan Part
// 2/3", introduction; its own net ends in 9 channels, f = 3). A pure
// permutation. For f = 2 in fp32 each thread reads one pixel of all 4 channels
// and writes a 2x2 output block as two 8-byte row pairs; otherwise each thread
// writes one output value.
#include "common.hpp"
#include "internal.hpp"

namespace is {

hipError_t launch_depth_to_space2(const float *z, float *out, int N, int H, int W, hipStream_t s);

namespace {

__global__ __launch_bounds__(256) void is_d2s2_f32(const float *__restrict__ z, float *__restrict__ out,
                                                  int N, int H, int W) {
  const long long total = (long long)N * H * W;
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long long)gridDim.x * blockDim.x) {
    const int j = (int)(o % W);
    const int i = (int)((o / W) % H);
    const long long n = o / ((long long)W * H);
    const size_t plane = (size_t)H * W;
    const float *zp = z + (size_t)n * 4 * plane + (size_t)i * W + j;
    const float a = zp[0], b = zp[plane], c = zp[2 * plane], d = zp[3 * plane];
    float *op = out + (size_t)n * 4 * plane + (size_t)(2 * i) * (2 * W) + 2 * j;
    *reinterpret_cast<float2 *>(op) = make_float2(a, b);
    *reinterpret_cast<float2 *>(op + 2 * W) = make_float2(c, d);
  }
}

__global__ __launch_bounds__(256) void is_d2s_f32(const float *__restrict__ z, float *__restrict__ out, int N,
                                                 int H, int W, int f) {
  const long long total = (long long)N * H * W * f * f;
  const int Wo = W * f;
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long long)gridDim.x * blockDim.x) {
    const int ox = (int)(o % Wo);
    const long long r = o / Wo;
    const int oy = (int)(r % ((long long)H * f));
    const long long n = r / ((long long)H * f);
    const int i = oy / f, dy = oy % f, j = ox / f, dx = ox % f;
    out[o] = z[((size_t)n * f * f + f * dy + dx) * H * W + (size_t)i * W + j];
  }
}

__global__ __launch_bounds__(256) void is_d2s_nhwc_f16(const _Float16 *__restrict__ z,
                                                      _Float16 *__restrict__ out, int N, int H, int W, int f,
                                                      int zc) {
  const long long total = (long long)N * H * W * f * f;
  const int Wo = W * f;
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long long)gridDim.x * blockDim.x) {
    const int ox = (int)(o % Wo);
    const long long r = o / Wo;
    const int oy = (int)(r % ((long long)H * f));
    const long long n = r / ((long long)H * f);
    const int i = oy / f, dy = oy % f, j = ox / f, dx = ox % f;
    out[o] = z[(((size_t)n * H + i) * W + j) * zc + f * dy + dx];
  }
}

unsigned grid_for(long long total) {
  long long blocks = (total + 255) / 256;
  return (unsigned)(blocks > 65536 ? 65536 : blocks);
}

}  // namespace

hipError_t launch_depth_to_space(const float *z, float *out, int N, int H, int W, int f, hipStream_t s) {
  if (f == 2) return launch_depth_to_space2(z, out, N, H, W, s);
  const long long total = (long long)N * H * W * f * f;
  if (total == 0) return hipSuccess;
  return launch_kernel(is_d2s_f32, dim3(grid_for(total)), dim3(256), 0, s, z, out, N, H, W, f);
}

hipError_t launch_depth_to_space_f16(const _Float16 *z, _Float16 *out, int N, int H, int W, int f, int zc,
                                     hipStream_t s) {
  const long long total = (long long)N * H * W * f * f;
  if (total == 0) return hipSuccess;
  return launch_kernel(is_d2s_nhwc_f16, dim3(grid_for(total)), dim3(256), 0, s, z, out, N, H, W, f, zc);
}

hipError_t launch_depth_to_space2(const float *z, float *out, int N, int H, int W, hipStream_t s) {
  const long long total = (long long)N * H * W;
  if (total == 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return launch_kernel(is_d2s2_f32, dim3((unsigned)blocks), dim3(256), 0, s, z, out, N, H, W);
}

}  // namespace is
