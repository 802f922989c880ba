// k_d2s.hip -- depth-to-space by 2 for the layer-by-layer chain.
//
// out[n,0,2i+dy,2j+dx] = z[n,2*dy+dx,i,j]: the last layer's 4 channels become one
// channel at twice the resolution (the output step of the upscaling network in
// "Optimizing convolution kernels - CNNs in Vulkan Part 2/3", introduction). A
// pure permutation. Each thread reads one pixel of all 4 channels and writes a
// 2x2 output block as two 8-byte row pairs.
#include "common.hpp"
#include "internal.hpp"

namespace is {
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

}  // namespace

hipError_t launch_depth_to_space2(const float *z, float *out, int N, int H, int W, hipStream_t s) {
  const long long total = (long long)N * H * W;
  if (total == 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return launch_kernel(is_d2s2_f32, dim3((unsigned)blocks), dim3(256), 0, s, z, out, N, H, W);
}

}  // namespace is
