// k8_pointwise.hip -- 1x1 filters over several channels, fp32 NCHW:
// y[n][k][p] = act(sum_c w[k][c] * x[n][c][p] + b[k]).
//
// With R = S = 1 the loop nest of "Optimizing convolution kernels - CNNs in
// Vulkan Part 2/3" ("Where we left off") has no window: each output pixel is
// a dot product over the channels, and the layer is bound by HBM for the
// channel counts of these networks (2CK FLOPs against 4(C + K) bytes per
// pixel). So there is no tile and no halo to stage ("Optimizing Memory
// Efficiency for Convolution Kernels on Kepler GPUs", arXiv 1705.10591, notes
// that 1x1 filters share no data between pixels):
//  * a thread owns 4 consecutive pixels of one image (one 16-byte vector per
//    channel plane; a wave reads 1 KB of a plane per load) and KB output
//    channels, a workgroup 1024 pixels;
//  * the input planes stream through registers, 4 channels per unrolled step,
//    every input vector read once per group of KB output channels;
//  * the workgroup's KB x C weights are staged once in LDS transposed (channel
//    major), so that the KB weights of channel c are KB/4 16-byte LDS reads
//    that every lane makes at the same address (broadcast, no bank conflict);
//  * bias, ReLU and 16-byte stores of each output plane.
#include "common.hpp"
#include "internal.hpp"

namespace is {
namespace {

constexpr int kThreads = 256;
constexpr int kPix = 4 * kThreads;     // pixels per workgroup
constexpr int kMaxLds = 48 * 1024;     // dynamic LDS of the staged weights, C * KB * 4 bytes
typedef float f4v __attribute__((ext_vector_type(4)));   // for the non-temporal builtins

template <int KB, bool RELU>
__global__ __launch_bounds__(kThreads) void is_k8_pointwise(const float *__restrict__ x, const float *__restrict__ w,
                                                           const float *__restrict__ bias, float *__restrict__ y,
                                                           int C, int HW, int K) {
  extern __shared__ float4 wt4[];      // [C][KB / 4]: channel c's KB weights
  float *wt = reinterpret_cast<float *>(wt4);
  lds_poison(wt4, C * KB * 4);
  const int tid = threadIdx.x;
  const int kg = blockIdx.y;
  const int n = blockIdx.z;
  for (int i = tid; i < C * KB; i += kThreads) {
    const int c = i / KB, f = i - c * KB;
    wt[i] = w[(size_t)(kg * KB + f) * C + c];
  }
  __syncthreads();

  const int p4 = blockIdx.x * kThreads + tid;   // 16-byte vector of the plane
  if (4 * p4 >= HW) return;
  const size_t plane4 = (size_t)HW / 4;
  const f4v *xp = reinterpret_cast<const f4v *>(x + (size_t)n * C * HW) + p4;

  float acc[KB][4];
#pragma unroll
  for (int f = 0; f < KB; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[f][i] = 0.f;

  auto step = [&](const f4v v, int c) __attribute__((always_inline)) {
    const float xv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < KB / 4; ++q) {
      const float4 wv = wt4[c * (KB / 4) + q];
      const float wq[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * q + e][i] = __builtin_fmaf(wq[e], xv[i], acc[4 * q + e][i]);
    }
  };
  int c = 0;
  for (; c + 4 <= C; c += 4) {
    f4v v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(xp + (size_t)(c + u) * plane4);
#pragma unroll
    for (int u = 0; u < 4; ++u) step(v[u], c + u);
  }
  for (; c < C; ++c) step(__builtin_nontemporal_load(xp + (size_t)c * plane4), c);

  float *yp = y + ((size_t)n * K + (size_t)kg * KB) * HW + 4 * (size_t)p4;
#pragma unroll
  for (int f = 0; f < KB; ++f) {
    const float b = bias ? bias[kg * KB + f] : 0.f;
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = acc[f][i] + b;
      if constexpr (RELU) o[i] = fmaxf(o[i], 0.f);
    }
    __builtin_nontemporal_store(f4v{o[0], o[1], o[2], o[3]}, reinterpret_cast<f4v *>(yp + (size_t)f * HW));
  }
}

using K8Fn = void (*)(const float *, const float *, const float *, float *, int, int, int);

template <bool RELU>
K8Fn pick(int kb) {
  switch (kb) {
    case 32: return is_k8_pointwise<32, RELU>;
    case 16: return is_k8_pointwise<16, RELU>;
    case 8: return is_k8_pointwise<8, RELU>;
    case 4: return is_k8_pointwise<4, RELU>;
    default: return nullptr;
  }
}

}  // namespace

bool configure_pointwise(Plan &p, int param) {
  const conv2d_desc &d = p.d;
  if (d.layout != IS_NCHW || d.in_dtype != IS_F32 || d.r != 1 || d.s != 1 || d.separable) return false;
  if (d.c < 2) return false;   // one channel: the single-channel kernels
  const long long hw = (long long)d.h * d.w;
  if (hw % 4 != 0 || hw == 0 || hw > 0x7FFFFFFF) return false;   // whole 16-byte vectors per plane
  if (d.n > 65535) return false;
  int kb = 0;
  for (int f : {32, 16, 8, 4})
    if (d.k % f == 0 && (long long)d.c * f * 4 <= kMaxLds) {
      kb = f;
      break;
    }
  if (param != 0) {   // a tuning variant: that many output channels per workgroup
    if (d.k % param != 0 || pick<false>(param) == nullptr || (long long)d.c * param * 4 > kMaxLds) return false;
    kb = param;
  }
  if (kb == 0) return false;
  const long long gx = (hw + kPix - 1) / kPix;
  if (gx > 0x7FFFFFFF || d.k / kb > 65535) return false;
  p.kid = kPointwise;
  p.name = "is_k8_pointwise";
  p.strip_rows = kb;   // output channels per workgroup
  p.grid_x = (int)gx;
  p.grid_y = d.k / kb;
  p.grid_z = d.n;
  p.block = kThreads;
  p.lds = d.c * kb * 4;
  p.tile_w = kPix;
  p.tile_h = 1;
  return true;
}

hipError_t launch_pointwise(const Plan &p, const float *x, const float *w, const float *b, float *y,
                            hipStream_t s) {
  const K8Fn fn = p.d.relu ? pick<true>(p.strip_rows) : pick<false>(p.strip_rows);
  if (!fn) return hipErrorInvalidValue;
  if ((long long)p.d.h * p.d.w == 0 || p.d.n == 0) return hipSuccess;
  return launch_kernel(fn, dim3(p.grid_x, p.grid_y, p.grid_z), dim3(p.block), (unsigned)p.lds, s, x, w, b, y,
                       p.d.c, p.d.h * p.d.w, p.d.k);
}

}  // namespace is
