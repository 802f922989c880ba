// k6_head_f16.hip -- fp16 NHWC layer with one input channel (a network's first
// layer: 1 -> K, K in {16, 32, 64}, 3x3 or 5x5), fp32 accumulation, fp16 output.
//
// With a single input channel the contraction of "Optimizing convolution
// kernels - CNNs in Vulkan Part 2/3" ("Where we left off": the sum over
// channels and filter taps) runs over the R*S <= 32 taps only, one k step of
// v_mfma_f32_16x16x32_f16 (the first layer of the pages' upscaling network,
// "Reducing memory traffic" table: 1 -> 64, 5x5):
//  * a workgroup of 4 waves owns a tile of 16 rows x 64 columns; the input
//    tile with its halo ((16 + R - 1) x (64 + S - 1) fp16 values) is loaded
//    into LDS once, pixels outside the image as 0;
//  * wave w owns the 16 columns 16w .. +16 of every tile row; per row, lane
//    (n16, g) gathers taps 8g .. 8g+7 of pixel n16 from LDS into one B
//    fragment (taps past R*S are 0), and one MFMA per 16 output channels
//    (A = 16 channels x 32 taps, zero-padded weights) gives 4 consecutive
//    channels of the pixel per lane;
//  * bias (fp32), optional ReLU, fp16 rounding (nearest even) and an 8-byte
//    store per lane and 16-channel block: the blocks' stores of one row fill
//    whole pixel lines back to back.
#include "common.hpp"
#include "internal.hpp"

namespace is {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));

constexpr int kTH = 16;                 // tile rows
constexpr int kTW = 64;                 // tile columns (4 waves x 16)
constexpr int kThreads = 256;
constexpr unsigned kOob = 0xFFFFFFF0u;

struct HeadArgs {
  const _Float16 *x;
  const _Float16 *w;
  const float *bias;
  _Float16 *y;
  int N, H, W, relu;
  int tiles_x, tiles_y;
};

template <int R, int K>
__global__ __launch_bounds__(kThreads) void is_k6_head_f16(HeadArgs a) {
  constexpr int P = (R - 1) / 2;
  constexpr int LW = kTW + R - 1;       // LDS tile width
  constexpr int LH = kTH + R - 1;       // LDS tile height
  constexpr int NOB = K / 16;
  static_assert(R * R <= 32, "the taps fit one k step");
  __shared__ _Float16 tile[LH * LW];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g = lane >> 4;

  const int t = blockIdx.x;
  const int tx = t % a.tiles_x;
  const int ty = (t / a.tiles_x) % a.tiles_y;
  const int n = t / (a.tiles_x * a.tiles_y);
  const int x0 = tx * kTW, y0 = ty * kTH;
  const size_t plane = (size_t)a.H * a.W;
  const _Float16 *xn = a.x + (size_t)n * plane;

  // ---- Input tile with halo, zero outside the image.
  for (int e = tid; e < LH * LW; e += kThreads) {
    const int gy = y0 - P + e / LW, gx = x0 - P + e % LW;
    const bool in = (unsigned)gy < (unsigned)a.H && (unsigned)gx < (unsigned)a.W;
    tile[e] = in ? xn[(size_t)gy * a.W + gx] : (_Float16)0.f;
  }

  // ---- Weights: A fragment of block ob holds, for output channel
  // 16*ob + n16, taps 8g .. 8g+7 (row-major over the R x R filter); taps past
  // R*R are 0. Bias: channels 16*ob + 4g .. +4 (the D rows of this lane).
  half8 wa[NOB];
  float bias[NOB][4];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = 8 * g + j;
      wa[ob][j] = k < R * R ? a.w[(16 * ob + n16) * R * R + k] : (_Float16)0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) bias[ob][e] = a.bias ? a.bias[16 * ob + 4 * g + e] : 0.f;
  }
  // LDS offsets of this lane's 8 taps for tile row 0 (taps past R*R read the
  // tile origin and are replaced by 0 below).
  int toff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = 8 * g + j;
    toff[j] = k < R * R ? (k / R) * LW + 16 * wave + n16 + k % R : 0;
  }
  __syncthreads();

  const int gx = x0 + 16 * wave + n16;
  const bool col_in = gx < a.W;
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
      a.y + (size_t)n * plane * K, (short)0, (int)(plane * K * 2), kBufferFlags);
#pragma unroll 2
  for (int r = 0; r < kTH; ++r) {
    half8 b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const _Float16 v = tile[toff[j] + r * LW];
      b[j] = (8 * g + j < R * R) ? v : (_Float16)0.f;
    }
    const int gy = y0 + r;
    const bool in = col_in & (gy < a.H);
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      const float4v acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[ob], b, float4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      _Float16 hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = acc[e] + bias[ob][e];
        if (a.relu) v = fmaxf(v, 0.f);
        hv[e] = (_Float16)v;
      }
      const unsigned off = in ? (unsigned)((((size_t)gy * a.W + gx) * K + 16 * ob + 4 * g) * 2) : kOob;
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2v, hv), ry, off, 0, 0);
    }
  }
}

template <int R>
auto pick_k(int k) -> void (*)(HeadArgs) {
  if (k == 16) return is_k6_head_f16<R, 16>;
  if (k == 32) return is_k6_head_f16<R, 32>;
  if (k == 64) return is_k6_head_f16<R, 64>;
  return nullptr;
}

auto pick(int r, int k) -> void (*)(HeadArgs) {
  if (r == 3) return pick_k<3>(k);
  if (r == 5) return pick_k<5>(k);
  return nullptr;
}

}  // namespace

bool configure_head_f16(Plan &p) {
  const conv2d_desc &d = p.d;
  if (d.layout != IS_NHWC || d.in_dtype != IS_F16 || d.out_dtype != IS_F16) return false;
  if (d.c != 1 || d.r != d.s || pick(d.r, d.k) == nullptr) return false;
  if (2.0 * d.h * (double)d.w * d.k >= 4.0e9) return false;   // 32-bit output offsets per image
  const long long tiles = (long long)((d.w + kTW - 1) / kTW) * ((d.h + kTH - 1) / kTH) * d.n;
  if (tiles > (1LL << 31) - 1) return false;
  p.kid = kHeadNhwcF16;
  p.name = "is_k6_head_f16";
  p.nseg = (d.w + kTW - 1) / kTW;
  p.nstrip = (d.h + kTH - 1) / kTH;
  p.ntiles = (int)tiles;
  p.grid_x = p.ntiles;
  p.grid_y = p.grid_z = 1;
  p.block = kThreads;
  p.lds = (kTH + d.r - 1) * (kTW + d.r - 1) * 2;
  p.tile_w = kTW;
  p.tile_h = kTH;
  return true;
}

hipError_t launch_head_f16(const Plan &p, const _Float16 *x, const _Float16 *w, const float *b, _Float16 *y,
                           hipStream_t s) {
  auto fn = pick(p.d.r, p.d.k);
  if (!fn) return hipErrorInvalidValue;
  HeadArgs a;
  a.x = x;
  a.w = w;
  a.bias = b;
  a.y = y;
  a.N = p.d.n;
  a.H = p.d.h;
  a.W = p.d.w;
  a.relu = p.d.relu;
  a.tiles_x = p.nseg;
  a.tiles_y = p.nstrip;
  return launch_kernel(fn, dim3(p.grid_x), dim3(p.block), 0, s, a);
}

}  // namespace is
