// k9_head_f32.hip -- fp32 NCHW layer with one input channel (a network's first
// layer: 1 -> K, K in {16, 32, 64}, 3x3 or 5x5), on the fp32 matrix cores.
//
// With one input channel the contraction of "Optimizing convolution kernels -
// CNNs in Vulkan Part 2/3" ("Where we left off": the sum over channels and
// filter taps) runs over the R*S taps only: 25 for the first layer of the
// pages' upscaling network ("Reducing memory traffic" table, 5x5). On the
// vector ALUs each output value costs R*S FMAs with a wave-uniform tap; here
// v_mfma_f32_16x16x4_f32 takes 4 taps x 16 pixels x 16 output channels per
// instruction (7 k steps of 4 taps for 5x5, the last 3 taps zero; 3 for 3x3).
// The layer reads 4 bytes and writes 4K per pixel, so it is bound by its write
// stream (118 MB per 1280x720 frame at K = 32). Design:
//  * persistent workgroups of 4 waves, kWgPerCu per CU, walking tiles of kTH
//    rows x 64 columns; the next tile's input (with its R-1 halo rows and
//    columns) is loaded into registers with branch-free buffer loads while the
//    current tile is computed and stored, then written to the other of two
//    LDS buffers;
//  * wave w owns columns 16w .. +16 of every tile row. Operands: A = 16 pixels
//    x 4 taps (lane (n16, g) reads the input value under tap 4ks + g of pixel
//    n16 from LDS, 0 past the last tap), B = 4 taps x 16 output channels (the
//    weights, in registers for the whole kernel), D = 4 consecutive pixels of
//    one output channel per lane: bias, optional ReLU, one 16-byte NCHW store;
//  * the tile's LDS rows are 84 floats apart: the 4 lane groups of a gather
//    read 16 consecutive floats each under 4 different taps, and at this pitch
//    those 4 runs fall on disjoint quarters of the 64 banks for every k step
//    and wave (rows of 66 or 68 floats put two of them on the same banks).
#include "common.hpp"
#include "internal.hpp"

namespace is {
namespace {

typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

constexpr int kTH = 16;                 // tile rows
constexpr int kTW = 64;                 // tile columns (4 waves x 16)
constexpr int kThreads = 256;
constexpr int kWgPerCu = 2;             // 8 waves per CU, 2 per SIMD
constexpr int kCus = 256;               // CUs the plan's grid is recorded for; launches use the device's
constexpr int kPitch = 84;              // LDS row pitch in floats (see above)
constexpr unsigned kOob = 0xFFFFFFF0u;

struct HeadF32Args {
  const float *x;
  const float *w;
  const float *bias;
  float *y;
  int N, H, W;
  int tiles_x, tiles_y, ntiles;
};

template <int R>
struct Geo {
  static constexpr int P = (R - 1) / 2;
  static constexpr int LW = kTW + R - 1;          // staged columns
  static constexpr int LH = kTH + R - 1;          // staged rows
  static_assert(kPitch >= LW, "rows fit their pitch");
  static constexpr int ELEMS = LH * LW;
  static constexpr int NLD = (ELEMS + kThreads - 1) / kThreads;   // loads per thread and tile
  static constexpr int DUMMY = LH * kPitch;       // where the past-the-tile load slots write
  static constexpr int SLOTS = DUMMY + 4;         // LDS floats per buffer
  static constexpr int NKS = (R * R + 3) / 4;     // k steps of 4 taps
};

// Issues the loads of tile t's input (with halo) into v; out-of-image and
// past-the-tile elements, and every element when t is past the last tile,
// read 0 (no branch: the loads stay in flight across the caller's work).
template <int R>
__device__ inline void load_tile(const HeadF32Args &a, int t, int tid, float (&v)[Geo<R>::NLD]) {
  using G = Geo<R>;
  const int tx = t % a.tiles_x;
  const int rest = t / a.tiles_x;
  const int ty = rest % a.tiles_y;
  const int n = rest / a.tiles_y;
  const int x0 = tx * kTW - G::P, y0 = ty * kTH - G::P;
  const size_t plane = (size_t)a.H * a.W;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(a.x) + (size_t)n * plane, (short)0, (int)(plane * 4), kBufferFlags);
#pragma unroll
  for (int q = 0; q < G::NLD; ++q) {
    const int e = tid + q * kThreads;
    const int gy = y0 + e / G::LW, gx = x0 + e % G::LW;
    const bool in = t < a.ntiles && e < G::ELEMS && (unsigned)gy < (unsigned)a.H && (unsigned)gx < (unsigned)a.W;
    const unsigned off = in ? (unsigned)(gy * a.W + gx) * 4u : kOob;
    v[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0));
  }
}

template <int R, int K, bool RELU>
__global__ __launch_bounds__(kThreads) void is_k9_head_f32(HeadF32Args a) {
  using G = Geo<R>;
  constexpr int NOB = K / 16;
  constexpr int NKS = G::NKS;
  __shared__ float tile[2][G::SLOTS];
  lds_poison(tile, sizeof(tile));

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g = lane >> 4;
  int t = blockIdx.x;
  if (t >= a.ntiles) return;

  // ---- Weights and bias (buffer loads: taps past R*R and a missing bias read 0).
  // B fragment (ob, ks) of this lane: w[16 ob + n16][4 ks + g].
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.w), (short)0, K * R * R * 4, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(a.bias), (short)0, a.bias ? K * 4 : 0, kBufferFlags);
  float wb[NOB][NKS];
  float bias[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) {
    const int c = 16 * ob + n16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int k = 4 * ks + g;
      const unsigned off = k < R * R ? (unsigned)(c * R * R + k) * 4u : kOob;
      wb[ob][ks] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, off, 0, 0));
    }
    bias[ob] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (unsigned)c * 4u, 0, 0));
  }
  // The tile loads are issued after the weight and bias loads (the scheduling
  // barrier keeps that order), and the wait below leaves only them in flight,
  // so that the tile loop never waits for these.
  __builtin_amdgcn_sched_barrier(0);
  float ld[G::NLD];
  load_tile<R>(a, t, tid, ld);
  __builtin_amdgcn_s_waitcnt(0x0F70 | G::NLD);

  // LDS offsets of this lane's A reads for tile row 0, one per k step (taps
  // past R*R read the tile origin and are replaced by 0 below).
  int toff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int k = 4 * ks + g;
    toff[ks] = k < R * R ? (k / R) * kPitch + 16 * wave + n16 + k % R : 0;
  }
  // LDS position of each of this thread's load slots (element e of the tile,
  // row-major with LW columns, at the row pitch; slots past the tile write a
  // spare element).
  int spos[G::NLD];
#pragma unroll
  for (int q = 0; q < G::NLD; ++q) {
    const int e = tid + q * kThreads;
    spos[q] = e < G::ELEMS ? (e / G::LW) * kPitch + e % G::LW : G::DUMMY;
  }
  const size_t plane = (size_t)a.H * a.W;

  // The tile's values go to LDS at the end of the previous iteration (the
  // first tile's here): written at the top of the loop body, the wait for
  // the prefetch loads would also cover the previous tile's output stores,
  // which went out after them (vector memory operations retire in issue
  // order), and the compiler's count for the first iteration, with no stores
  // in flight, is the one it keeps for every iteration.
#pragma unroll
  for (int q = 0; q < G::NLD; ++q) tile[0][spos[q]] = ld[q];
  for (int buf = 0; t < a.ntiles; t += gridDim.x, buf ^= 1) {
    // tile[buf] is complete, and every wave has finished reading tile[buf ^ 1].
    __syncthreads();
    load_tile<R>(a, t + (int)gridDim.x, tid, ld);

    const int tx = t % a.tiles_x;
    const int rest = t / a.tiles_x;
    const int ty = rest % a.tiles_y;
    const int n = rest / a.tiles_y;
    const int gx = tx * kTW + 16 * wave + 4 * g;   // first of this lane's 4 output pixels
    const bool col_in = gx < a.W;                  // W % 4 == 0: the 4 pixels are all in or all out
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        a.y + (size_t)n * plane * K, (short)0, (int)(plane * K * 4), kBufferFlags);
    const float *tb = tile[buf];
    // Fully unrolled: an inner loop holding only stores would make the
    // compiler wait for the prefetch loads before entering it.
#pragma unroll
    for (int r = 0; r < kTH; ++r) {
      float av[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const float v = tb[toff[ks] + r * kPitch];
        av[ks] = (4 * ks + g < R * R) ? v : 0.f;
      }
      const int gy = ty * kTH + r;
      const bool in = col_in & (gy < a.H);
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob) {
        float4v acc = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ks], wb[ob][ks], acc, 0, 0, 0);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = acc[e] + bias[ob];
          if constexpr (RELU) o[e] = fmaxf(o[e], 0.f);
        }
        const unsigned off =
            in ? (unsigned)(((size_t)(16 * ob + n16) * plane + (size_t)gy * a.W + gx) * 4u) : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4v, float4v{o[0], o[1], o[2], o[3]}), ry,
                                               off, 0, 0);
      }
    }
    // The next tile's values into the other buffer (past the last tile: zeros).
#pragma unroll
    for (int q = 0; q < G::NLD; ++q) tile[buf ^ 1][spos[q]] = ld[q];
  }
}

using K9Fn = void (*)(HeadF32Args);

template <int R, bool RELU>
K9Fn pick_k(int k) {
  if (k == 16) return is_k9_head_f32<R, 16, RELU>;
  if (k == 32) return is_k9_head_f32<R, 32, RELU>;
  if (k == 64) return is_k9_head_f32<R, 64, RELU>;
  return nullptr;
}

template <bool RELU>
K9Fn pick(int r, int k) {
  if (r == 3) return pick_k<3, RELU>(k);
  if (r == 5) return pick_k<5, RELU>(k);
  return nullptr;
}

}  // namespace

bool configure_head_f32(Plan &p) {
  const conv2d_desc &d = p.d;
  if (d.layout != IS_NCHW || d.in_dtype != IS_F32 || d.out_dtype != IS_F32 || d.separable) return false;
  if (d.c != 1 || d.r != d.s || pick<false>(d.r, d.k) == nullptr) return false;
  if (d.w % 4 != 0) return false;                                // 16-byte output vectors
  if (4.0 * d.h * (double)d.w * d.k >= 2.0e9) return false;     // 32-bit offsets inside one image's output
  const long long tiles = (long long)((d.w + kTW - 1) / kTW) * ((d.h + kTH - 1) / kTH) * d.n;
  if (tiles > (1LL << 31) - 1) return false;
  p.kid = kHeadNchwF32;
  p.name = "is_k9_head_f32";
  p.nseg = (d.w + kTW - 1) / kTW;
  p.nstrip = (d.h + kTH - 1) / kTH;
  p.ntiles = (int)tiles;
  p.grid_x = (int)(tiles < kCus * kWgPerCu ? tiles : kCus * kWgPerCu);
  p.grid_y = p.grid_z = 1;
  p.block = kThreads;
  p.lds = 2 * ((kTH + d.r - 1) * kPitch + 4) * 4;
  p.tile_w = kTW;
  p.tile_h = kTH;
  return true;
}

hipError_t launch_head_f32(const Plan &p, const float *x, const float *w, const float *b, float *y,
                           hipStream_t s) {
  const K9Fn fn = p.d.relu ? pick<true>(p.d.r, p.d.k) : pick<false>(p.d.r, p.d.k);
  if (!fn) return hipErrorInvalidValue;
  if (p.ntiles == 0) return hipSuccess;
  HeadF32Args a;
  a.x = x;
  a.w = w;
  a.bias = b;
  a.y = y;
  a.N = p.d.n;
  a.H = p.d.h;
  a.W = p.d.w;
  a.tiles_x = p.nseg;
  a.tiles_y = p.nstrip;
  a.ntiles = p.ntiles;
  // Persistent over the tiles: kWgPerCu workgroups per CU of this device.
  const long long cap = (long long)device_cu_count() * kWgPerCu;
  const int grid = (int)(p.ntiles < cap ? p.ntiles : cap);
  return launch_kernel(fn, dim3(grid), dim3(p.block), 0, s, a);
}

}  // namespace is
