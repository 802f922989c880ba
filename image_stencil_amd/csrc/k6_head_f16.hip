// k6_head_f16.hip -- fp16 NHWC layer with one input channel (a network's first
// layer: 1 -> K, K in {16, 32, 64}, 3x3 or 5x5), fp32 accumulation, fp16 output.
//
// With a single input channel the contraction of "Optimizing convolution
// kernels - CNNs in Vulkan Part 2/3" ("Where we left off": the sum over
// channels and filter taps) runs over the R*S <= 32 taps only, one k step of
// v_mfma_f32_16x16x32_f16 (the first layer of the pages' upscaling network,
// "Reducing memory traffic" table: 1 -> 64, 5x5). The layer writes K fp16
// values per pixel and reads one, so it is bound by the HBM write stream; the
// design keeps that stream busy from the first cycle to the last:
//  * persistent workgroups of 4 waves (one per CU) walk tiles of kTH rows x 64
//    columns; the input tile with its halo ((kTH + R - 1) x (64 + R - 1) fp16
//    values) of the NEXT tile is loaded into registers (branch-free buffer
//    loads, 0 outside the image) while the current tile is computed and
//    stored, then written to the other of two LDS buffers;
//  * wave w owns columns 16w .. +16 of every tile row; per row, lane (n16, g)
//    gathers taps 8g .. 8g+7 of pixel n16 from LDS into one B fragment (taps
//    past R*R are 0), and one MFMA per 16 output channels (A = 16 channels x
//    32 taps, zero-padded weights) gives 4 channels of the pixel per lane;
//  * the A rows of blocks 2p and 2p+1 are permuted so that a lane's 8 results
//    of the two blocks are the consecutive channels 32p + 8g .. +8: bias
//    (fp32), optional ReLU, fp16 rounding (nearest even) and one 16-byte
//    store per lane and block pair; the 4 lanes of a pixel fill 64 bytes of
//    its channel line.
#include "common.hpp"
#include "internal.hpp"

namespace is {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

constexpr int kTH = 32;                 // tile rows
constexpr int kTW = 64;                 // tile columns (4 waves x 16)
constexpr int kThreads = 256;
constexpr int kWgPerCu = 1;
constexpr int kCus = 256;   // CUs the plan's grid is recorded for; launches use the device's
constexpr unsigned kOob = 0xFFFFFFF0u;

struct HeadArgs {
  const _Float16 *x;
  const _Float16 *w;
  const float *bias;
  _Float16 *y;
  int N, H, W, relu;
  int tiles_x, tiles_y, ntiles;
};

// Output channel of row m of A block ob: blocks 2p and 2p+1 interleave in
// groups of 4 so that D rows 4g .. 4g+3 of both blocks are the channels
// 32p + 8g .. 32p + 8g + 7 (one 16-channel block: the identity).
template <int K>
__device__ constexpr int a_row_channel(int ob, int m) {
  if constexpr (K == 16) {
    return m;
  } else {
    return 32 * (ob >> 1) + 8 * (m >> 2) + 4 * (ob & 1) + (m & 3);
  }
}

// LDS row pitch (fp16 elements) of the staged tile. A B-fragment gather reads,
// for one tap slot j, 16 consecutive pixels of each of the 4 lane groups g at
// taps 8g + j, i.e. 4 rows of the tile; with rows LW = 64 + R - 1 apart those 4
// runs of 8 banks overlap (up to 3 distinct dwords per bank for R = 5, 2 for
// R = 3, counting 64 banks of 4 bytes). Pitches of 136 (R = 3) and 142 (R = 5)
// elements put the 4 runs on disjoint banks for every j and every wave.
constexpr int tile_pitch(int R) { return R == 3 ? 136 : (R == 5 ? 142 : kTW + R - 1); }

template <int R>
struct TileGeo {
  static constexpr int P = (R - 1) / 2;
  static constexpr int LW = kTW + R - 1;          // staged columns
  static constexpr int LH = kTH + R - 1;          // staged rows
  static constexpr int LWP = tile_pitch(R);       // LDS row pitch
  static_assert(LWP >= LW, "rows fit their pitch");
  static constexpr int ELEMS = LH * LW;
  static constexpr int NLD = (ELEMS + kThreads - 1) / kThreads;
  static constexpr int DUMMY = LH * LWP;          // where the past-the-tile load slots write
  static constexpr int SLOTS = DUMMY + 2;         // LDS elements per buffer
};

// Issues the loads of tile t's input (with halo) into v; out-of-image and
// past-the-tile elements, and every element when t is past the last tile,
// read 0 (no branch: the loads stay in flight across the caller's work).
template <int R>
__device__ inline void load_tile(const HeadArgs &a, int t, int tid, unsigned (&v)[TileGeo<R>::NLD]) {
  using G = TileGeo<R>;
  const int tx = t % a.tiles_x;
  const int rest = t / a.tiles_x;
  const int ty = rest % a.tiles_y;
  const int n = rest / a.tiles_y;
  const int x0 = tx * kTW - G::P, y0 = ty * kTH - G::P;
  const size_t plane = (size_t)a.H * a.W;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16 *>(a.x) + (size_t)n * plane, (short)0, (int)(plane * 2), kBufferFlags);
#pragma unroll
  for (int q = 0; q < G::NLD; ++q) {
    const int e = tid + q * kThreads;
    const int gy = y0 + e / G::LW, gx = x0 + e % G::LW;
    const bool in = t < a.ntiles && e < G::ELEMS && (unsigned)gy < (unsigned)a.H && (unsigned)gx < (unsigned)a.W;
    const unsigned off = in ? (unsigned)(gy * a.W + gx) * 2u : kOob;
    v[q] = __builtin_amdgcn_raw_buffer_load_b16(rx, off, 0, 0);
  }
}

template <int R, int K>
__global__ __launch_bounds__(kThreads) void is_k6_head_f16(HeadArgs a) {
  using G = TileGeo<R>;
  constexpr int NOB = K / 16;
  static_assert(R * R <= 32, "the taps fit one k step");
  // Padded to whole load rounds, so that every thread writes every round
  // (branch-free: a conditional write would leave the compiler unsure
  // which prefetch loads are still in flight).
  __shared__ _Float16 tile[2][G::SLOTS];
  lds_poison(tile, sizeof(tile));

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g = lane >> 4;
  int t = blockIdx.x;
  if (t >= a.ntiles) return;

  // ---- Weights and bias (buffer loads: taps past R*R and a missing bias read 0).
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16 *>(a.w), (short)0, K * R * R * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(a.bias), (short)0, a.bias ? K * 4 : 0, kBufferFlags);
  half8 wa[NOB];
  float bias[NOB][4];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) {
    const int c = a_row_channel<K>(ob, n16);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = 8 * g + j;
      const unsigned off = k < R * R ? (unsigned)(c * R * R + k) * 2u : kOob;
      wa[ob][j] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rw, off, 0, 0));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      bias[ob][e] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rb, (unsigned)a_row_channel<K>(ob, 4 * g + e) * 4u, 0, 0));
  }
  // The tile loads are issued after the weight and bias loads (the
  // scheduling barrier keeps that order), and the wait below leaves only
  // them in flight: weights and bias must be in registers before the tile
  // loop, or the compiler, unable to tell them from the loop's own stores at
  // the loop header, waits on those stores every tile.
  __builtin_amdgcn_sched_barrier(0);
  unsigned ld[G::NLD];
  load_tile<R>(a, t, tid, ld);
  __builtin_amdgcn_s_waitcnt(0x0F70 | G::NLD);

  // LDS offsets of this lane's 8 taps for tile row 0 (taps past R*R read the
  // tile origin and are replaced by 0 below).
  int toff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = 8 * g + j;
    toff[j] = k < R * R ? (k / R) * G::LWP + 16 * wave + n16 + k % R : 0;
  }
  // LDS position of each of this thread's load slots (element e of the tile,
  // row-major with LW columns, at its row's pitch; slots past the tile write a
  // spare element).
  int spos[G::NLD];
#pragma unroll
  for (int q = 0; q < G::NLD; ++q) {
    const int e = tid + q * kThreads;
    spos[q] = e < G::ELEMS ? (e / G::LW) * G::LWP + e % G::LW : G::DUMMY;
  }
  const size_t plane = (size_t)a.H * a.W;

  for (int buf = 0; t < a.ntiles; t += gridDim.x, buf ^= 1) {
#pragma unroll
    for (int q = 0; q < G::NLD; ++q)
      tile[buf][spos[q]] = __builtin_bit_cast(_Float16, (unsigned short)ld[q]);
    __syncthreads();
    load_tile<R>(a, t + (int)gridDim.x, tid, ld);

    const int tx = t % a.tiles_x;
    const int rest = t / a.tiles_x;
    const int ty = rest % a.tiles_y;
    const int n = rest / a.tiles_y;
    const int gx = tx * kTW + 16 * wave + n16;
    const bool col_in = gx < a.W;
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        a.y + (size_t)n * plane * K, (short)0, (int)(plane * K * 2), kBufferFlags);
    const _Float16 *tb = tile[buf];
    // Fully unrolled: an inner loop holding only stores would make the
    // compiler wait for the prefetch loads before entering it.
#pragma unroll
    for (int r = 0; r < kTH; ++r) {
      half8 b;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const _Float16 v = tb[toff[j] + r * G::LWP];
        b[j] = (8 * g + j < R * R) ? v : (_Float16)0.f;
      }
      const int gy = ty * kTH + r;
      const bool in = col_in & (gy < a.H);
      const unsigned pix = (unsigned)(gy * a.W + gx) * (unsigned)K;
      float4v acc[NOB];
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob)
        acc[ob] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[ob], b, float4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      _Float16 hv[NOB][4];
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = acc[ob][e] + bias[ob][e];
          if (a.relu) v = fmaxf(v, 0.f);
          hv[ob][e] = (_Float16)v;
        }
      }
      if constexpr (K == 16) {
        const unsigned off = in ? (pix + 4u * g) * 2u : kOob;
        half4 h4 = {hv[0][0], hv[0][1], hv[0][2], hv[0][3]};
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2v, h4), ry, off, 0, 0);
      } else {
#pragma unroll
        for (int p = 0; p < NOB / 2; ++p) {
          const unsigned off = in ? (pix + 32u * p + 8u * g) * 2u : kOob;
          half8 h8 = {hv[2 * p][0], hv[2 * p][1], hv[2 * p][2], hv[2 * p][3],
                      hv[2 * p + 1][0], hv[2 * p + 1][1], hv[2 * p + 1][2], hv[2 * p + 1][3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4v, h8), ry, off, 0, 0);
        }
      }
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
  p.grid_x = (int)(tiles < kCus * kWgPerCu ? tiles : kCus * kWgPerCu);
  p.grid_y = p.grid_z = 1;
  p.block = kThreads;
  p.lds = 2 * ((kTH + d.r - 1) * tile_pitch(d.r) + 2) * 2;
  p.tile_w = kTW;
  p.tile_h = kTH;
  return true;
}

hipError_t launch_head_f16(const Plan &p, const _Float16 *x, const _Float16 *w, const float *b, _Float16 *y,
                           hipStream_t s) {
  auto fn = pick(p.d.r, p.d.k);
  if (!fn) return hipErrorInvalidValue;
  if (p.ntiles == 0) return hipSuccess;
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
  a.ntiles = p.ntiles;
  // Persistent over the tiles: kWgPerCu workgroups per CU of this device.
  const long long cap = (long long)device_cu_count() * kWgPerCu;
  const int grid = (int)(p.ntiles < cap ? p.ntiles : cap);
  return launch_kernel(fn, dim3(grid), dim3(p.block), 0, s, a);
}

}  // namespace is
