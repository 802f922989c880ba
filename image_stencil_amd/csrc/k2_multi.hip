// k2_multi.hip -- multi-channel fp32 NCHW layer, square odd filters r = s in {1, 3, 5}.
//
// The "general case" kernel of "Optimizing Memory Efficiency for Convolution
// Kernels on Kepler GPUs" (arXiv 1705.10591; its Algorithm 2 and the sections
// on the general-case thread layout and memory access), rebuilt for CDNA:
//  * a workgroup of 4 waves owns a 64 x 16 tile of output pixels for FT output
//    channels (the page's TB over F_TB filters and one image block);
//  * input channels are staged CS at a time in LDS with their halo (the page's
//    C_SH channels of image blocks kept in shared memory), straight from HBM
//    to LDS with gfx950's buffer_load ... lds, double-buffered so that the
//    next slab streams in while this one is computed (the page's prefetch);
//    reads outside the image return 0 through the buffer range check;
//  * each lane accumulates 4 contiguous pixels x FT output channels in
//    registers (the page's W_T x F_T register block with one thread owning
//    contiguous outputs), reading per input row one 16-byte LDS vector plus
//    its left/right neighbours through DPP row shifts (the page's row of
//    W_T + K - 1 pixels reused across K rounds);
//  * filter taps are wave-uniform and live in scalar registers: every FMA takes
//    its weight as the scalar operand (the page's broadcast of filter values);
//  * output channels beyond FT are spread over workgroups (the page's TB_X),
//    bias and ReLU are applied in the epilogue and each lane writes 16-byte
//    vectors, so a wave's stores are whole 256-byte row segments.
#include "common.hpp"
#include "internal.hpp"

namespace is {
namespace {

// Cache policy of the output stores: non-temporal. Each output value is
// written once; with F planes per tile the store stream is most of the
// traffic (8 filters on one channel: 512 of 576 MB), and streaming stores
// measured 23% faster there (124.9 -> 96.1 us on 4096x4096), with no loss in
// the layer-by-layer chain, whose next layer reads these planes back.
constexpr int kNonTemporalStore = 2;

constexpr int kTW = 64;              // output columns per tile (16 lanes x 4)
constexpr int kTH = 16;              // output rows per tile (4 waves x 4 rows)
constexpr int kThreads = 256;
constexpr int kG = kTW / 4 + 2;      // 16-byte groups per staged row: x0-4 .. x0+TW+3
constexpr int kMainG = kTW / 4;      // the tile's own groups, x0 .. x0+TW-1 (256 bytes)
constexpr unsigned kOob = 0xFFFFFFF0u;   // byte offset past any buffer: reads 0

constexpr int kDppRowShr1 = 0x111;   // lane reads lane-1 inside its row of 16
constexpr int kDppRowShl1 = 0x101;   // lane reads lane+1 inside its row of 16

__device__ __forceinline__ float row_prev(float src, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), kDppRowShr1,
                                                    0xf, 0xf, false));
}
__device__ __forceinline__ float row_next(float src, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), kDppRowShl1,
                                                    0xf, 0xf, false));
}

template <int R, int CS>
struct Geo {
  static constexpr int P = (R - 1) / 2;
  static constexpr int LH = kTH + R - 1;                 // staged rows
  static constexpr int V4 = CS * LH * kG;                // 16-byte vectors per slab
  // Slab layout in LDS: first every staged row's 16 own groups (rows 256 bytes
  // apart), then every row's 2 halo groups (left, right). A read takes 4 rows x
  // 16 lanes of consecutive groups; gfx950 serves such a read without bank
  // conflicts only when its rows lie a multiple of 256 bytes apart (rows of
  // 18 groups, 288 bytes apart, measured 2-way conflicts).
  static constexpr int MAINV4 = CS * LH * kMainG;
  static constexpr int CHUNKS = (V4 + 63) / 64;          // wave-sized DMA chunks
  static constexpr int ROUNDS = (CHUNKS + 3) / 4;        // chunks per wave (4 waves)
  static constexpr int PADV4 = ROUNDS * 4 * 64;          // LDS vectors per buffer
};

// Issue this wave's DMA chunks of one slab: chunk j*4+wave covers LDS vectors
// [(j*4+wave)*64, +64); lane i writes vector (j*4+wave)*64 + i.
template <int R, int CS>
__device__ __forceinline__ void issue_slab(__amdgpu_buffer_rsrc_t rs, float4 *buf, int wave,
                                           const unsigned *voff) {
  using G = Geo<R, CS>;
#pragma unroll
  for (int j = 0; j < G::ROUNDS; ++j) {
    float4 *dst = buf + (j * 4 + wave) * 64;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)dst, 16, voff[j],
                                             0, 0, 0);
  }
}

// D2S: the layer has 4 output channels and its output goes through a 2x
// depth-to-space, out[n][0][2i+dy][2j+dx] = z[n][2dy+dx][i][j] (y is then
// N x 1 x 2H x 2W), done in the epilogue instead of a pass of its own.
template <int R, int FT, int CS, bool RELU, bool D2S>
__global__ __launch_bounds__(kThreads) void is_k2_multi(const float *__restrict__ x,
                                                        const float *__restrict__ w,
                                                        const float *__restrict__ bias,
                                                        float *__restrict__ y, int C, int H, int W, int K,
                                                        int ntx, int nty, int nkg, int ntiles) {
  using G = Geo<R, CS>;
  constexpr int P = G::P;
  __shared__ float4 buf0[G::PADV4];
  __shared__ float4 buf1[G::PADV4];
  lds_poison(buf0, sizeof(buf0));
  lds_poison(buf1, sizeof(buf1));

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane >> 4;          // row inside the wave's 4 rows
  const int lc = lane & 15;          // 4-column group inside the tile

  const int tile = xcd_remap(blockIdx.x, ntiles);
  const int tx = tile % ntx;
  const int ty = (tile / ntx) % nty;
  const int kg = (tile / (ntx * nty)) % nkg;
  const int n = tile / (ntx * nty * nkg);
  const int x0 = tx * kTW, y0 = ty * kTH;
  const size_t HW = (size_t)H * W;

  // Per-lane byte offsets of this lane's DMA vectors inside a slab (same for
  // every slab: the resource base moves instead).
  unsigned voff[G::ROUNDS];
#pragma unroll
  for (int j = 0; j < G::ROUNDS; ++j) {
    const int q = (j * 4 + wave) * 64 + lane;
    int c, lrow, g;
    if (q < G::MAINV4) {
      c = q / (G::LH * kMainG);
      const int rem = q - c * (G::LH * kMainG);
      lrow = rem / kMainG;
      g = 1 + rem - lrow * kMainG;
    } else {
      const int h = q - G::MAINV4;
      c = h / (G::LH * 2);
      const int rem = h - c * (G::LH * 2);
      lrow = rem / 2;
      g = (rem & 1) ? kG - 1 : 0;
    }
    const int gy = y0 - P + lrow;
    const int gx = x0 - 4 + 4 * g;
    const bool in = q < G::V4 && gy >= 0 && gy < H && gx >= 0 && gx < W;
    voff[j] = in ? (unsigned)(((size_t)c * HW + (size_t)gy * W + gx) * 4) : kOob;
  }

  const float *xn = x + (size_t)n * C * HW;
  const unsigned slab_bytes = (unsigned)(CS * HW * 4);
  auto slab_rsrc = [&](int c0) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(xn + (size_t)c0 * HW), (short)0,
                                             (int)slab_bytes, kBufferFlags);
  };

  float acc[FT][4];
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[f][p] = 0.f;

  // Weights of this group's first channel, read through the constant address
  // space so that the wave-uniform loads become scalar loads into SGPRs.
  const __attribute__((address_space(4))) float *wk =
      (const __attribute__((address_space(4))) float *)(w + (size_t)kg * FT * C * R * R);
  const int row0 = wave * 4 + lr;                      // tile row of this lane's outputs
  // LDS vector indices of this lane's 16-byte input vector and of the halo
  // vector it may need (lc 0: left of the tile; lc 15: right; others share
  // lane 0's address so the read is a broadcast).
  const int halo_g = lc == 15 ? 1 : 0;

  // One input channel: its R row windows in VGPRs, then every output channel f
  // in turn with its R*R taps in SGPRs. The taps of channel f+2 are requested
  // while f computes (scalar loads of 8 + 1 dwords), and scheduling barriers
  // keep the compiler from hoisting all of them at once, which would exhaust
  // the scalar registers.
  auto compute = [&](const float4 *bf, int c0) {
    // The next channel's LDS vectors are read before this channel's FMAs and
    // turned into its window after them, so that the LDS latency is hidden.
    float4 raw_o[2][R], raw_h[2][R];
    auto read_raw = [&](int c, int b) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int crow = c * G::LH + row0 + u;
        raw_o[b][u] = bf[crow * kMainG + lc];
        if constexpr (P > 0) raw_h[b][u] = bf[G::MAINV4 + crow * 2 + halo_g];
      }
    };
    read_raw(0, 0);
#pragma unroll
    for (int c = 0; c < CS; ++c) {
      float win[R][4 + 2 * P];
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const float4 o4 = raw_o[c & 1][u];
        win[u][P + 0] = o4.x; win[u][P + 1] = o4.y; win[u][P + 2] = o4.z; win[u][P + 3] = o4.w;
        if constexpr (P > 0) {
          const float4 h4 = raw_h[c & 1][u];
          const float hv[4] = {h4.x, h4.y, h4.z, h4.w};
          const float ov[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
          for (int q = 1; q <= P; ++q) {
            win[u][P - q] = row_prev(ov[4 - q], hv[4 - q]);
            win[u][P + 3 + q] = row_next(ov[q - 1], hv[q - 1]);
          }
        }
      }
      if (c + 1 < CS) read_raw(c + 1, (c + 1) & 1);
      constexpr int D = 2;   // prefetch distance in output channels
      float wt[D + 1][R * R];
      auto load_taps = [&](float *dst, int f) {
        // The empty asm makes the offset opaque, so the loads cannot be hoisted
        // above this point or merged with those of other channels.
        int off = (c0 + c) * R * R + f * C * R * R;
        asm volatile("" : "+s"(off));
#pragma unroll
        for (int t = 0; t < R * R; ++t) dst[t] = wk[off + t];
      };
#pragma unroll
      for (int f = 0; f < D && f < FT; ++f) load_taps(wt[f], f);
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        if (f + D < FT) load_taps(wt[(f + D) % (D + 1)], f + D);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < R; ++u)
#pragma unroll
          for (int v = 0; v < R; ++v)
#pragma unroll
            for (int p = 0; p < 4; ++p)
              acc[f][p] = __builtin_fmaf(wt[f % (D + 1)][u * R + v], win[u][p + v], acc[f][p]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const int nslab = C / CS;
  issue_slab<R, CS>(slab_rsrc(0), buf0, wave, voff);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int s = 0; s < nslab; s += 2) {
    if (s + 1 < nslab) issue_slab<R, CS>(slab_rsrc((s + 1) * CS), buf1, wave, voff);
    compute(buf0, s * CS);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (s + 1 >= nslab) break;
    if (s + 2 < nslab) issue_slab<R, CS>(slab_rsrc((s + 2) * CS), buf0, wave, voff);
    compute(buf1, (s + 1) * CS);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Epilogue: bias, ReLU, 16-byte stores (dropped outside the image).
  const int oy = y0 + row0;
  const int ox = x0 + 4 * lc;
  const bool in = oy < H && ox < W;
  if constexpr (D2S) {
    static_assert(FT == 4, "depth-to-space takes 4 channels");
    // This lane's 4 columns of the 4 channels become 8 columns of output rows
    // 2*oy (channels 0, 1 interleaved) and 2*oy + 1 (channels 2, 3): two
    // 16-byte stores per row; W % 4 == 0 keeps them whole.
    float o[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const float b = bias ? bias[f] : 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        o[f][p] = acc[f][p] + b;
        if constexpr (RELU) o[f][p] = fmaxf(o[f][p], 0.f);
      }
    }
    float *yn = y + (size_t)n * 4 * HW;
    const __amdgpu_buffer_rsrc_t rs_o =
        __builtin_amdgcn_make_buffer_rsrc(yn, (short)0, (int)(4 * HW * 4), kBufferFlags);
#pragma unroll
    for (int dy = 0; dy < 2; ++dy) {
      const int c0 = 2 * dy;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned off =
            in ? (unsigned)((((size_t)(2 * oy + dy) * (2 * W)) + 2 * ox + 4 * h) * 4) : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int,
                               make_float4(o[c0][2 * h], o[c0 + 1][2 * h], o[c0][2 * h + 1], o[c0 + 1][2 * h + 1])),
            rs_o, off, 0, 0);
      }
    }
    return;
  }
  float *yn = y + ((size_t)n * K + (size_t)kg * FT) * HW;
  const __amdgpu_buffer_rsrc_t rs_o = __builtin_amdgcn_make_buffer_rsrc(
      yn, (short)0, (int)(FT * HW * 4), kBufferFlags);
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    const float b = bias ? bias[kg * FT + f] : 0.f;
    float o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      o[p] = acc[f][p] + b;
      if constexpr (RELU) o[p] = fmaxf(o[p], 0.f);
    }
    const unsigned off = in ? (unsigned)(((size_t)f * HW + (size_t)oy * W + ox) * 4) : kOob;
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, make_float4(o[0], o[1], o[2], o[3])),
        rs_o, off, 0, kNonTemporalStore);
  }
}

using K2Fn = void (*)(const float *, const float *, const float *, float *, int, int, int, int, int, int, int,
                      int);

template <bool RELU>
K2Fn pick(int r, int ft, int cs) {
#define IS_K2_CASE(RR, FF, CC) \
  if (r == RR && ft == FF && cs == CC) return is_k2_multi<RR, FF, CC, RELU, false>;
  // multi-channel layers (slabs of 4 channels)
  IS_K2_CASE(3, 32, 4) IS_K2_CASE(3, 16, 4) IS_K2_CASE(3, 8, 4) IS_K2_CASE(3, 4, 4)
  IS_K2_CASE(5, 32, 4) IS_K2_CASE(1, 32, 4) IS_K2_CASE(1, 16, 4) IS_K2_CASE(1, 8, 4)
  IS_K2_CASE(1, 4, 4)
  // one input channel and F filters (the page's special case with F > 1)
  IS_K2_CASE(5, 32, 1) IS_K2_CASE(3, 32, 1) IS_K2_CASE(1, 32, 1)
  IS_K2_CASE(5, 16, 1) IS_K2_CASE(3, 16, 1) IS_K2_CASE(1, 16, 1)
  IS_K2_CASE(5, 8, 1) IS_K2_CASE(3, 8, 1) IS_K2_CASE(1, 8, 1)
  IS_K2_CASE(5, 4, 1) IS_K2_CASE(3, 4, 1) IS_K2_CASE(1, 4, 1)
  IS_K2_CASE(5, 2, 1) IS_K2_CASE(3, 2, 1) IS_K2_CASE(1, 2, 1)
#undef IS_K2_CASE
  return nullptr;
}

// With the depth-to-space epilogue: the 3x3 layer with 4 output channels.
template <bool RELU>
K2Fn pick_d2s(int r, int ft, int cs) {
  if (r == 3 && ft == 4 && cs == 4) return is_k2_multi<3, 4, 4, RELU, true>;
  return nullptr;
}

}  // namespace

bool configure_multi(Plan &p, int param) {
  const conv2d_desc &d = p.d;
  if (d.layout != IS_NCHW || d.in_dtype != IS_F32 || d.r != d.s) return false;
  if (d.w % 4 != 0) return false;
  const int cs = (d.c % 4 == 0) ? 4 : 1;
  // Output channels per workgroup: as many as divide K, up to 32. With one
  // input channel there is a single slab, so a workgroup loads, computes and
  // stores in sequence; 16 channels give twice the workgroups to overlap those
  // phases (the 1 -> 32 5x5 layer of a 1280x720 frame: 35.5 against 38.5 us).
  int ft = 0;
  for (int f : {32, 16, 8, 4, 2})
    if (d.k % f == 0 && !(d.c == 1 && f == 32 && d.k % 16 == 0 && pick<false>(d.r, 16, cs))) {
      ft = f;
      break;
    }
  if (param != 0) {   // a tuning variant: that many output channels per workgroup
    if (d.k % param != 0) return false;
    ft = param;
  }
  if (ft == 0 || pick<false>(d.r, ft, cs) == nullptr) return false;
  // One slab's bytes and each image's bytes must stay below 4 GB for the
  // 32-bit buffer offsets.
  const double img_bytes = 4.0 * d.c * (double)d.h * d.w;
  const double out_bytes = 4.0 * d.k * (double)d.h * d.w;
  if (img_bytes >= 4.0e9 || out_bytes >= 4.0e9) return false;
  p.kid = kMultiChannel;
  p.name = "is_k2_multi";
  p.nseg = (d.w + kTW - 1) / kTW;
  p.nstrip = (d.h + kTH - 1) / kTH;
  p.strip_rows = ft;   // output channels per workgroup
  p.vec = cs;          // input channels per LDS slab
  const long long tiles = (long long)p.nseg * p.nstrip * (d.k / ft) * d.n;
  if (tiles > (1LL << 31) - 1) return false;
  p.ntiles = (int)tiles;
  p.grid_x = p.ntiles;
  p.grid_y = p.grid_z = 1;
  p.block = kThreads;
  const int lh = kTH + d.r - 1;
  const int chunks = (cs * lh * kG + 63) / 64;
  p.lds = 2 * ((chunks + 3) / 4) * 4 * 64 * 16;
  p.tile_w = kTW;
  p.tile_h = kTH;
  return true;
}

bool multi_d2s_supported(const Plan &p) {
  return p.kid == kMultiChannel && p.d.k == 4 && pick_d2s<false>(p.d.r, p.strip_rows, p.vec) != nullptr;
}

hipError_t launch_multi_d2s(const Plan &p, const float *x, const float *w, const float *b, float *y,
                            hipStream_t s) {
  const conv2d_desc &d = p.d;
  if (!multi_d2s_supported(p)) return hipErrorInvalidValue;
  const int ft = p.strip_rows, cs = p.vec;
  const K2Fn fn = d.relu ? pick_d2s<true>(d.r, ft, cs) : pick_d2s<false>(d.r, ft, cs);
  return launch_kernel(fn, dim3(p.grid_x), dim3(p.block), 0, s, x, w, b, y, d.c, d.h, d.w, d.k, p.nseg,
                       p.nstrip, d.k / ft, p.ntiles);
}

hipError_t launch_multi(const Plan &p, const float *x, const float *w, const float *b, float *y,
                        hipStream_t s) {
  const conv2d_desc &d = p.d;
  const int ft = p.strip_rows, cs = p.vec;
  const K2Fn fn = d.relu ? pick<true>(d.r, ft, cs) : pick<false>(d.r, ft, cs);
  if (!fn) return hipErrorInvalidValue;
  return launch_kernel(fn, dim3(p.grid_x), dim3(p.block), 0, s, x, w, b, y, d.c, d.h, d.w, d.k, p.nseg,
                     p.nstrip, d.k / ft, p.ntiles);
}

}  // namespace is
