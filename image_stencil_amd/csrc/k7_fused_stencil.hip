// k7_fused_stencil.hip -- two or three single-channel fp32 filters applied one
// after another in one pass (a stencil pipeline stage group).
//
// The fusion follows "Model-Based Warp Overlapped Tiling for Image Processing
// Programs on GPUs" (arXiv 1909.07190, abstract and its tiling scheme): each
// warp (here a wave64) owns an overlapped tile, evaluates every stage of the
// group on it in registers with warp-level exchange only, and writes only the
// last stage; the halo columns that neighbouring tiles also compute are
// recomputed instead of exchanged. Per stage the streaming scheme is the
// single-channel kernel's ("Optimizing Memory Efficiency for Convolution
// Kernels on Kepler GPUs", arXiv 1705.10591, special case, Algorithm 1):
//  * a wave owns a window of 256 columns (4 per lane) and sweeps a strip of
//    rows downward, one input row per step; row neighbours come from adjacent
//    lanes by DPP wave shifts (0 beyond the wave);
//  * each stage keeps its R rolling output rows in registers: an input row
//    adds its contribution to the R rows it touches, after which the oldest
//    row is complete and moves on to the next stage as that stage's input row
//    (the ring then rotates, so the unrolled code needs no slot indexing);
//  * an intermediate row or column outside the image is set to 0 before the
//    next stage reads it (each stage's own zero padding);
//  * the stages' halos shrink the valid part of the window: after all stages
//    lanes [a, 64 - a) hold finished columns, a = ceil(sum of Q / 4), so
//    windows overlap by 8a columns and a wave writes 256 - 8a of them;
//    vertically a strip computes sum(P) extra rows above and below;
//  * taps are wave-uniform scalar operands; rows are prefetched 4 steps ahead.
#include "common.hpp"
#include "internal.hpp"

namespace is {
namespace {

constexpr int kCols = 4 * kWave;   // window columns per wave
constexpr int kPF = 4;             // steps per unrolled block = rows prefetched ahead
constexpr unsigned kOob = 0xFFFFFFF0u;
// Output stores are non-temporal (the image is written once; measured 3-4%
// faster). Input loads keep the default policy: neighbouring windows and
// strips re-read the overlap rows and columns.
constexpr int kNonTemporal = 2;

struct FusedArgs {
  const float *x;
  float *y;
  const float *w[3];
  const float *b[3];
  int H, W;
  int relu_mask;                   // bit l: ReLU after stage l
  int strip_rows, nseg, nstrip, ntiles;
  int step;                        // output columns per window (256 - 8a)
  int lanes_off;                   // a
};

// The neighbour lane's value, 0 for the lane at the wave's edge (a DPP wave
// shift with bound control: the lane without a source reads zero, so no
// register has to hold a zero "old" value).
__device__ __forceinline__ float prev_lane_or_zero(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kDppWaveShr1, 0xf, 0xf, true));
}
__device__ __forceinline__ float next_lane_or_zero(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kDppWaveShl1, 0xf, 0xf, true));
}

template <int R>
struct Ring {
  float acc[R > 0 ? R : 1][4];
};

// Buffer resource of image row t when lo <= t < hi, else an empty one (loads
// read 0, stores are dropped, no memory access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float *base, int t, int lo, int hi, int W) {
  const bool in = t >= lo && t < hi;
  const float *p = base + (size_t)(in ? t : 0) * (size_t)W;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), (short)0, in ? W * 4 : 0, kBufferFlags);
}

// One stage on one input row (this lane's 4 columns): add the row to the R
// rolling output rows, hand out the oldest (now complete) one and rotate. A
// recycled slot starts at the stage's bias, so a finished row already holds
// bias + sum of products.
template <int R>
__device__ __forceinline__ void stage_row(Ring<R> &g, const float *wt, float bias, const float (&in)[4],
                                          float (&out)[4]) {
  constexpr int Q = (R - 1) / 2;
  float win[4 + 2 * Q];
#pragma unroll
  for (int i = 0; i < 4; ++i) win[Q + i] = in[i];
#pragma unroll
  for (int q = 1; q <= Q; ++q) {
    win[Q - q] = prev_lane_or_zero(in[4 - q]);
    win[Q + 3 + q] = next_lane_or_zero(in[q - 1]);
  }
  // Ring slot j holds output row (input row - Q + j): it takes filter row R-1-j.
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int s = 0; s < R; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) g.acc[j][i] = __builtin_fmaf(wt[(R - 1 - j) * R + s], win[i + s], g.acc[j][i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = g.acc[0][i];
#pragma unroll
  for (int j = 0; j + 1 < R; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) g.acc[j][i] = g.acc[j + 1][i];
#pragma unroll
  for (int i = 0; i < 4; ++i) g.acc[R - 1][i] = bias;
}

// ReLU and the zero padding of a finished row in one clamp per value: the
// median of (v, lo, hi) is max(v, 0) for lo = 0, hi = +inf (ReLU), v for
// lo = -inf, hi = +inf (none), and 0 for lo = hi = 0 (a row or column outside
// the image, which the next stage must read as zero).
struct Clamp {
  float lo, hi;
};
__device__ __forceinline__ Clamp row_clamp(bool relu, bool keep) {
  return Clamp{keep ? (relu ? 0.f : -__builtin_inff()) : 0.f, keep ? __builtin_inff() : 0.f};
}
__device__ __forceinline__ void finish_row(float (&v)[4], Clamp c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_fmed3f(v[i], c.lo, c.hi);
}

template <int R>
__device__ __forceinline__ void load_taps(float *dst, const float *w) {
  const __attribute__((address_space(4))) float *wk = (const __attribute__((address_space(4))) float *)w;
#pragma unroll
  for (int t = 0; t < R * R; ++t) dst[t] = wk[t];
}

template <int R1, int R2, int R3>
__global__ __launch_bounds__(kWave) void is_k7_fused_stencil(FusedArgs a) {
  constexpr int P1 = (R1 - 1) / 2, P2 = (R2 - 1) / 2, P3 = R3 > 0 ? (R3 - 1) / 2 : 0;
  constexpr int PS = P1 + P2 + P3;

  const int lane = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, a.ntiles);
  const int seg = tile % a.nseg;
  const int strip = (tile / a.nseg) % a.nstrip;
  const int n = tile / (a.nseg * a.nstrip);
  const int col = seg * a.step - 4 * a.lanes_off + 4 * lane;   // this lane's first column
  const bool col_in = col >= 0 && col < a.W;                    // W % 4 == 0: whole lane in or out
  const bool keep = col_in && lane >= a.lanes_off && lane < kWave - a.lanes_off;
  const int y0 = strip * a.strip_rows;
  const int rows_out = min(a.strip_rows, a.H - y0);
  const int NT = rows_out + 2 * PS;   // steps: input rows y0-PS .. y0+rows_out+PS-1
  const int t0 = y0 - PS;

  const size_t plane = (size_t)a.H * (size_t)a.W;
  const float *xp = a.x + (size_t)n * plane;
  float *yp = a.y + (size_t)n * plane;
  // Negative columns become offsets past any row (read 0); so do columns >= W.
  const unsigned off = (unsigned)col * 4u;
  const unsigned off_st = keep ? off : kOob;

  float w1[R1 * R1], w2[R2 * R2], w3[R3 > 0 ? R3 * R3 : 1];
  load_taps<R1>(w1, a.w[0]);
  load_taps<R2>(w2, a.w[1]);
  if constexpr (R3 > 0) load_taps<R3>(w3, a.w[2]);
  const float b1 = a.b[0] ? a.b[0][0] : 0.f;
  const float b2 = a.b[1] ? a.b[1][0] : 0.f;
  const float b3 = (R3 > 0 && a.b[2]) ? a.b[2][0] : 0.f;
  const bool relu1 = a.relu_mask & 1, relu2 = (a.relu_mask >> 1) & 1, relu3 = (a.relu_mask >> 2) & 1;

  Ring<R1> g1;
  Ring<R2> g2;
  Ring<R3> g3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < R1; ++j) g1.acc[j][i] = b1;
#pragma unroll
    for (int j = 0; j < R2; ++j) g2.acc[j][i] = b2;
#pragma unroll
    for (int j = 0; j < (R3 > 0 ? R3 : 1); ++j) g3.acc[j][i] = b3;
  }
  // The last stage's row is stored only inside the strip, so its clamp is
  // fixed; the inner stages' depend on the row (rows above or below the
  // image are zero padding for the next stage).
  const Clamp c_last = row_clamp(R3 > 0 ? relu3 : relu2, true);

  float pf[kPF][4];
#pragma unroll
  for (int p = 0; p < kPF; ++p) {
    const float4 v = __builtin_bit_cast(
        float4, __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(xp, t0 + p, 0, a.H, a.W), off, 0, 0));
    pf[p][0] = v.x; pf[p][1] = v.y; pf[p][2] = v.z; pf[p][3] = v.w;
    __builtin_amdgcn_sched_barrier(0);
  }

  // No branch inside the loop: steps past NT read rows whose results are
  // never stored (outside the strip's store range), so each unrolled block is
  // one straight sequence of loads, FMAs and stores.
  for (int kb = 0; kb < NT; kb += kPF) {
    static_for<kPF>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      const int t = t0 + kb + p;
      float in[4] = {pf[p][0], pf[p][1], pf[p][2], pf[p][3]};
      float o1[4], o2[4], o3[4];
      stage_row<R1>(g1, w1, b1, in, o1);
      const int e1 = t - P1;
      finish_row(o1, row_clamp(relu1, col_in && e1 >= 0 && e1 < a.H));
      stage_row<R2>(g2, w2, b2, o1, o2);
      const int e2 = e1 - P2;
      float *res = o2;
      int eL = e2;
      if constexpr (R3 > 0) {
        finish_row(o2, row_clamp(relu2, col_in && e2 >= 0 && e2 < a.H));
        stage_row<R3>(g3, w3, b3, o2, o3);
        eL = e2 - P3;
        finish_row(o3, c_last);
        res = o3;
      } else {
        finish_row(o2, c_last);
      }
      const __amdgpu_buffer_rsrc_t rs_o = row_rsrc(yp, eL, y0, y0 + rows_out, a.W);
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int,
                             make_float4(res[0], res[1], res[2], res[3])),
          rs_o, off_st, 0, kNonTemporal);
      __builtin_amdgcn_sched_barrier(0);
      const float4 v = __builtin_bit_cast(
          float4, __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(xp, t + kPF, 0, a.H, a.W), off, 0, 0));
      pf[p][0] = v.x; pf[p][1] = v.y; pf[p][2] = v.z; pf[p][3] = v.w;
    });
  }
}

using K7Fn = void (*)(FusedArgs);

K7Fn pick(const int *r, int count) {
#define IS_K7_2(A, B) \
  if (count == 2 && r[0] == A && r[1] == B) return is_k7_fused_stencil<A, B, 0>;
#define IS_K7_3(A, B, C) \
  if (count == 3 && r[0] == A && r[1] == B && r[2] == C) return is_k7_fused_stencil<A, B, C>;
  IS_K7_2(3, 3) IS_K7_2(3, 5) IS_K7_2(5, 3) IS_K7_2(5, 5)
  IS_K7_3(3, 3, 3) IS_K7_3(3, 3, 5) IS_K7_3(3, 5, 3) IS_K7_3(5, 3, 3)
  IS_K7_3(3, 5, 5) IS_K7_3(5, 3, 5) IS_K7_3(5, 5, 3) IS_K7_3(5, 5, 5)
  // one 7x7 filter in the group (two would need more scalar registers than
  // the taps of a wave can hold)
  IS_K7_2(7, 3) IS_K7_2(3, 7) IS_K7_2(7, 5) IS_K7_2(5, 7)
  IS_K7_3(7, 3, 3) IS_K7_3(3, 7, 3) IS_K7_3(3, 3, 7)
#undef IS_K7_2
#undef IS_K7_3
  return nullptr;
}

}  // namespace

FusedStencilGeo fused_stencil_geometry(const conv_chain_desc *d, int first, int count) {
  FusedStencilGeo g{};
  if (!d || d->dtype != IS_F32 || count < 2 || count > 3 || first < 0 || first + count > d->n_layers) return g;
  if (d->w % 4 != 0 || d->w <= 0 || d->h <= 0 || d->n <= 0) return g;
  int r[3], qs = 0;
  for (int l = 0; l < count; ++l) {
    const conv_layer_desc &L = d->layer[first + l];
    if (L.c != 1 || L.k != 1 || L.r != L.s) return g;
    r[l] = L.r;
    qs += (L.r - 1) / 2;
  }
  if (!pick(r, count)) return g;
  if ((double)d->h * d->w * 4.0 >= 2.0e9) return g;   // 32-bit offsets per image
  g.lanes_off = (qs + 3) / 4;
  g.step = kCols - 8 * g.lanes_off;
  g.nseg = (d->w + g.step - 1) / g.step;
  // Strip height as in the single-channel kernel (64 rows, fewer when the
  // image gives fewer than 4096 waves), but at least 16: every strip also
  // computes sum(P) rows above and below.
  int rows = 64;
  while (rows > 16 && (long long)g.nseg * ((d->h + rows - 1) / rows) * d->n < 4096) rows >>= 1;
  g.strip_rows = rows;
  g.nstrip = (d->h + rows - 1) / rows;
  const long long tiles = (long long)g.nseg * g.nstrip * d->n;
  if (tiles > (1LL << 31) - 1) return g;
  g.ntiles = (int)tiles;
  g.ok = true;
  return g;
}

hipError_t launch_fused_stencil(const conv_chain_desc *d, int first, int count, const float *x,
                                const float *const *w, const float *const *b, float *y, hipStream_t s) {
  const FusedStencilGeo g = fused_stencil_geometry(d, first, count);
  if (!g.ok) return hipErrorInvalidValue;
  int r[3] = {0, 0, 0};
  FusedArgs a{};
  a.x = x;
  a.y = y;
  a.relu_mask = 0;
  for (int l = 0; l < count; ++l) {
    r[l] = d->layer[first + l].r;
    a.w[l] = w[first + l];
    a.b[l] = b ? b[first + l] : nullptr;
    if (d->layer[first + l].relu) a.relu_mask |= 1 << l;
  }
  const K7Fn fn = pick(r, count);
  if (!fn) return hipErrorInvalidValue;
  a.H = d->h;
  a.W = d->w;
  a.strip_rows = g.strip_rows;
  a.nseg = g.nseg;
  a.nstrip = g.nstrip;
  a.ntiles = g.ntiles;
  a.step = g.step;
  a.lanes_off = g.lanes_off;
  return launch_kernel(fn, dim3(g.ntiles), dim3(kWave), 0, s, a);
}

}  // namespace is
