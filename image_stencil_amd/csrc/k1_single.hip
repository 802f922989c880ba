// k1_single.hip -- single-channel fp32 filtering (C = K = 1, NCHW), r, s in {1,3,5,7}.
//
// The "special case" kernel of "Optimizing Memory Efficiency for Convolution
// Kernels on Kepler GPUs" (arXiv 1705.10591), sections "thread layout" (3.1) and
// "memory access schedule" with its Algorithm 1, rebuilt for a CDNA wave64:
//  * a wave owns a strip of 256 columns x `strip_rows` rows (the page's H x W
//    image block; its best block was 256 wide) and sweeps it top to bottom, one
//    input row per step, so every input pixel is fetched from HBM once plus a
//    thin halo (the page's communication-optimal global reads);
//  * each lane keeps 4 contiguous columns, read and written as one 16-byte
//    access (the page's n pixels per thread, with n matched to the access width);
//  * horizontal sharing: the page stages each row in shared memory so that
//    neighbours can read each other's pixels. Inside one wave the same exchange
//    is a DPP wavefront shift of registers (no LDS traffic, no barrier); only
//    lanes 0 and 63 fetch the 16-byte halo outside the wave's 256 columns;
//  * vertical sharing stays in registers as on the page: a ring of r rolling
//    output rows, each input row adding its contribution to the r output rows
//    it touches; the oldest row is complete after its last filter row and is
//    stored, then recycled;
//  * the filter sits in scalar registers (wave-uniform operand of every FMA),
//    the analogue of the page's constant-memory broadcast;
//  * the next rows are prefetched U steps ahead into registers (the page's
//    prefetch that overlaps global loads with the FMAs);
//  * separable filters w[u][v] = col[u] * row[v] (SEP): each input row is
//    filtered once along the row (S FMAs per pixel) and that row result enters
//    the R rolling output rows with the column taps (R FMAs), R + S FMAs per
//    pixel instead of R * S;
//  * F filters on the one channel (the page's general case with a single input
//    channel): each input row, fetched once, feeds F rings of rolling output
//    rows, and every step stores one row of each of the F output planes. The
//    F * R * S taps stay in scalar registers, so F * R * S is kept <= 72.
#include "common.hpp"
#include "internal.hpp"

#include <limits.h>

namespace is {
namespace {

constexpr int kSegCols = 4 * kWave;   // 256 output columns per wave
// Cache policy. The output is written once: non-temporal stores. The image
// loads of a filter with halo columns (S > 1) keep their lines: those lines
// hold the halo columns that the waves of the neighbouring segments load soon
// after, and a non-temporal load lets L2 drop them first. Measured on
// 8192x8192, the five filter cases launched in turn in one process (two
// builds interleaved): FETCH_SIZE 276-278 MiB for the 256 MiB image with
// non-temporal loads and 258-275 MiB without; 3x3 101.5 -> 96.0 us, 5x5
// 110.7 -> 100.1, 7x7 124.1 -> 105.9, separable 7x7 113.8 -> 98.0. A 1x1
// filter has no halo: its loads stay non-temporal (97.3 against 99.6 us).
constexpr int kNonTemporal = 2;
template <int Q>
constexpr int load_policy() { return Q > 0 ? 0 : kNonTemporal; }

template <int R, int F>
struct Unroll {   // rows per unrolled step: a multiple of R (ring slots are static)
  // With F filters the F rings take the registers that a deeper prefetch
  // would use.
  static constexpr int value = R == 1 ? 4 : (R == 3 && F == 1 ? 6 : R);
};

struct Row4 {
  float v[4];
};

// Buffer resource of image row t when lo <= t < hi, else an empty one. Loads
// past num_records return 0 and stores past it are dropped, without a memory
// access: this gives the zero padding of columns >= W and of rows outside the
// image, and lets the row loop run without branches (rows outside the strip's
// range are read as zeros and their outputs discarded).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float *base, int t, int lo, int hi,
                                                           int W) {
  const bool in = t >= lo && t < hi;
  const float *p = base + (size_t)(in ? t : 0) * (size_t)W;   // select, no branch
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), (short)0, in ? W * 4 : 0,
                                           kBufferFlags);
}

// Load one input row into `m` (this lane's 4 columns) and `h` (Q halo
// columns: lane 0 gets the Q columns left of the segment, lane 63 the Q
// columns right of it, both in column order). Byte offsets are 32-bit;
// offsets outside the row (negative ones included, as unsigned values) read
// as 0. The halo loads fill exactly the Q registers they use: a wider load
// with dead destination registers lets the allocator reuse them while the load
// is in flight, and the wait that write then needs stalls on every load issued
// before it.
template <int Q>
struct Halo {
  float v[Q > 0 ? Q : 1];
};

template <bool VEC, int Q>
__device__ __forceinline__ void load_row(__amdgpu_buffer_rsrc_t rs, int off_m, int off_h, Row4 &m,
                                         Halo<Q> &h) {
  if constexpr (VEC) {
    const float4 a =
        __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off_m, 0, load_policy<Q>()));
    m.v[0] = a.x; m.v[1] = a.y; m.v[2] = a.z; m.v[3] = a.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m.v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off_m + 4 * i, 0, 0));
  }
  // One dword load per halo column: each is range-checked on its own (the
  // halo may straddle the row end when W is not a multiple of 4), and no
  // wider load leaves a dead destination register.
#pragma unroll
  for (int i = 0; i < Q; ++i)
    h.v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off_h + 4 * i, 0, load_policy<Q>()));
}

template <int R, int S, bool VEC, bool RELU, bool SEP, int F>
__global__ __launch_bounds__(kWave) void is_k1_single(const float *__restrict__ x,
                                                     const float *__restrict__ w,
                                                     const float *__restrict__ bias,
                                                     float *__restrict__ y, int H, int W,
                                                     int strip_rows, int nseg, int nstrip,
                                                     int ntiles) {
  constexpr int P = (R - 1) / 2, Q = (S - 1) / 2;
  constexpr int U = Unroll<R, F>::value;
  constexpr int NW = 4 + 2 * Q;   // window: 4 own columns plus Q each side

  const int lane = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, ntiles);
  const int seg = tile % nseg;
  const int strip = (tile / nseg) % nstrip;
  const int n = tile / (nseg * nstrip);
  const int x0 = seg * kSegCols;
  const int col = x0 + 4 * lane;
  const int y0 = strip * strip_rows;
  const int rows_out = min(strip_rows, H - y0);
  const int NT = rows_out + 2 * P;   // input rows y0-P .. y0+rows_out-1+P

  const size_t plane = (size_t)H * (size_t)W;
  const float *xp = x + (size_t)n * plane;
  float *yp = y + (size_t)n * F * plane;   // output plane f of image n at yp + f * plane

  // Byte offsets inside a row. Lanes other than 0 and 63 aim their halo load
  // past any row so that it reads nothing.
  const int off_m = 4 * col;
  const int off_h = lane == 0 ? 4 * (x0 - Q) : (lane == kWave - 1 ? 4 * (x0 + kSegCols) : INT_MIN);

  // Taps: F*R*S filter values (filter f's at f*R*S), or (SEP) R column taps
  // then S row taps.
  constexpr int NTAPS = SEP ? R + S : F * R * S;
  float wr[NTAPS];
#pragma unroll
  for (int i = 0; i < NTAPS; ++i) wr[i] = w[i];
  float bv[F];
#pragma unroll
  for (int f = 0; f < F; ++f) bv[f] = bias ? bias[f] : 0.f;

  // Input rows this strip needs: y0-P .. y0+rows_out-1+P, clipped to the image.
  const int in_hi = min(H, y0 + rows_out + P);

  // Prologue loads in row order (kept so by the scheduling barriers): the row
  // loop waits for its rows oldest first, and a reordered prologue would make
  // its first wait cover every load in flight.
  Row4 pf[U];
  Halo<Q> ph[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    load_row<VEC, Q>(row_rsrc(xp, y0 - P + i, 0, in_hi, W), off_m, off_h, pf[i], ph[i]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // acc[f][slot]: filter f's ring of the R output rows that the current input
  // row touches; output row o (relative ro = o - y0) lives in slot
  // (ro + 2P) mod R.
  float acc[F][R][4];
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int s = 0; s < R; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[f][s][i] = 0.f;

  // No branch inside the loop: the rounds past NT read zero rows and store
  // nothing (their rows are outside both buffer ranges), so the loads, the
  // stores and their waits form one straight sequence per U rows, and the
  // wait before each row covers that row's loads only, not the U-1 prefetched
  // after it.
  //
  // The first block of U rows and, when it is whole, the last one are
  // compiled separately so that they skip the products for output rows outside
  // the strip (rows above it in the first block, below it in the last), which
  // no store would keep: 2P rows' worth of FMAs at each end, 8.6% of the
  // 7x7 strip's work.
  auto block = [&](int rb, auto first_c, auto last_c) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
#pragma unroll
    for (int p = 0; p < U; ++p) {
      const int r = rb + p;
      const Row4 c = pf[p];
      const Halo<Q> h = ph[p];

      float win[NW];
#pragma unroll
      for (int i = 0; i < 4; ++i) win[Q + i] = c.v[i];
#pragma unroll
      for (int q = 1; q <= Q; ++q) {
        win[Q - q] = from_prev_lane(c.v[4 - q], h.v[Q - q]);
        win[Q + 3 + q] = from_next_lane(c.v[q - 1], h.v[q - 1]);
      }

      // SEP: the row pass of this input row, once for all R output rows.
      float hrow[4];
      if constexpr (SEP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hrow[i] = wr[R] * win[i];
#pragma unroll
          for (int v = 1; v < S; ++v) hrow[i] = __builtin_fmaf(wr[R + v], win[i + v], hrow[i]);
        }
      }

      // Input row r feeds relative output rows r-2P+j, j = 0..R-1, with
      // filter row R-1-j. j = R-1 is the first contribution to output row r:
      // it starts that slot with product + bias instead of clearing it.
#pragma unroll
      for (int j = 0; j < R; ++j) {
        // Output row r-2P+j: above the strip when FIRST and p + j < 2P, below
        // it when LAST (r = NT-U+p) and p + j >= U.
        if ((FIRST && p + j < 2 * P) || (LAST && p + j >= U)) continue;
        const int slot = (p + j) % R;
        const int u = R - 1 - j;
        if constexpr (SEP) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[0][slot][i] = j == R - 1 ? __builtin_fmaf(wr[u], hrow[i], bv[0])
                                         : __builtin_fmaf(wr[u], hrow[i], acc[0][slot][i]);
          continue;
        }
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
          for (int v = 0; v < S; ++v)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[f][slot][i] = (j == R - 1 && v == 0)
                                    ? __builtin_fmaf(wr[(f * R + u) * S + v], win[i + v], bv[f])
                                    : __builtin_fmaf(wr[(f * R + u) * S + v], win[i + v], acc[f][slot][i]);
      }

      // Output row r-2P (slot p mod R) is complete (the bias entered with its
      // first product); it is stored, in each of the F planes, only when it
      // lies inside the strip.
#pragma unroll
      for (int f = 0; f < F; ++f) {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] = acc[f][p % R][i];
          if constexpr (RELU) o[i] = fmaxf(o[i], 0.f);
        }
        const __amdgpu_buffer_rsrc_t rs_o = row_rsrc(yp + (size_t)f * plane, y0 + r - 2 * P, y0, y0 + rows_out, W);
        if constexpr (VEC) {
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int,
                                 make_float4(o[0], o[1], o[2], o[3])),
              rs_o, off_m, 0, kNonTemporal);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, o[i]), rs_o,
                                                  off_m + 4 * i, 0, 0);
        }
      }
      // Prefetch U rows ahead into the registers this row has just released
      // (the scheduling barrier keeps the load after the row's last FMA, so
      // that it can reuse them instead of holding U + 1 rows live).
      __builtin_amdgcn_sched_barrier(0);
      load_row<VEC, Q>(row_rsrc(xp, y0 - P + r + U, 0, in_hi, W), off_m, off_h, pf[p], ph[p]);
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  const int nb = (NT + U - 1) / U;
  const int rb_last = (nb - 1) * U;
  const bool last_whole = nb >= 2 && NT - rb_last == U;
  block(0, yes{}, no{});
  const int rb_end = last_whole ? rb_last : nb * U;
  for (int rb = U; rb < rb_end; rb += U) block(rb, no{}, no{});
  if (last_whole) block(rb_last, no{}, yes{});
}

using K1Fn = void (*)(const float *, const float *, const float *, float *, int, int, int, int, int,
                      int);

template <bool VEC, bool RELU>
K1Fn pick(int r, int s) {
#define IS_K1_CASE(RR, SS) \
  if (r == RR && s == SS) return is_k1_single<RR, SS, VEC, RELU, false, 1>;
#define IS_K1_ROW(RR) IS_K1_CASE(RR, 1) IS_K1_CASE(RR, 3) IS_K1_CASE(RR, 5) IS_K1_CASE(RR, 7)
  IS_K1_ROW(1) IS_K1_ROW(3) IS_K1_ROW(5) IS_K1_ROW(7)
#undef IS_K1_ROW
#undef IS_K1_CASE
  return nullptr;
}

// Separable filters, square sizes.
template <bool VEC, bool RELU>
K1Fn pick_sep(int r, int s) {
  if (r != s) return nullptr;
  if (r == 3) return is_k1_single<3, 3, VEC, RELU, true, 1>;
  if (r == 5) return is_k1_single<5, 5, VEC, RELU, true, 1>;
  if (r == 7) return is_k1_single<7, 7, VEC, RELU, true, 1>;
  return nullptr;
}

// F filters on one channel, square sizes with F * R * R <= 72 taps.
template <bool VEC, bool RELU>
K1Fn pick_fanout(int f, int r, int s) {
  if (r != s) return nullptr;
#define IS_K1_FAN(FF, RR) \
  if (f == FF && r == RR) return is_k1_single<RR, RR, VEC, RELU, false, FF>;
  IS_K1_FAN(2, 1) IS_K1_FAN(2, 3) IS_K1_FAN(2, 5)
  IS_K1_FAN(4, 1) IS_K1_FAN(4, 3)
  IS_K1_FAN(8, 1) IS_K1_FAN(8, 3)
#undef IS_K1_FAN
  return nullptr;
}

template <bool VEC, bool RELU>
K1Fn pick_any(const conv2d_desc &d) {
  if (d.k > 1) return d.separable ? nullptr : pick_fanout<VEC, RELU>(d.k, d.r, d.s);
  return d.separable ? pick_sep<VEC, RELU>(d.r, d.s) : pick<VEC, RELU>(d.r, d.s);
}

}  // namespace

bool configure_single(Plan &p, int param) {
  const conv2d_desc &d = p.d;
  if (d.c != 1 || d.layout != IS_NCHW || d.in_dtype != IS_F32) return false;
  if (d.r > 7 || d.s > 7) return false;
  // Byte offsets inside a row are 32-bit: the row range 4 W and the halo
  // offset 4 (x0 + 256) of the last segment must stay below 2^31.
  if (4.0 * ((double)d.w + kSegCols) >= 2147483648.0) return false;
  if (pick_any<true, false>(d) == nullptr) return false;
  const int nseg = (d.w + kSegCols - 1) / kSegCols;
  // Strip height: a wave keeps about one prefetch window of rows in flight, so
  // the bytes in flight per CU grow with the number of resident waves. 64 rows
  // give 4096 waves (16 per CU) on an 8192x8192 image. Each strip also reads
  // the 2P halo rows it shares with its neighbours, which L2 seldom still holds
  // (the neighbour reads them at the other end of its sweep): FETCH_SIZE reads
  // 266-280 MiB for the 256 MiB image (3x3 .. 7x7). Sweeping odd strips upward,
  // so that both reads of a halo row coincide, brought that to 258-260 MiB but
  // was 2-3% slower on the 3x3 and 5x5 (builds interleaved in one process).
  // 16-row strips made the 3x3 and 5x5 3-5% faster but the 7x7 launched after
  // them 20% slower at the same shader clock; 128 rows were 7-15% slower, and
  // heights that are not powers of two (22 .. 66 rows) 2-10% slower than the
  // neighbouring powers of two.
  int rows = 64;
  while (rows > 8 && (long long)nseg * ((d.h + rows - 1) / rows) * d.n < 4096) rows >>= 1;
  if (d.k > 1) {
    // F filters: 64-row strips (1024 waves on a 4096x4096 image; 32 rows
    // measured 1-5% slower, 16 and 128 rows 5-30% slower). Measured against
    // the multi-channel kernel (LDS-staged tile, the F planes' stores spread
    // over a workgroup's waves, streaming stores) on 4096x4096: this one is
    // faster only with two 5x5 filters (40 against 52 us); it ties with two
    // 3x3 filters and is 14-42% slower with two 1x1 or four filters, and
    // slower with eight and on small images, which give it too few waves.
    // So the plan takes it for two 5x5 filters on large images; every other
    // one-channel shape it can run lists it among the tuning variants.
    rows = 64;
    if (param == 0 && (d.k != 2 || d.r != 5 || (long long)nseg * ((d.h + rows - 1) / rows) * d.n < 1024))
      return false;
  }
  if (param != 0) {   // a tuning variant: 4 to 256 rows
    if (param < 4 || param > 256) return false;
    rows = param;
  }
  const int nstrip = (d.h + rows - 1) / rows;
  p.kid = kSingleChannel;
  p.name = d.separable ? "is_k1_single_separable" : (d.k > 1 ? "is_k1_single_fanout" : "is_k1_single");
  p.nseg = nseg;
  p.nstrip = nstrip;
  p.strip_rows = rows;
  p.ntiles = nseg * nstrip * d.n;
  p.grid_x = p.ntiles;
  p.grid_y = 1;
  p.grid_z = 1;
  p.block = kWave;
  p.lds = 0;
  p.tile_w = kSegCols;
  p.tile_h = rows;
  p.vec = (d.w % 4 == 0) ? 1 : 0;
  return true;
}

hipError_t launch_single(const Plan &p, const float *x, const float *w, const float *b, float *y,
                         hipStream_t s) {
  const bool relu = p.d.relu != 0;
  const K1Fn fn = p.vec ? (relu ? pick_any<true, true>(p.d) : pick_any<true, false>(p.d))
                        : (relu ? pick_any<false, true>(p.d) : pick_any<false, false>(p.d));
  if (!fn) return hipErrorInvalidValue;
  return launch_kernel(fn, dim3(p.grid_x), dim3(p.block), 0, s, x, w, b, y, p.d.h, p.d.w,
                     p.strip_rows, p.nseg, p.nstrip, p.ntiles);
}

}  // namespace is
