// k5_mfma_f32.hip -- fp32 NCHW 3x3 layer with 32 input and 32 output channels
// as an implicit GEMM on the gfx950 fp32 matrix cores, with bias and ReLU.
//
// The layer y[o][p] = b[o] + sum_k W[o][k] X[k][p] over k = (tap t = 3u + v,
// channel c) is a dense contraction of length 9 * 32 = 288 (the "blocked GEMM"
// view of a convolution that "Optimizing Memory Efficiency for Convolution
// Kernels on Kepler GPUs" sets against its direct method). At 32 channels the
// direct fp32 kernel is bound by the vector ALUs; v_mfma_f32_16x16x4_f32 does
// the same fp32 products and sums at twice that ceiling (157.3 vs 78.6 TFLOP/s
// without packed FP32). Design:
//  * persistent workgroups of 8 waves (2 per SIMD), one per CU, looping over
//    13 x 32 pixel tiles (2240 on a 1280x720 frame: 9 rounds of 256 CUs, the last 75% full;
//    12-row tiles needed 10 rounds, 120 rows per CU against 117); tiles of one
//    XCD are neighbours so halo re-reads hit its L2;
//  * the input tile with its halo (32 channels x 15 rows x 40 columns, aligned
//    16-byte chunks) streams HBM -> LDS by 16-byte buffer_load ... lds,
//    double-buffered against the MFMAs; pixels outside the image read as 0
//    through the range check;
//  * LDS keeps the NCHW order; the channel-plane pitch of 624 floats (600 used)
//    is an odd multiple of 16 banks: the 16 lanes of one channel read 16
//    consecutive floats, and the 4 channels of a read sit 16 banks apart; the
//    two tile buffers fill the 160 KB of LDS;
//  * wave w computes output channels 16*(w&1) .. +16 for columns
//    16*((w>>1)&1) .. +16 of tile rows 0..6 (w < 4) or 7..12 (w >= 4); its 72
//    weight fragments (all 288 k) stay in registers. Two waves per SIMD hide
//    each other's operand-read and epilogue stalls: with 4 waves (one per SIMD,
//    each taking all 13 rows) the layer took 149.8 us against 142.6 us with 8
//    (interleaved in one process, the same results bit for bit); the two row
//    halves read 17 input rows per tile instead of 15;
//  * MFMA operands: A = 16 pixels x 4 channels of one tap (one LDS float per
//    lane), B = 4 channels x 16 output channels (weights), D = 4 consecutive
//    pixels of one output channel per lane, stored as one 16-byte NCHW vector;
//  * rolling rows: the A fragment of input row i (tap column v, channel quad)
//    is read once and feeds output rows i, i-1 and i-2 through filter rows 0, 1
//    and 2; an output row is final after input row +2 and is stored from the
//    accumulators inside the loop (bias, optional ReLU).
#include "common.hpp"
#include "internal.hpp"

namespace is {
namespace {

typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

constexpr int kC = 32;                        // input channels
constexpr int kK = 32;                        // output channels
constexpr int kTR = 13, kTC = 32;             // output tile: rows x columns
constexpr int kIR = kTR + 2;                  // input rows with halo
// An input row is loaded as 10 aligned 16-byte chunks, image columns x0-4 ..
// x0+35, of which x0-1 .. x0+32 are used (LDS column 3 holds x0-1).
constexpr int kChunksRow = 10;
constexpr int kIC = 4 * kChunksRow;           // LDS floats per input row
constexpr int kPlaneChunks = 156;             // 16-byte slots per channel plane, 150 used
constexpr int kPlane = 4 * kPlaneChunks;      // LDS floats per channel plane (624)
constexpr int kChunks = kC * kPlaneChunks;    // 16-byte slots per input tile, padding included
constexpr int kWaves = 8;                     // 2 per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kRounds = (kChunks + kThreads - 1) / kThreads;   // 16-byte DMA rounds per thread and tile
constexpr int kBufFloats = kRounds * kThreads * 4;   // floats per LDS tile buffer (whole rounds)
constexpr int kCQ = kC / 4;                   // channel quads (k steps per tap)
constexpr int kKS = 9 * kCQ;                  // k steps of 4
// Output rows of a wave: waves 0-3 take tile rows 0..6 and waves 4-7 rows
// 7..12 of the same columns and channels.
template <int RH>
struct Rows {
  static constexpr int O0 = RH ? 7 : 0;
  static constexpr int O1 = RH ? kTR : 7;
};
constexpr unsigned kOob = 0xFFFFFFF0u;
static_assert(kPlane % 32 == 16, "plane pitch: 16 banks apart");
static_assert(kIR * kChunksRow <= kPlaneChunks, "the tile rows fit the plane");
static_assert(kC * kPlane <= kBufFloats, "the tile fits its buffer");

struct MfmaF32Args {
  const float *x;
  const float *w;
  const float *bias;
  float *y;
  int N, H, W, relu;
  int tiles_x, tiles_y, ntiles;
};

__global__ __launch_bounds__(kThreads, 1) void is_k5_mfma_f32(MfmaF32Args a) {
  __shared__ float lds[2 * kBufFloats];
  lds_poison(lds, sizeof(lds));

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;   // pixel of A, output channel of B and D
  const int g = lane >> 4;     // channel of A and B inside a quad; pixel group of D
  const int ob = wave & 1;     // output channels 16*ob .. +16
  const int ch = (wave >> 1) & 1;   // tile columns 16*ch .. +16
  const int rh = wave >> 2;    // row half (8 waves)

  // ---- Tile schedule: XCD x (= blockIdx mod 8) walks its own contiguous range.
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int per_xcd = (a.ntiles + 7) / 8;
  const int lo = xcd * per_xcd;
  const int hi = min(a.ntiles, lo + per_xcd);
  const int step = G >> 3;
  int tile = lo + (blockIdx.x >> 3);

  const int H = a.H, W = a.W;
  const size_t plane = (size_t)H * W;
  auto tile_origin = [&](int tl, int &n, int &y0, int &x0) {
    const int tx = tl % a.tiles_x;
    const int ty = (tl / a.tiles_x) % a.tiles_y;
    n = tl / (a.tiles_x * a.tiles_y);
    y0 = ty * kTR;
    x0 = tx * kTC;
  };
  // LDS chunk s of a buffer holds channel s / kPlaneChunks, tile row
  // r / kChunksRow and chunk r % kChunksRow of r = s % kPlaneChunks (image row
  // y0-1+row, columns x0-4+4*chunk .. +4); chunks outside the image are loaded
  // as 0 (W is a multiple of 4, so a chunk is wholly in or out), and so are the
  // plane padding and the chunks of the last round past the tile. One DMA
  // round j moves chunks (4j + wave) * 64 + lane.
  struct Dma {
    __amdgpu_buffer_rsrc_t rx;
    int y0, x0;
    bool any;   // false: no tile to load, every round reads nothing
  };
  auto dma_for = [&](int tl) -> Dma {
    Dma d;
    int n;
    d.any = tl < hi;
    tile_origin(d.any ? tl : 0, n, d.y0, d.x0);
    d.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.x + (size_t)n * kC * plane), (short)0,
                                             (int)(kC * plane * 4), kBufferFlags);
    return d;
  };
  // Branch-free and in 32-bit arithmetic (the plan keeps an image's input under
  // 2 GB): the rounds sit between the MFMAs, where a divergent branch would
  // break the instruction stream.
  const int plane_i = H * W;
  auto issue_round = [&](const Dma &d, float *buf, int j) {
    const unsigned s = (unsigned)((j * kWaves + wave) * 64 + lane);
    const unsigned c = s / kPlaneChunks;
    const unsigned r = s - c * kPlaneChunks;
    const unsigned row = r / kChunksRow;
    const unsigned k = r - row * kChunksRow;
    const int gy = d.y0 - 1 + (int)row, gx = d.x0 - 4 + 4 * (int)k;
    const bool in = d.any & (s < (unsigned)kChunks) & (row < (unsigned)kIR) & ((unsigned)gy < (unsigned)H) &
                    ((unsigned)gx < (unsigned)W);
    const unsigned off = in ? (unsigned)((int)c * plane_i + gy * W + gx) * 4u : kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        d.rx, (__attribute__((address_space(3))) void *)(buf + (j * kWaves + wave) * 64 * 4), 16, off, 0, 0, 0);
  };

  // ---- Weights: coalesced 16-byte loads of the KCRS tensor, then the first
  // tile's DMA, then the weights through the second tile buffer (rows of 292
  // floats) while that DMA is in flight. Fragment (t, cq) of this lane is
  // W[16ob + n16][4cq + g][t].
  float wb[kKS];
  float bv;
  {
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.w), (short)0, kK * kC * 9 * 4, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.bias), (short)0, a.bias ? kK * 4 : 0, kBufferFlags);
    constexpr int kVecRow = kC * 9 / 4;        // 72 vectors per output channel
    constexpr int kVecs = kK * kVecRow;
    constexpr int kVecPerThread = (kVecs + kThreads - 1) / kThreads;
    constexpr int kWPitch = kC * 9 + 4;        // 16-byte aligned rows
    static_assert(kK * kWPitch <= kBufFloats, "the weights fit one tile buffer");
    uint4v t[kVecPerThread];
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j)
      t[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, (j * kThreads + tid) * 16, 0, 0);   // past the end: 0
    {
      const Dma d0 = dma_for(tile);
#pragma unroll
      for (int j = 0; j < kRounds; ++j) issue_round(d0, lds, j);
    }
    // The bias after the DMA: it is first used after the wait for that DMA.
    bv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (16 * ob + n16) * 4, 0, 0));
    float *wl = lds + kBufFloats;
    // Whole 16-byte vectors: this compiler narrows a 16-byte buffer load whose
    // elements are taken apart one by one to a single dword.
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j) {
      const int v = j * kThreads + tid;
      const int o = v / kVecRow, r = v - o * kVecRow;
      if (kVecs % kThreads == 0 || v < kVecs) *reinterpret_cast<uint4v *>(wl + o * kWPitch + 4 * r) = t[j];
    }
    lds_barrier();
    const float *wp = wl + (16 * ob + n16) * kWPitch + g * 9;
#pragma unroll
    for (int tp = 0; tp < 9; ++tp)
#pragma unroll
      for (int cq = 0; cq < kCQ; ++cq) wb[tp * kCQ + cq] = wp[cq * 4 * 9 + tp];
    lds_barrier();   // the second buffer takes the next tile's DMA from here on
  }

  // Float offset (inside a buffer) of this lane's A reads for tap column v at
  // tile row 0: channel g of the quad, image column x0 - 1 + 16*ch + n16 + v
  // (LDS column 3 holds x0 - 1).
  const int aoff = g * kPlane + 3 + 16 * ch + n16;

  // The next tile's DMA rounds are spread over the first 3/5 of the MFMA
  // loop, between the reads: spread to the very end, the last round's latency
  // would be exposed at every tile boundary.
  auto compute_store = [&](auto rh_c, int tl, const float *buf, const Dma &dn, float *nbuf) {
    using RW = Rows<decltype(rh_c)::value>;
    constexpr int O0 = RW::O0, O1 = RW::O1;
    constexpr int kReads = (O1 + 2 - O0) * 3 * kCQ;
    constexpr int kIssue = kReads * 3 / 5;
    int n, y0, x0;
    tile_origin(tl, n, y0, x0);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        a.y + (size_t)n * kK * plane, (short)0, (int)(kK * plane * 4), kBufferFlags);
    const int gx = x0 + 16 * ch + 4 * g;
    const bool col_in = gx < W;
    const unsigned col_off = (unsigned)(((size_t)(16 * ob + n16) * plane + gx) * 4);
    float4v acc[O1 - O0];
#pragma unroll
    for (int o = 0; o < O1 - O0; ++o) acc[o] = float4v{0.f, 0.f, 0.f, 0.f};
    constexpr int kAhead = 16;
    auto read_a = [&](int q) -> float {
      const int i = O0 + q / (3 * kCQ), v = (q / kCQ) % 3, cq = q % kCQ;
      return buf[aoff + cq * 4 * kPlane + i * kIC + v];
    };
    float ring[kAhead];
#pragma unroll
    for (int q = 0; q < kAhead; ++q) ring[q] = read_a(q);
    static_for<kReads>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      constexpr int j0 = q < kIssue ? (q * kRounds + kIssue - 1) / kIssue : kRounds;
      constexpr int j1 = q < kIssue ? ((q + 1) * kRounds + kIssue - 1) / kIssue : kRounds;
      if constexpr (j1 > j0) {
#pragma unroll
        for (int j = j0; j < j1; ++j) issue_round(dn, nbuf, j);
        __builtin_amdgcn_sched_barrier(0);
      }
      const float av = ring[q % kAhead];
      if constexpr (q + kAhead < kReads) ring[q % kAhead] = read_a(q + kAhead);
      constexpr int i = O0 + q / (3 * kCQ), v = (q / kCQ) % 3, cq = q % kCQ;
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int o = i - u;
        if (o >= O0 && o < O1)
          acc[o - O0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, wb[(3 * u + v) * kCQ + cq], acc[o - O0], 0, 0, 0);
      }
      if constexpr (v == 2 && cq == kCQ - 1 && i - 2 >= O0 && i - 2 < O1) {
        constexpr int o = i - 2;
        const int gy = y0 + o;
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r[e] = acc[o - O0][e] + bv;
          if (a.relu) r[e] = fmaxf(r[e], 0.f);
        }
        const unsigned off = ((gy < H) & col_in) ? col_off + (unsigned)gy * (unsigned)W * 4u : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4v, float4v{r[0], r[1], r[2], r[3]}),
                                               ry, off, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // Wait for the next tile's DMA but not for the output stores issued after
    // its last round: vector-memory operations retire in issue order on gfx9.
    constexpr int q_last = ((kRounds - 1) * kIssue) / kRounds;
    constexpr int stores = [] {
      int c = 0;
      for (int o = O0; o < O1; ++o)
        if ((o + 2 - O0) * 3 * kCQ + 3 * kCQ - 1 >= q_last) ++c;
      return c;
    }();
    static_assert(stores < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((stores & 0xF) | ((stores >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  };

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int cur = 0;
  while (tile < hi) {
    const int next = tile + step;
    if (rh == 0)
      compute_store(std::integral_constant<int, 0>{}, tile, lds + cur * kBufFloats, dma_for(next),
                    lds + (cur ^ 1) * kBufFloats);
    else
      compute_store(std::integral_constant<int, 1>{}, tile, lds + cur * kBufFloats, dma_for(next),
                    lds + (cur ^ 1) * kBufFloats);
    __syncthreads();
    tile = next;
    cur ^= 1;
  }
}

}  // namespace

bool configure_mfma_f32(Plan &p) {
  const conv2d_desc &d = p.d;
  if (d.layout != IS_NCHW || d.in_dtype != IS_F32 || d.out_dtype != IS_F32) return false;
  if (d.c != kC || d.k != kK || d.r != 3 || d.s != 3) return false;
  if (d.w % 4 != 0) return false;   // 16-byte output vectors
  // 32-bit buffer offsets inside one image of the input and of the output.
  if (4.0 * kC * (double)d.h * d.w >= 2.0e9) return false;
  const long long tiles = (long long)((d.w + kTC - 1) / kTC) * ((d.h + kTR - 1) / kTR) * d.n;
  if (tiles > (1LL << 31) - 1) return false;
  p.kid = kMfmaNchwF32;
  p.name = "is_k5_mfma_f32";
  p.nseg = (d.w + kTC - 1) / kTC;
  p.nstrip = (d.h + kTR - 1) / kTR;
  p.ntiles = (int)tiles;
  // Persistent: one workgroup per CU (its LDS fills the CU); fewer when there
  // are fewer tiles.
  p.grid_x = persistent_grid(p.ntiles, 256);
  p.grid_y = p.grid_z = 1;
  p.block = kThreads;
  p.lds = 2 * kBufFloats * 4;
  p.tile_w = kTC;
  p.tile_h = kTR;
  return true;
}

hipError_t launch_mfma_f32(const Plan &p, const float *x, const float *w, const float *b, float *y,
                           hipStream_t s) {
  MfmaF32Args a;
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
  return launch_kernel(is_k5_mfma_f32, dim3(persistent_grid(p.ntiles, device_cu_count())), dim3(p.block), 0,
                       s, a);
}

}  // namespace is
