// k4_mfma.hip -- fp16 NHWC 3x3 layer with 64 input and 64 output channels as an
// implicit GEMM on the gfx950 matrix cores, fp32 accumulation, fp16 output.
//
// For output pixel p and output channel o the layer is
//   y[p][o] = b[o] + sum_k W[o][k] * X[k][p],  k = (tap t = 3u + v, channel c),
// a dense contraction of length 9 * 64 = 576 (the "blocked GEMM" view of a
// convolution that "Optimizing Memory Efficiency for Convolution Kernels on
// Kepler GPUs" contrasts with its direct method; here the wide-channel layer
// really is that contraction, so it runs on MFMA). Design:
//  * persistent workgroups, one per CU; each loops over 16 x 32 pixel
//    tiles of an image, tiles of one XCD being neighbours so halo re-reads hit
//    that XCD's L2;
//  * the input tile with its 1-pixel halo (18 x 34 pixels x 128 bytes) streams
//    HBM -> LDS by buffer_load ... lds, double-buffered against the MFMAs;
//    pixels outside the image read as 0 through the buffer range check;
//  * LDS holds each pixel's 64 channels as eight 16-byte chunks, permuted by the
//    XOR swizzle of "CUDA shared memory swizzling" (its formula, with 16-byte
//    elements and chunks) over rows of SWZ bytes, so that 16 lanes reading the
//    same chunk of 16 consecutive pixels hit distinct banks;
//  * 8 waves, 2 per SIMD: wave w owns the 16 output channels 16*(w%4) .. +16
//    (one A block) for the 16 columns 16*(w/4) .. +16 of all 16 tile rows; its
//    18 weight fragments (all 576 k) stay in registers. Two waves per SIMD
//    let one wave's MFMAs run while the other waits for its LDS reads (a
//    build with 2 A blocks per wave and 4 waves is kept behind OB_PER_WAVE);
//  * v_mfma_f32_16x16x32_f16: A = 16 output channels x 32 k (weights), B = 32 k
//    x 16 pixels (one 16-byte LDS read per lane), D = 4 consecutive output
//    channels of one pixel per lane;
//  * rolling rows, as in the single-channel kernel: the B fragment of input
//    row i (tap column v, channel half h) is read once and feeds the output rows
//    i, i-1 and i-2 through filter rows 0, 1 and 2, so a wave reads 18 x 6
//    fragments per tile instead of 16 x 18;
//  * an output row is final once input row +2 has been read: it gets the fp32
//    bias, the optional ReLU and fp16 rounding (nearest even) and is stored
//    from the accumulators inside the MFMA loop, so stores overlap the matrix
//    work and the tile needs no epilogue phase.
#include "common.hpp"
#include "internal.hpp"

#include <stdlib.h>

#ifndef OB_PER_WAVE
#define OB_PER_WAVE 1
#endif

namespace is {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));

constexpr int kC = 64;                       // input channels
constexpr int kK = 64;                       // output channels
constexpr int kTR = 16, kTC = 32;            // output tile: rows x columns
constexpr int kIR = kTR + 2, kIC = kTC + 2;  // input tile with halo
constexpr int kChunks = kIR * kIC * 8;       // 16-byte chunks per input tile
// Output-channel blocks of 16 per wave. With 1, each wave holds 16 output
// channels (72 weight VGPRs, 64 accumulators) and the workgroup has 8 waves,
// 2 per SIMD, so one wave's MFMAs run while the other waits for its LDS reads;
// with 2, a B read feeds twice the MFMAs but each SIMD has a single wave.
constexpr int kOB = OB_PER_WAVE;
constexpr int kGroups = kK / (16 * kOB);     // output-channel groups
constexpr int kWaves = kGroups * 2;          // x 2 tile-column halves
constexpr int kThreads = 64 * kWaves;
constexpr int kRounds = (kChunks + kThreads - 1) / kThreads;   // DMA rounds per thread
constexpr int kBufChunks = kRounds * kThreads;                 // chunks per LDS buffer
constexpr unsigned kOob = 0xFFFFFFF0u;
constexpr int kPB = kTR;                     // 16-pixel blocks per wave: one per tile row
constexpr int kReadSteps = (kTR + 2) * 6;    // B reads per wave and tile
// The next tile's DMA rounds are issued during the first kIssueSteps read
// steps; output stores issued after the last round: output row o is stored
// (two 8-byte stores) at read step 6 * (o + 2) + 5.
constexpr int kIssueSteps = kReadSteps * 3 / 5;
constexpr int stores_after_last_round() {
  const int q_last = ((kRounds - 1) * kIssueSteps) / kRounds;
  int n = 0;
  for (int o = 0; o < kTR; ++o)
    if (6 * (o + 2) + 5 >= q_last) n += kOB;
  return n;
}
constexpr int kStores = stores_after_last_round();
// s_waitcnt immediate (gfx9 encoding): vmcnt <= kStores (bits 3:0 and 15:14),
// expcnt and lgkmcnt not waited for (all ones).
constexpr int kWaitDmaNotStores = (kStores & 0xF) | ((kStores >> 4) << 14) | (0x7 << 4) | (0xF << 8);
static_assert(kStores < 64, "vmcnt field");

static_assert(kK * (kC * 9 * 2 + 16) <= 2 * kBufChunks * 16, "weights are staged in the tile buffers");

constexpr int kRowSlots = kIC * 8;           // 16-byte slots per input tile row

// Slot of chunk c (0..7) of column cx inside one input-tile row. Each tile row
// is its own swizzled array: rows of SWZ bytes (one pixel for 128, a pixel pair
// for 256) whose 16-byte chunks are permuted by XOR with the row index, the
// formula of "CUDA shared memory swizzling" with 16-byte elements and chunks.
// SWZ = 0 keeps the plain layout. Row-local keys keep the permutation the same
// in every tile row, so a row step is a constant offset.
template <int SWZ>
__device__ __forceinline__ int slot_in_row(int cx, int c) {
  if constexpr (SWZ == 0) {
    return cx * 8 + c;
  } else {
    constexpr int NX = SWZ / 16;           // chunks per swizzle row
    constexpr int PPR = NX / 8;            // pixels per swizzle row
    const int y = cx / PPR;
    const int x = (cx % PPR) * 8 + c;
    return y * NX + swizzle_col(y, x, NX, 16, 16);
  }
}

// Inverse: column and chunk stored at slot si of a tile row. The XOR swizzle is
// an involution inside each swizzle row, so the same map undoes it.
template <int SWZ>
__device__ __forceinline__ void chunk_at(int si, int &cx, int &c) {
  if constexpr (SWZ == 0) {
    cx = si >> 3;
    c = si & 7;
  } else {
    constexpr int NX = SWZ / 16;
    constexpr int PPR = NX / 8;
    const int y = si / NX;
    const int x = swizzle_col(y, si % NX, NX, 16, 16);
    cx = y * PPR + x / 8;
    c = x % 8;
  }
}

struct MfmaArgs {
  const _Float16 *x;
  const _Float16 *w;
  const float *bias;
  _Float16 *y;
  int N, H, W, relu;
  int tiles_x, tiles_y, ntiles;
};

// The DMA source of one tile: the image's buffer resource and the tile origin.
struct TileDma {
  __amdgpu_buffer_rsrc_t rx;
  int y0, x0;
  bool any;   // false: no tile to load, every round reads nothing
};

template <int SWZ>
__global__ __launch_bounds__(kThreads, 1) void is_k4_mfma(MfmaArgs a) {
  __shared__ uint4v lds[2 * kBufChunks];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;     // pixel (B, D) or output channel (A) inside a 16-block
  const int g = lane >> 4;       // k group of 8 (A, B) or channel group of 4 (D)
  const int og = wave % kGroups;  // output channels 16*kOB*og .. +16*kOB
  const int ch = wave / kGroups;  // tile-column half: columns 16*ch .. 16*ch+15

  // ---- Weights: copy the KCRS tensor into LDS with 16-byte loads, each output
  // channel's 576 halves on a row of 1168 bytes (16 bytes of padding spread
  // the 16 channels a fragment read touches over distinct banks); then every
  // lane gathers its 36 A fragments (2 channel blocks x 18 k steps): fragment
  // (ob, ks) holds channels 32h + 8g .. +8 of tap t = ks/2 for output channel
  // 16*(kOB*og + ob) + n16, i.e. 8 halves 9 apart in the channel's row.
  constexpr int kWRow = kC * 9 * 2 + 16;   // bytes per padded weight row
  {
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16 *>(a.w), (short)0, kK * kC * 9 * 2, kBufferFlags);
    constexpr int kVecRow = kC * 9 * 2 / 16;   // 72 vectors per output channel
    constexpr int kVecPerThread = kK * kVecRow / kThreads;
    static_assert(kVecPerThread * kThreads == kK * kVecRow, "whole vectors per thread");
    // All loads first, then the LDS writes: a load-write loop would wait for
    // each load in turn, 18 round trips to L2 before the first tile.
    uint4v t[kVecPerThread];
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j)
      t[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, (j * kThreads + tid) * 16, 0, 0);
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j) {
      const int v = j * kThreads + tid;
      const int o = v / kVecRow, r = v - o * kVecRow;
      *reinterpret_cast<uint4v *>(reinterpret_cast<char *>(lds) + o * kWRow + r * 16) = t[j];
    }
  }
  __syncthreads();
  half8 wa[kOB][18];
  {
    const char *wl = reinterpret_cast<const char *>(lds);
#pragma unroll
    for (int ob = 0; ob < kOB; ++ob)
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const int o = 16 * (kOB * og + ob) + n16;
        const int t = ks >> 1, h = ks & 1;
        const _Float16 *src =
            reinterpret_cast<const _Float16 *>(wl + o * kWRow) + (32 * h + 8 * g) * 9 + t;
#pragma unroll
        for (int j = 0; j < 8; ++j) wa[ob][ks][j] = src[9 * j];
      }
  }
  float bias[kOB][4];
#pragma unroll
  for (int ob = 0; ob < kOB; ++ob)
#pragma unroll
    for (int i = 0; i < 4; ++i) bias[ob][i] = a.bias ? a.bias[16 * (kOB * og + ob) + 4 * g + i] : 0.f;
  __syncthreads();

  // ---- Tile schedule: XCD x (= blockIdx mod 8) walks its own contiguous range.
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int per_xcd = (a.ntiles + 7) / 8;
  const int lo = xcd * per_xcd;
  const int hi = min(a.ntiles, lo + per_xcd);
  const int step = G >> 3;
  int tile = lo + (blockIdx.x >> 3);

  const size_t img = (size_t)a.H * a.W * kC;   // halves per image
  auto tile_origin = [&](int tl, int &n, int &y0, int &x0) {
    const int tx = tl % a.tiles_x;
    const int ty = (tl / a.tiles_x) % a.tiles_y;
    n = tl / (a.tiles_x * a.tiles_y);
    y0 = ty * kTR;
    x0 = tx * kTC;
  };
  // DMA of one tile, in rounds: round j moves LDS slots (4j + wave) * 64 + lane
  // of a buffer. Offsets are branch-free 32-bit arithmetic (the plan keeps an
  // image under 4 GB): the rounds of the next tile sit between the MFMAs,
  // where a divergent branch would break the instruction stream.
  auto dma_for = [&](int tl) -> TileDma {
    TileDma d;
    int n;
    d.any = tl < hi;
    tile_origin(d.any ? tl : 0, n, d.y0, d.x0);
    d.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16 *>(a.x + (size_t)n * img), (short)0,
                                             (int)(img * 2), kBufferFlags);
    return d;
  };
  auto issue_round = [&](const TileDma &d, uint4v *buf, int j) {
    const unsigned s = (unsigned)((j * kWaves + wave) * 64 + lane);
    const unsigned ry = s / kRowSlots;
    int cx, c;
    chunk_at<SWZ>((int)(s - ry * kRowSlots), cx, c);
    const int gy = d.y0 - 1 + (int)ry;
    const int gx = d.x0 - 1 + cx;
    const bool in = d.any & (s < (unsigned)kChunks) & ((unsigned)gy < (unsigned)a.H) & ((unsigned)gx < (unsigned)a.W);
    const unsigned off = in ? (unsigned)(((gy * a.W + gx) * kC + c * 8) * 2) : kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        d.rx, (__attribute__((address_space(3))) void *)(buf + (j * kWaves + wave) * 64), 16, off, 0, 0, 0);
  };

  // Byte offsets (inside a tile buffer) of this lane's B reads for filter column
  // v and channel half h at input-tile row 0; row i adds i tile rows.
  int boff[3][2];
#pragma unroll
  for (int v = 0; v < 3; ++v)
#pragma unroll
    for (int h = 0; h < 2; ++h) boff[v][h] = slot_in_row<SWZ>(16 * ch + n16 + v, 4 * h + g) * 16;

  // The next tile's DMA rounds are issued between the reads of the first 3/5
  // of the MFMA loop (round j at read step j * kIssueSteps / kRounds): issued
  // in a burst before the loop they delay its first MFMAs, and spread to the
  // very end the last round's latency is exposed at the tile boundary.
  auto compute_store = [&](int tl, const uint4v *buf, const TileDma &dn, uint4v *nbuf) {
    int n, y0, x0;
    tile_origin(tl, n, y0, x0);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        a.y + (size_t)n * img, (short)0, (int)(img * 2), kBufferFlags);
    // Byte offset of this lane's 4 output channels in its output column (32-bit
    // offsets: the plan keeps an image under 4 GB), or an out-of-range offset
    // when the column is outside the image; row gy adds gy * W * 128 bytes.
    const int gx = x0 + 16 * ch + n16;
    const bool col_in = gx < a.W;
    const unsigned col_off = (unsigned)(gx * kK + 16 * kOB * og + 4 * g) * 2u;
    const unsigned row_bytes = (unsigned)a.W * kK * 2u;
    float4v acc[kPB][kOB];
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb)
#pragma unroll
      for (int ob = 0; ob < kOB; ++ob) acc[pb][ob] = float4v{0.f, 0.f, 0.f, 0.f};
    // Reads go in (input row i, tap column v, channel half h) order; read i
    // feeds output rows i - u, u = 0..2 (those inside the tile), with the A
    // fragment of k step 2(3u + v) + h, for both output-channel blocks. Each read
    // is issued kAhead reads early into a ring of registers; scheduling
    // barriers between reads keep the compiler from hoisting more reads than
    // the ring holds.
    constexpr int kReads = kReadSteps;
    constexpr int kAhead = 8;
    auto read_b = [&](int q) -> half8 {
      const int i = q / 6, v = (q % 6) >> 1, h = q & 1;
      const char *p = reinterpret_cast<const char *>(buf) + boff[v][h] + i * kRowSlots * 16;
      return *reinterpret_cast<const half8 *>(p);
    };
    half8 ring[kAhead];
#pragma unroll
    for (int q = 0; q < kAhead; ++q) ring[q] = read_b(q);
    static_for<kReads>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      // rounds issued at this step: j with j * kIssueSteps / kRounds == q
      constexpr int j0 = q < kIssueSteps ? (q * kRounds + kIssueSteps - 1) / kIssueSteps : kRounds;
      constexpr int j1 = q < kIssueSteps ? ((q + 1) * kRounds + kIssueSteps - 1) / kIssueSteps : kRounds;
      if constexpr (j1 > j0) {
#pragma unroll
        for (int j = j0; j < j1; ++j) issue_round(dn, nbuf, j);
        // keeps the rounds ahead of this step's stores (the tile-end wait
        // counts the stores issued after the last round)
        __builtin_amdgcn_sched_barrier(0);
      }
      const half8 b = ring[q % kAhead];
      if constexpr (q + kAhead < kReads) ring[q % kAhead] = read_b(q + kAhead);
      constexpr int i = q / 6, v = (q % 6) >> 1, h = q & 1;
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int o = i - u;
        if (o >= 0 && o < kTR) {
          const int ks = 2 * (3 * u + v) + h;
#pragma unroll
          for (int ob = 0; ob < kOB; ++ob)
            acc[o][ob] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[ob][ks], b, acc[o][ob], 0, 0, 0);
        }
      }
      // The last read of input row i completes output row i - 2: add the bias,
      // apply the ReLU, round to fp16 (nearest even) and store it straight from
      // the accumulators, so that the output leaves while the matrix cores keep
      // working. Each lane writes 4 channels (8 bytes) of one pixel; the four
      // lanes of a pixel and the other waves fill its 128-byte line in L2 before
      // it is written back.
      if constexpr (v == 2 && h == 1 && i >= 2) {
        constexpr int o = i - 2;
        const int gy = y0 + o;
#pragma unroll
        for (int ob = 0; ob < kOB; ++ob) {
          _Float16 hv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float r = acc[o][ob][e] + bias[ob][e];
            if (a.relu) r = fmaxf(r, 0.f);
            hv[e] = (_Float16)r;
          }
          const unsigned off =
              ((gy < a.H) & col_in) ? (unsigned)gy * row_bytes + col_off + 32u * ob : kOob;
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2v, hv), ry, off, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  {
    const TileDma d0 = dma_for(tile);
#pragma unroll
    for (int j = 0; j < kRounds; ++j) issue_round(d0, lds, j);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int cur = 0;
  while (tile < hi) {
    const int next = tile + step;
    compute_store(tile, lds + cur * kBufChunks, dma_for(next), lds + (cur ^ 1) * kBufChunks);
    // Wait for the next tile's DMA but not for the output stores issued after
    // its last round: vector-memory operations retire in issue order on gfx9.
    __builtin_amdgcn_s_waitcnt(kWaitDmaNotStores);
    __syncthreads();
    tile = next;
    cur ^= 1;
  }
}

}  // namespace

bool configure_mfma(Plan &p) {
  const conv2d_desc &d = p.d;
  if (d.layout != IS_NHWC || d.in_dtype != IS_F16 || d.out_dtype != IS_F16) return false;
  if (d.c != kC || d.k != kK || d.r != 3 || d.s != 3) return false;
  if (2.0 * d.h * (double)d.w * kC >= 4.0e9) return false;   // 32-bit offsets per image
  const long long tiles = (long long)((d.w + kTC - 1) / kTC) * ((d.h + kTR - 1) / kTR) * d.n;
  if (tiles > (1LL << 31) - 1) return false;
  p.kid = kMfmaNhwcF16;
  p.name = "is_k4_mfma";
  p.nseg = (d.w + kTC - 1) / kTC;
  p.nstrip = (d.h + kTR - 1) / kTR;
  p.ntiles = (int)tiles;
  // Persistent: one workgroup per CU (its LDS and registers fill the CU),
  // 8 XCDs x 32 CUs; fewer when there are fewer tiles (kept a multiple of 8).
  int g = 256;
  while (g > 8 && g / 2 >= p.ntiles) g /= 2;
  p.grid_x = g;
  p.grid_y = p.grid_z = 1;
  p.block = kThreads;
  p.lds = 2 * kBufChunks * 16;
  p.tile_w = kTC;
  p.tile_h = kTR;
  // Swizzle row bytes: 128 gives the fewest SQ_LDS_BANK_CONFLICT cycles of 0,
  // 128 and 256. IMGSTENCIL_K4_SWIZZLE=0|128|256 overrides it (read when the
  // plan is created) so that the three layouts can be measured.
  p.vec = 128;
  if (const char *e = getenv("IMGSTENCIL_K4_SWIZZLE")) {
    const int v = atoi(e);
    if (v == 0 || v == 128 || v == 256) p.vec = v;
  }
  return true;
}

hipError_t launch_mfma(const Plan &p, const _Float16 *x, const _Float16 *w, const float *b, _Float16 *y,
                       hipStream_t s) {
  MfmaArgs a;
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
  switch (p.vec) {
    case 0: return launch_kernel(is_k4_mfma<0>, dim3(p.grid_x), dim3(p.block), 0, s, a);
    case 128: return launch_kernel(is_k4_mfma<128>, dim3(p.grid_x), dim3(p.block), 0, s, a);
    default: return launch_kernel(is_k4_mfma<256>, dim3(p.grid_x), dim3(p.block), 0, s, a);
  }
}

}  // namespace is
