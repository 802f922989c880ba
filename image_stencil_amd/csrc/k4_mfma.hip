// k4_mfma.hip -- fp16 NHWC 3x3 layer as an implicit GEMM on the gfx950 matrix
// cores, fp32 accumulation, fp16 output: 64 or 32 input channels, 64, 32 or 16
// output channels (the layers of the pages' upscaling network; fewer real
// output channels run as 16 with zero weights beyond them).
//
// For output pixel p and output channel o the layer is
//   y[p][o] = b[o] + sum_k W[o][k] * X[k][p],  k = (tap t = 3u + v, channel c),
// a dense contraction of length 9 * C (the "blocked GEMM" view of a
// convolution that "Optimizing Memory Efficiency for Convolution Kernels on
// Kepler GPUs" contrasts with its direct method; here the wide-channel layer
// really is that contraction, so it runs on MFMA). The layer sits at the fp16
// ridge point of the chip (288 FLOP per byte of compulsory HBM traffic against
// 312 for 2.5 PFLOP/s over 8 TB/s), so the design keeps the memory streams
// running at full rate under the matrix work:
//  * a workgroup owns a unit: a strip TC pixels wide and UR output rows high of
//    one image (64->64: 32 x 64, one unit per CU at 8 x 256 x 256; fewer output
//    channels widen the strip so that 8 waves stay busy). Units of one XCD are
//    neighbours so that halo rows and columns hit that XCD's L2. A unit's
//    UR + 2 input rows are walked top to bottom in stages of 4 rows;
//  * input rows stream HBM -> LDS by buffer_load ... lds into a ring of D + 1
//    stages, D stages ahead of the stage being read (D = 5 for 64->64, less
//    where wider rows fill the LDS): no tile-sized double buffer that must be
//    complete at a tile boundary. A row is TC pixels x 2C bytes, with its two
//    halo pixels stored after them; each wave moves half a row per stage plus
//    the row's halo pixels. Pixels outside the image read as 0 through the
//    buffer range check;
//  * LDS holds each pixel's C channels as C/8 16-byte chunks, permuted by the
//    XOR swizzle of "CUDA shared memory swizzling" (its formula, with 16-byte
//    elements and chunks) over rows of SWZ bytes, so that 16 lanes reading the
//    same chunk of 16 consecutive pixels hit distinct banks;
//  * 8 waves, 2 per SIMD: wave w owns 16 output channels (one A block) for 16
//    columns of every row (64 outputs: blocks w%4, column halves w/4); its
//    9 * C/32 weight fragments (all 9C k) stay in registers;
//  * v_mfma_f32_16x16x32_f16: A = 16 output channels x 32 k (weights), B = 32 k
//    x 16 pixels (one 16-byte LDS read per lane), D = 4 consecutive output
//    channels of one pixel per lane;
//  * rolling rows: the B fragment of input row i (tap column v, channel half h)
//    is read once and feeds output rows i, i-1 and i-2 through filter rows 0,
//    1 and 2, so only three rows of accumulators are live;
//  * an output row is final once input row +2 has been read: it gets the fp32
//    bias, the optional ReLU and fp16 rounding (nearest even) and goes to an
//    LDS staging area; after the stage's barrier every wave copies its share
//    of the stage's rows to HBM as whole lines (1 KB contiguous per wave
//    operation, 16 bytes per lane, non-temporal), while the matrix cores work
//    on the next stage.
#include "common.hpp"
#include "internal.hpp"


namespace is {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));
typedef unsigned int uint3v __attribute__((ext_vector_type(3)));

constexpr unsigned kOob = 0xFFFFFFF0u;
// Cache policy of the input DMA and the output stores: non-temporal (gfx950 nt
// bit). Every byte is moved once; measured faster than the default policy.
constexpr int kNonTemporal = 2;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsMax = 160 * 1024;
constexpr int kMaxMainOps = 4;   // 16-byte DMA operations per row half, at most

// Geometry of the layer with C input and K output channels. HEAD = r > 0:
// the layer's input is not read from HBM but computed in the unit, as the
// output of a first layer 1 -> C with an r x r filter (the "head"), from the
// one-channel image.
template <int C, int K, int URX = 0, int HEAD = 0>
struct K4Cfg {
  static constexpr int NH = C / 32;             // k steps (32 channels) per tap
  static constexpr int CPP = C / 8;             // 16-byte chunks per input pixel
  static constexpr int KPP = K / 8;             // 16-byte chunks per output pixel
  static constexpr int NOB = K / 16;            // 16-channel output blocks
  static constexpr int NCB = kWaves / NOB;      // 16-pixel column blocks of a unit
  static constexpr int TC = 16 * NCB;           // unit width (output pixels)
  static constexpr int UR = URX ? URX : (K == 16 ? 32 : 64);   // unit height (output rows)
  static constexpr int IN_ROWS = UR + 2;        // input rows of a unit, halo included
  static constexpr int S = 4;                   // input rows per stage
  static constexpr int STAGES = (IN_ROWS + S - 1) / S;
  // 16-byte slots of a row: TC pixels, then 256 bytes for the 2 halo pixels
  // (the 4-byte halo DMA writes 64 lanes x 4 bytes; with 32 channels its
  // second half holds zeros).
  static constexpr int ROW_SLOTS = TC * CPP + 16;
  static constexpr int HALO_SLOT = TC * CPP;    // the 16 slots of the two halo pixels (halo_rel)
  static constexpr int ROW_BYTES = ROW_SLOTS * 16;
  static constexpr int STAGE_BYTES = S * ROW_BYTES;
  static constexpr int OUT_ROW_BYTES = TC * K * 2;       // one output row of the unit, fp16
  // Output staging: two stage buffers (a stage's rows are copied out while the
  // next stage's are written), or one where two would leave fewer than 4 ring
  // slots, i.e. fewer than 3 stages of DMA in flight (the 64- and 128-pixel
  // units of 64 -> 32 and 32 -> 16); one buffer costs a second barrier per
  // stage, between the copy-out reads and the stage's first row write.
  static constexpr int FIT2 = (kLdsMax - 2 * S * OUT_ROW_BYTES) / STAGE_BYTES;
  static constexpr int SBUF = (HEAD == 0 && FIT2 < 4) ? 1 : 2;
  static constexpr int STAGING_BYTES = SBUF * S * OUT_ROW_BYTES;
  static constexpr int FIT = (kLdsMax - STAGING_BYTES) / STAGE_BYTES;   // ring slots that fit
  // Stages in flight ahead of the one read: D DMA stages, or (HEAD) 2 stages
  // of head rows computed ahead.
  static constexpr int D = HEAD ? 2 : (FIT - 1 < 5 ? FIT - 1 : 5);
  static constexpr int NST = HEAD ? 3 : D + 1;  // ring slots
  static constexpr int RING_BYTES = NST * STAGE_BYTES;
  // HEAD: the unit's one-channel image strip, STRIP_ROWS rows from y0-1-HP and
  // 52 columns from x0-1-HP (the head's windows over the halo pixels and the
  // three 16-pixel blocks it is computed in), fp16, after the ring and staging
  // (or after the weights' pass through LDS, whichever is larger).
  static constexpr int HP = HEAD ? (HEAD - 1) / 2 : 0;
  static constexpr int STRIP_COLS = 52;
  static constexpr int STRIP_ROWS = HEAD ? IN_ROWS + 2 * HP : 0;
  static constexpr int STRIP_ROW_BYTES = STRIP_COLS * 2;
  static constexpr int STRIP_OFF_RAW = RING_BYTES + STAGING_BYTES > K * (C * 9 * 2 + 16)
                                           ? RING_BYTES + STAGING_BYTES
                                           : K * (C * 9 * 2 + 16);
  static constexpr int STRIP_OFF = (STRIP_OFF_RAW + 15) / 16 * 16;
  static constexpr int STRIP_BYTES = STRIP_ROWS * STRIP_ROW_BYTES;
  static constexpr int LDS_BYTES = HEAD ? STRIP_OFF + STRIP_BYTES : RING_BYTES + STAGING_BYTES;
  static constexpr int READS_PER_ROW = 3 * NH;  // B reads per input row: tap column x channel half
  static constexpr int READS = IN_ROWS * READS_PER_ROW;
  static constexpr int READS_PER_STAGE = S * READS_PER_ROW;
  static constexpr int KS = 9 * NH;             // A fragments (k steps)
  static constexpr int MAIN_OPS = TC * CPP / 2 / 64;     // 16-byte DMA operations per row half
  static constexpr int DMA_OPS = MAIN_OPS + 1;  // DMA operations per wave and stage
  // Weights are staged once, in ring slots PRE.. and the staging area, while
  // the DMA of the first unit's first PRE stages fills the slots before them
  // (HEAD: from the start of LDS, before any head row is computed).
  static constexpr int PRE = HEAD ? 0 : (D < 3 ? D : 3);
  static constexpr int WROW = C * 9 * 2 + 16;   // bytes per padded weight row
  static constexpr int WSTAGE = PRE * STAGE_BYTES;
  // HEAD: head rows are computed for a stage by all 8 waves, wave w taking row
  // w / 2 of the stage and output-channel blocks 2 (w % 2) and 2 (w % 2) + 1,
  // in three 16-pixel blocks (pixels -1 .. 46 of the row; -1 .. TC used), at
  // read steps HEAD_STEP + 7 p (gather) and + 3 (products, writes).
  static constexpr int HEAD_STEP = 1;

  static_assert(HALO_SLOT % 16 == 0 && TC % 16 == 0, "halo slots keep the 256-byte bank period");
  static_assert(kWaves == 2 * S, "each wave moves half of one row of a stage");
  static_assert(S * OUT_ROW_BYTES == kWaves * 2 * 1024, "each wave stores two 1 KB pieces of a stage");
  static_assert(MAIN_OPS * 64 * 2 == TC * CPP, "whole DMA operations per row half");
  static_assert(MAIN_OPS <= kMaxMainOps, "unit geometry");
  static_assert(D >= 2, "the wait scheme needs two stages ahead");
  static_assert(LDS_BYTES <= kLdsMax, "LDS");
  static_assert(WSTAGE + K * WROW <= LDS_BYTES, "weights fit beside the first stages");
  static_assert(READS_PER_STAGE > 3, "stores and DMA sit at read steps 0, 2 and 3 of a stage");
  static_assert(SBUF == 2 || READS_PER_ROW - 1 >= 2, "one staging buffer: no row write before read step 2");
  static_assert(SBUF == 2 || FIT - 1 >= 3, "one staging buffer buys a third stage of DMA in flight");
  static_assert(HEAD == 0 || (C == 64 && (HEAD == 3 || HEAD == 5) && TC == 32),
                "the head feeds a 64-channel layer of 32-pixel units");
  static_assert(HEAD == 0 || HEAD_STEP + 7 * 2 + 3 < READS_PER_STAGE, "head steps inside a stage");
  static_assert(HEAD == 0 || 16 * 3 + 2 * HP + 2 - HP <= STRIP_COLS, "strip covers the head windows");
};

// ---- VMEM operations of one wave, in program order, per unit:
//   prologue: DMA of stages 0 .. D-1 (DMA_OPS operations each, nothing in
//             between);
//   stage s:  2 stores of stage s-1's rows (s >= 1), then DMA_OPS DMA
//             operations of stage s + D (if it exists).
// vmcnt counts both kinds and they retire in issue order, so "stage `target`'s
// DMA is complete" is "at most vm_after(target, s) operations are outstanding"
// at the end of stage s (s = -1: at the end of the prologue).
template <class G>
constexpr int ops_in_stage(int s) {
  return (s >= 1 ? 2 : 0) + (s + G::D < G::STAGES ? G::DMA_OPS : 0);
}
template <class G>
constexpr int vm_after(int target, int s) {
  int n = 0;
  int from = target - G::D;                    // stage in which target's DMA was issued
  if (from < 0) {
    n += G::DMA_OPS * (G::D - 1 - target);     // later prologue DMAs
    from = -1;
  }
  for (int k = from + 1; k <= s; ++k) n += ops_in_stage<G>(k);
  return n;
}
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Slot of chunk c (0..CPP-1) of pixel px inside one input row. Each row is its
// own swizzled array: rows of SWZ bytes (several pixels when a pixel is shorter)
// whose 16-byte chunks are permuted by XOR with the row index, the formula of
// "CUDA shared memory swizzling" with 16-byte elements and chunks. SWZ = 0
// keeps the plain layout.
template <int SWZ, int CPP>
__host__ __device__ constexpr int slot_in_row(int px, int c) {
  if constexpr (SWZ == 0) {
    return px * CPP + c;
  } else {
    constexpr int NX = SWZ / 16;           // chunks per swizzle row
    constexpr int PPR = NX / CPP;          // pixels per swizzle row
    const int y = px / PPR;
    const int x = (px % PPR) * CPP + c;
    return y * NX + swizzle_col(y, x, NX, 16, 16);
  }
}

// Slot (0..15, after HALO_SLOT) of chunk c of the left (side 0, column x0 - 1)
// or right (side 1, column x0 + TC) halo pixel. A B read takes 16
// consecutive pixels of a row, and a read of the whole wave runs at full rate
// when every one of the LDS's 64 banks (4 bytes each, 16 slots of 16 bytes per
// 256 bytes) receives the same number of accesses. The row's pixels achieve
// that by the swizzle; a halo pixel takes the place modulo 16 slots of the
// pixel one swizzle period away (pixel 15 for the left halo, 16 for the right,
// TC being a multiple of 16), so that reads which include it stay balanced.
// Where those two places coincide (the 256-byte swizzle), the halo pixels
// keep plain positions: left chunks at 0 .. CPP-1, right ones after them.
template <int SWZ, int CPP>
__host__ __device__ constexpr bool halo_balanced() {
  for (int a = 0; a < CPP; ++a)
    for (int b = 0; b < CPP; ++b)
      if ((slot_in_row<SWZ, CPP>(15, a) & 15) == (slot_in_row<SWZ, CPP>(16, b) & 15)) return false;
  return true;
}
template <int SWZ, int CPP>
__host__ __device__ constexpr int halo_rel(int side, int c) {
  if constexpr (halo_balanced<SWZ, CPP>()) return slot_in_row<SWZ, CPP>(side ? 16 : 15, c) & 15;
  return side * CPP + c;
}
// Every halo chunk has a slot of its own among the 16.
template <int SWZ, int CPP>
__host__ __device__ constexpr bool halo_slots_distinct() {
  for (int i = 0; i < 2 * CPP; ++i)
    for (int j = i + 1; j < 2 * CPP; ++j)
      if (halo_rel<SWZ, CPP>(i / CPP, i % CPP) == halo_rel<SWZ, CPP>(j / CPP, j % CPP)) return false;
  for (int i = 0; i < 2 * CPP; ++i)
    if (halo_rel<SWZ, CPP>(i / CPP, i % CPP) < 0 || halo_rel<SWZ, CPP>(i / CPP, i % CPP) > 15) return false;
  return true;
}

// Inverse: pixel and chunk stored at slot si of a row's pixel part. The XOR
// swizzle is an involution inside each swizzle row, so the same map undoes it.
template <int SWZ, int CPP>
__device__ __forceinline__ void chunk_at(int si, int &px, int &c) {
  if constexpr (SWZ == 0) {
    px = si / CPP;
    c = si % CPP;
  } else {
    constexpr int NX = SWZ / 16;
    constexpr int PPR = NX / CPP;
    const int y = si / NX;
    const int x = swizzle_col(y, si % NX, NX, 16, 16);
    px = y * PPR + x / CPP;
    c = x % CPP;
  }
}

struct MfmaArgs {
  const _Float16 *x;
  const _Float16 *w;
  const float *bias;
  _Float16 *y;
  int N, H, W, relu;   // relu: which instance the launch picks (not read by the kernel)
  int kvalid;   // output channels in w and bias; the rest of K computes zeros
  int units_x, units_y, nunits;
  // HEAD: x is the one-channel image (N x H x W fp16); the head's C x 1 x r x r
  // fp16 weights, its fp32 bias (or null) and ReLU flag.
  const _Float16 *wh;
  const float *bh;
  int relu_h;
};

// Where one unit's bytes live: the image's buffer resources, the unit origin,
// and the column parts of this lane's DMA and store offsets (kOob outside).
// A plain struct sized for the widest rows: a class template instantiated in
// the kernel template made this compiler drop the kernels' host-side stubs.
struct UnitGeo {
  __amdgpu_buffer_rsrc_t rx, ry;
  int y0, x0;
  unsigned dcol[kMaxMainOps], hcol;
  unsigned scol[2];
};

// D2S = 3: the layer's first 9 channels go through a 3x3 depth-to-space on
// the way out (y is N x 3H x 3W fp16, out[3i+dy][3j+dx] = z[i][j][3dy+dx]),
// in place of the staged rows' 16-channel pixel lines; 16 output channels only.
// URX: unit height other than the default 64 rows (60 divides a 720-row frame).
template <int SWZ, int C, int K, int D2S = 0, int URX = 0, int HEAD = 0, bool RELU = false>
__global__ __launch_bounds__(kThreads, 1) void is_k4_mfma(MfmaArgs a) {
  using G = K4Cfg<C, K, URX, HEAD>;
  static_assert(D2S == 0 || (D2S == 3 && K == 16), "depth-to-space by 3 of the first 9 of 16 channels");
  static_assert(halo_slots_distinct<SWZ, G::CPP>(), "halo chunks need slots of their own");
  __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
  lds_poison(lds, sizeof(lds));

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;       // pixel (B, D) or output channel (A) inside a 16-block
  const int g = lane >> 4;         // k group of 8 (A, B) or channel group of 4 (D)
  const int og = wave % G::NOB;    // output channels 16*og .. +16
  const int ch = wave / G::NOB;    // unit column block: columns 16*ch .. 16*ch+15

  // ---- Unit schedule: XCD x (= blockIdx mod 8) walks its own contiguous range.
  const int xcd = blockIdx.x & 7;
  const int per_xcd = (a.nunits + 7) / 8;
  const int hi = min(a.nunits, xcd * per_xcd + per_xcd);
  const int step = gridDim.x >> 3;
  int unit = xcd * per_xcd + (blockIdx.x >> 3);
  if (unit >= hi) return;

  const size_t img_in = (size_t)a.H * a.W * C;    // halves per input image
  const size_t img_out = (size_t)a.H * a.W * K;   // halves per output image
  const unsigned in_row_bytes = (unsigned)a.W * C * 2u;
  const unsigned out_row_bytes = (unsigned)a.W * K * 2u;

  // ---- DMA of one stage: wave w moves row w/2 of the stage, its half w%2
  // (MAIN_OPS 1 KB operations, 64 slots each), and the row's two halo pixels
  // (one 4-byte-per-lane operation: C/2 lanes per pixel, the remaining lanes,
  // if any, read nothing and write zeros after them). Both waves of a row load
  // its halo: they write the same bytes to the same place, which keeps every
  // wave's operation count equal and the instruction stream free of branches.
  // Offsets are branch-free 32-bit arithmetic (the plan keeps an image under
  // 4 GB). The halo DMA is 4 bytes per lane even for 32 channels: a narrower
  // LDS DMA still writes a dword per lane.
  const int drow = wave >> 1;
  const int dhalf = wave & 1;
  int dpx[G::MAIN_OPS], dc[G::MAIN_OPS];
#pragma unroll
  for (int j = 0; j < G::MAIN_OPS; ++j)
    chunk_at<SWZ, G::CPP>(dhalf * (G::TC * G::CPP / 2) + 64 * j + lane, dpx[j], dc[j]);
  // Halo DMA: lane l writes bytes 4l .. 4l + 3 of the 16 halo slots, i.e.
  // dword l % 4 of slot l / 4, so it loads that dword of the chunk stored
  // there (halo_rel), or nothing (the slot is unused and gets zeros).
  int hside = 2, hchunk = 0;
#pragma unroll
  for (int side = 0; side < 2; ++side)
#pragma unroll
    for (int c = 0; c < G::CPP; ++c)
      if (halo_rel<SWZ, G::CPP>(side, c) == (lane >> 2)) {
        hside = side;
        hchunk = c;
      }
  const int hpx = hside ? G::TC : -1;
  // Stores: the stage's staged rows are 2 pieces of 1 KB per wave, piece
  // 2w + j covering bytes [1024 (2w + j), +1024) of the 4 rows in row-major
  // order (row w/2), 16 bytes per lane: pixel spx[j], chunk sc[j].
  const int sr = wave >> 1;
  int spx[2], sc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int byte = (2 * (wave & 1) + j) * 1024 + 16 * lane;
    spx[j] = byte / (2 * K);
    sc[j] = (byte % (2 * K)) / 16;
  }
  // D2S: a stage's 4 staged rows make 12 output-row segments (row, dy) of
  // 3 x TC fp16 values; wave w stores segments 2w and 2w + 1 (waves 6 and 7
  // have none and store out of range, which keeps every wave's operation
  // count at 2 per stage), 12 bytes per lane: pixels 2 lane, 2 lane + 1,
  // channels 3 dy .. 3 dy + 2 of each.
  int drow_s[2], ddy[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int seg = 2 * wave + j;
    drow_s[j] = seg < 3 * G::S ? seg / 3 : 0;
    ddy[j] = seg < 3 * G::S ? seg % 3 : -1;
  }

  auto unit_geo = [&](int u) -> UnitGeo {
    UnitGeo q;
    const int tx = u % a.units_x;
    const int ty = (u / a.units_x) % a.units_y;
    const int n = u / (a.units_x * a.units_y);
    q.y0 = ty * G::UR;
    q.x0 = tx * G::TC;
    q.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16 *>(a.x + (size_t)n * img_in), (short)0,
                                             (int)(img_in * 2), kBufferFlags);
    if constexpr (D2S) {
      q.ry = __builtin_amdgcn_make_buffer_rsrc(a.y + (size_t)n * 9 * a.H * a.W, (short)0,
                                               (int)((size_t)18 * a.H * a.W), kBufferFlags);
    } else {
      q.ry = __builtin_amdgcn_make_buffer_rsrc(a.y + (size_t)n * img_out, (short)0, (int)(img_out * 2),
                                               kBufferFlags);
    }
#pragma unroll
    for (int j = 0; j < G::MAIN_OPS; ++j) {
      const int gx = q.x0 + dpx[j];
      q.dcol[j] = gx < a.W ? (unsigned)((gx * C + dc[j] * 8) * 2) : kOob;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (D2S) {
        const int sx = q.x0 + 2 * lane;   // W is even: sx < W covers sx + 1
        q.scol[j] = (ddy[j] >= 0 && sx < a.W) ? (unsigned)(6 * sx) : kOob;
      } else {
        const int sx = q.x0 + spx[j];
        q.scol[j] = sx < a.W ? (unsigned)((sx * K + sc[j] * 8) * 2) : kOob;
      }
    }
    const int hx = q.x0 + hpx;
    q.hcol = (hside < 2 && (unsigned)hx < (unsigned)a.W) ? (unsigned)(hx * C * 2 + hchunk * 16 + 4 * (lane & 3))
                                                          : kOob;
    return q;
  };
  auto issue_stage = [&](const UnitGeo &q, int t) {
    const int li = t * G::S + drow;                      // input row of the unit
    const int gy = q.y0 - 1 + li;
    const bool row_in = (li < G::IN_ROWS) & ((unsigned)gy < (unsigned)a.H);
    const unsigned roff = (unsigned)gy * in_row_bytes;
    char *dst = lds + (t % G::NST) * G::STAGE_BYTES + drow * G::ROW_BYTES;
#pragma unroll
    for (int j = 0; j < G::MAIN_OPS; ++j) {
      const unsigned off = (row_in & (q.dcol[j] != kOob)) ? roff + q.dcol[j] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          q.rx, (__attribute__((address_space(3))) void *)(dst + (dhalf * (G::TC * G::CPP / 2) + 64 * j) * 16),
          16, off, 0, 0, kNonTemporal);
    }
    {
      const unsigned off = (row_in & (q.hcol != kOob)) ? roff + q.hcol : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          q.rx, (__attribute__((address_space(3))) void *)(dst + G::HALO_SLOT * 16), 4, off, 0, 0, kNonTemporal);
    }
  };

  // ---- HEAD: the layer's input rows are computed here from the one-channel
  // image: z[px][c] = f16(act_h(bh[c] + sum_{u,v} wh[c][u][v] x[gy-HP+u][gx-HP+v]))
  // for the unit's input row gy and pixel gx, 0 outside the image (the zero
  // padding of this layer's input). One v_mfma_f32_16x16x32_f16 per 16
  // channels x 16 pixels: A = 16 channels x 32 taps (taps past HEAD^2 have
  // zero weights), B = 32 taps x 16 pixels gathered from the image strip in
  // LDS, D = 4 consecutive channels of one pixel per lane, which go to the
  // pixel's place in the ring row exactly as the DMA of an input row puts them
  // (same swizzle, same halo slots).
  constexpr int kHeadTaps = HEAD * HEAD;
  constexpr int kStripElems = G::STRIP_ROWS * G::STRIP_COLS;
  constexpr int kStripPerThread = HEAD ? (kStripElems + kThreads - 1) / kThreads : 1;
  half8 ha[2];            // head weights of channel blocks 2 (wave % 2) and + 1
  float hb[2][4];         // their biases for this lane's 4 channels
  int toff[8];            // byte offsets in the strip of this lane's taps 8g .. 8g+7
  const int hrow = wave >> 1;             // stage row this wave computes
  const int hob = 2 * (wave & 1);         // first of its two channel blocks
  if constexpr (HEAD) {
    const __amdgpu_buffer_rsrc_t rwh = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<_Float16 *>(a.wh), (short)0, C * kHeadTaps * 2, kBufferFlags);
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      const int o = 16 * (hob + b2) + n16;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tap = 8 * g + j;
        const unsigned off = tap < kHeadTaps ? (unsigned)((o * kHeadTaps + tap) * 2) : kOob;
        ha[b2][j] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rwh, off, 0, 0));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) hb[b2][e] = a.bh ? a.bh[16 * (hob + b2) + 4 * g + e] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tap = 8 * g + j;
      toff[j] = tap < kHeadTaps ? (tap / HEAD) * G::STRIP_ROW_BYTES + (tap % HEAD) * 2 : 0;
    }
  }
  // The image strip of unit geometry q: STRIP_ROWS x 52 fp16 values from
  // (q.y0 - 1 - HP, q.x0 - 1 - HP), 0 outside the image; loaded into registers
  // (strip_load) and then written to LDS (strip_store).
  auto strip_load = [&](int u, unsigned short (&sv)[kStripPerThread]) {
    const int tx = u % a.units_x;
    const int ty = (u / a.units_x) % a.units_y;
    const int n = u / (a.units_x * a.units_y);
    const int sy0 = ty * G::UR - 1 - G::HP, sx0 = tx * G::TC - 1 - G::HP;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<_Float16 *>(a.x + (size_t)n * a.H * a.W), (short)0, (int)((size_t)a.H * a.W * 2), kBufferFlags);
#pragma unroll
    for (int e = 0; e < kStripPerThread; ++e) {
      const int idx = e * kThreads + tid;
      const int gy = sy0 + idx / G::STRIP_COLS, gx = sx0 + idx % G::STRIP_COLS;
      const bool in = idx < kStripElems && (unsigned)gy < (unsigned)a.H && (unsigned)gx < (unsigned)a.W;
      sv[e] = __builtin_amdgcn_raw_buffer_load_b16(rs, in ? (unsigned)((gy * a.W + gx) * 2) : kOob, 0, 0);
    }
  };
  auto strip_store = [&](const unsigned short (&sv)[kStripPerThread]) {
#pragma unroll
    for (int e = 0; e < kStripPerThread; ++e) {
      const int idx = e * kThreads + tid;
      if (kStripElems % kThreads == 0 || idx < kStripElems)
        *reinterpret_cast<unsigned short *>(lds + G::STRIP_OFF + idx * 2) = sv[e];
    }
  };
  // B fragment of pixel block p (pixels 16p - 1 + n16 of the row) for unit
  // input row li: image rows li .. li + 2 HP of the strip.
  auto head_gather = [&](int li, int p) -> half8 {
    half8 b;
    const char *base = lds + G::STRIP_OFF + li * G::STRIP_ROW_BYTES + (16 * p + n16) * 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const _Float16 v = *reinterpret_cast<const _Float16 *>(base + toff[j]);
      b[j] = 8 * g + j < kHeadTaps ? v : (_Float16)0.f;   // as the weights past HEAD^2
    }
    return b;
  };
  // Products of pixel block p of input row li and its two channel blocks, and
  // their place in ring slot `slot` (row hrow of that stage).
  auto head_finish = [&](const UnitGeo &q, int slot, int li, int p, const half8 &bfrag) {
    const int px = 16 * p - 1 + n16;
    const int gy = q.y0 - 1 + li, gx = q.x0 + px;
    const bool inside = (unsigned)gy < (unsigned)a.H && (unsigned)gx < (unsigned)a.W;
    char *row = lds + slot * G::STAGE_BYTES + hrow * G::ROW_BYTES;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      const float4v d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha[b2], bfrag, float4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      _Float16 hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float r = d[e] + hb[b2][e];
        if (a.relu_h) r = fmaxf(r, 0.f);
        hv[e] = inside ? (_Float16)r : (_Float16)0.f;
      }
      const int c = 2 * (hob + b2) + (g >> 1);
      const int sl = px < 0 ? G::HALO_SLOT + halo_rel<SWZ, G::CPP>(0, c)
                            : (px >= G::TC ? G::HALO_SLOT + halo_rel<SWZ, G::CPP>(1, c)
                                           : slot_in_row<SWZ, G::CPP>(px, c));
      if (px <= G::TC) *reinterpret_cast<uint2v *>(row + sl * 16 + (g & 1) * 8) = __builtin_bit_cast(uint2v, hv);
    }
  };
  // Head rows of stage t of the unit (all of them: the prologue's stages).
  auto head_stage = [&](const UnitGeo &q, int t) {
    const int li = t * G::S + hrow;
    if (li < G::IN_ROWS) {
#pragma unroll
      for (int p = 0; p < 3; ++p) head_finish(q, t % G::NST, li, p, head_gather(li, p));
    }
  };

  // ---- Weights and bias: bias and coalesced weight loads first, then the DMA
  // of the first unit's first PRE stages, then the weights' trip through LDS,
  // so that the DMA latency overlaps it. Each output channel's 9C halves go on
  // a row of 18C + 16 bytes (the padding puts the rows of 8 consecutive
  // channels on distinct banks). Fragment ks = NH*t + h of lane (n16, g) holds
  // channels c0 .. c0+8 (c0 = 32h + 8g) of tap t for output channel
  // o = 16*og + n16: halves 9jj + t (jj = 0..7) of the 72 halves
  // w[o][c0 .. c0+8][0..3][0..3], 144 contiguous bytes of o's row, read as 9
  // 16-byte vectors per channel half and sorted in registers. Output channels
  // from kvalid on have no weights or bias: the range checks of the buffer
  // resources read them as 0.
  UnitGeo geo = unit_geo(unit);
  half8 wa[G::KS];
  float bias[4];
  {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int o = 16 * og + 4 * g + e;
      bias[e] = (a.bias && o < a.kvalid) ? a.bias[o] : 0.f;
    }
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<_Float16 *>(a.w), (short)0, a.kvalid * C * 9 * 2, kBufferFlags);
    constexpr int kVecRow = C * 9 * 2 / 16;     // vectors per output channel
    constexpr int kVecs = K * kVecRow;
    constexpr int kVecPerThread = (kVecs + kThreads - 1) / kThreads;
    uint4v t[kVecPerThread];
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j)
      t[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, (j * kThreads + tid) * 16, 0, 0);
    if constexpr (!HEAD) {
#pragma unroll
      for (int st = 0; st < G::PRE; ++st) issue_stage(geo, st);
    }
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j) {
      const int v = j * kThreads + tid;
      const int o = v / kVecRow, r = v - o * kVecRow;
      if (kVecs % kThreads == 0 || v < kVecs)
        *reinterpret_cast<uint4v *>(lds + G::WSTAGE + o * G::WROW + r * 16) = t[j];
    }
  }
  lds_barrier();
  {
    const int o = 16 * og + n16;
    half8 raw[G::NH][9];
#pragma unroll
    for (int h = 0; h < G::NH; ++h)
#pragma unroll
      for (int j = 0; j < 9; ++j)
        raw[h][j] =
            *reinterpret_cast<const half8 *>(lds + G::WSTAGE + o * G::WROW + (32 * h + 8 * g) * 18 + 16 * j);
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      const int t = ks / G::NH, h = ks % G::NH;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) wa[ks][jj] = raw[h][(9 * jj + t) / 8][(9 * jj + t) % 8];
    }
  }
  lds_barrier();   // the weights' LDS is ring space from here on
  // The first unit's first D stages: DMA, or (HEAD) the image strip and the
  // head rows of stages 0 and 1.
  auto unit_start = [&](const UnitGeo &q, int u, int from) {
    if constexpr (HEAD) {
      unsigned short sv[kStripPerThread];
      strip_load(u, sv);
      strip_store(sv);
      lds_barrier();
#pragma unroll
      for (int st = 0; st < G::D; ++st) head_stage(q, st);
    } else {
#pragma unroll
      for (int st = from; st < G::D; ++st) issue_stage(q, st);
    }
  };
  unit_start(geo, unit, G::PRE);

  // Byte offsets (inside a row) of this lane's B reads for filter column v and
  // channel half h: pixel 16*ch + n16 + v - 1 of the row, chunk 4h + g.
  int boff[3][G::NH];
#pragma unroll
  for (int v = 0; v < 3; ++v)
#pragma unroll
    for (int h = 0; h < G::NH; ++h) {
      const int px = 16 * ch + n16 + v - 1;
      const int c = 4 * h + g;
      const int slot = px < 0 ? G::HALO_SLOT + halo_rel<SWZ, G::CPP>(0, c)
                              : (px >= G::TC ? G::HALO_SLOT + halo_rel<SWZ, G::CPP>(1, c)
                                             : slot_in_row<SWZ, G::CPP>(px, c));
      boff[v][h] = slot * 16;
    }
  // Staging: output row r of a stage holds pixel px's K channels as K/8 chunks
  // of 16 bytes, chunk c at position c ^ skey(px), its two 8-byte halves swapped
  // when shalf(px). A fragment write (8 bytes per lane) is served 16 lanes at a
  // time over 32 banks (128 bytes): its 16 lanes write 16 consecutive pixels,
  // the same 4 channels of each, and skey (which 16-byte position within the
  // pixel's 128-byte window) with shalf (which half) give the 16 pixels 16
  // distinct 8-byte places in that window. A line read (16 bytes per lane)
  // takes whole pixels, so it keeps all 64 banks equally loaded; the halves
  // are swapped back in registers. This lane writes channels 16*og + 4g .. +4
  // of pixel 16*ch + n16; it reads chunk sc[j] of pixel spx[j].
  constexpr int kPixPerWin = 64 / K;   // pixels per 128-byte window
  auto skey = [](int px) { return (px / kPixPerWin) & (G::KPP - 1); };
  auto shalf = [](int px) { return (px >> 3) & 1; };
  const int wpx = 16 * ch + n16;
  const int soff_w = G::RING_BYTES + wpx * 2 * K + (((2 * og + (g >> 1)) ^ skey(wpx)) * 16) +
                     (((g & 1) ^ shalf(wpx)) * 8);
  int soff_r[2];
  bool sswap[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    soff_r[j] = G::RING_BYTES + sr * G::OUT_ROW_BYTES + spx[j] * 2 * K + ((sc[j] ^ skey(spx[j])) * 16);
    sswap[j] = shalf(spx[j]) != 0;
  }
  // D2S staging: a staged row holds the first 9 channels as 9 planes of TC
  // fp16 values, plane c = 3 dy + dx at c * kD2sPlane bytes. A fragment write
  // puts each of its (up to) 4 channels into its plane: 16 lanes write 32
  // consecutive bytes, and the plane pitch of 68 dwords puts the planes that
  // one instruction writes (c, c + 4, c + 8) 16 dwords apart on the banks. A
  // copy-out read takes one dword (pixels 2 lane, 2 lane + 1) from each of a
  // segment's 3 planes: 64 consecutive dwords, one per bank. (With the
  // pixel-major layout of the other layers, those reads were 2-byte loads of
  // pixels 64 bytes apart: 54% of the LDS cycles were bank conflicts.)
  constexpr int kD2sPlane = 272;
  static_assert(!D2S || (9 * kD2sPlane <= G::OUT_ROW_BYTES && 2 * G::TC <= kD2sPlane), "D2S planes fit a staged row");
  int doff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    doff[j] = G::RING_BYTES + drow_s[j] * G::OUT_ROW_BYTES + 3 * (ddy[j] < 0 ? 0 : ddy[j]) * kD2sPlane + 4 * lane;
  const int d2s_w = G::RING_BYTES + 2 * wpx;   // + row + plane c * kD2sPlane
  const unsigned out3_row_bytes = (unsigned)a.W * 6u;   // D2S output row: 3W fp16

  while (true) {
    // ---- Unit prologue: stages 0 .. D-1 are in flight; the first two must
    // have landed before the first read.
    if constexpr (!HEAD) __builtin_amdgcn_s_waitcnt(waitcnt_vm(vm_after<G>(1, -1)));
    lds_barrier();

    auto read_b = [&](int q) -> half8 {
      const int i = q / G::READS_PER_ROW, v = (q % G::READS_PER_ROW) / G::NH, h = q % G::NH;
      const char *p = lds + ((i / G::S) % G::NST) * G::STAGE_BYTES + (i % G::S) * G::ROW_BYTES + boff[v][h];
      return *reinterpret_cast<const half8 *>(p);
    };
    // This wave's two 1 KB pieces of staged row sr of stage t, to registers
    // and then to HBM (output row t*S + sr - 2 of the unit).
    auto read_staged = [&](int t, uint4v (&sv)[2]) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (D2S) {
          // Planes dx = 0, 1, 2 of the segment: (pixel 2 lane, pixel 2 lane + 1)
          // each; the output takes both pixels' 3 values in turn.
          const char *base = lds + (t % G::SBUF) * G::S * G::OUT_ROW_BYTES + doff[j];
          const unsigned d0 = *reinterpret_cast<const unsigned *>(base);
          const unsigned d1 = *reinterpret_cast<const unsigned *>(base + kD2sPlane);
          const unsigned d2 = *reinterpret_cast<const unsigned *>(base + 2 * kD2sPlane);
          sv[j] = uint4v{(d0 & 0xFFFFu) | (d1 << 16), (d2 & 0xFFFFu) | (d0 & 0xFFFF0000u),
                         (d1 >> 16) | (d2 & 0xFFFF0000u), 0u};
        } else {
          const uint4v v = *reinterpret_cast<const uint4v *>(lds + soff_r[j] + (t % G::SBUF) * G::S * G::OUT_ROW_BYTES);
          sv[j] = sswap[j] ? uint4v{v.z, v.w, v.x, v.y} : v;
        }
      }
    };
    auto store_stage = [&](int t, const uint4v (&sv)[2]) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (D2S) {
          const int o = t * G::S + drow_s[j] - 2;
          const int gy = geo.y0 + o;
          const bool row_out = (o >= 0) & (o < G::UR) & (gy < a.H);
          const unsigned off = (row_out & (geo.scol[j] != kOob))
                                   ? (unsigned)(3 * gy + ddy[j]) * out3_row_bytes + geo.scol[j]
                                   : kOob;
          const uint3v v3 = {sv[j].x, sv[j].y, sv[j].z};
          __builtin_amdgcn_raw_buffer_store_b96(v3, geo.ry, off, 0, kNonTemporal);
        } else {
          const int o = t * G::S + sr - 2;
          const int gy = geo.y0 + o;
          const bool row_out = (o >= 0) & (o < G::UR) & (gy < a.H);
          const unsigned off =
              (row_out & (geo.scol[j] != kOob)) ? (unsigned)gy * out_row_bytes + geo.scol[j] : kOob;
          __builtin_amdgcn_raw_buffer_store_b128(sv[j], geo.ry, off, 0, kNonTemporal);
        }
      }
    };

    constexpr int kAhead = 8;
    half8 ring[kAhead];
    half8 hfrag = {};   // HEAD: the pixel block gathered for the next head products
#pragma unroll
    for (int q = 0; q < kAhead; ++q) ring[q] = read_b(q);
    float4v acc[4];
    uint4v sv[2];
    static_for<G::READS>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      constexpr int i = q / G::READS_PER_ROW, v = (q % G::READS_PER_ROW) / G::NH, h = q % G::NH;
      constexpr int t = i / G::S;                          // stage of input row i
      constexpr int qs = q % G::READS_PER_STAGE;           // read step inside the stage
      // Stage t - 1's rows leave for HBM; stage t + D's rows start their DMA.
      if constexpr (t >= 1 && qs == 0) read_staged(t - 1, sv);
      // One staging buffer: every wave's copy-out reads are done before any
      // wave writes this stage's first row (read step 2 or later).
      if constexpr (G::SBUF == 1 && t >= 1 && qs == 1) lds_barrier();
      if constexpr (t >= 1 && qs == 2) store_stage(t - 1, sv);
      if constexpr (!HEAD && t + G::D < G::STAGES && qs == 3) issue_stage(geo, t + G::D);
      // HEAD: the head rows of stage t + 2, pixel block p gathered at step
      // HEAD_STEP + 7p and finished three steps later.
      constexpr bool kHeadStep = HEAD && t + 2 < G::STAGES && qs >= G::HEAD_STEP &&
                                 qs <= G::HEAD_STEP + 14 + 3 && (qs - G::HEAD_STEP) % 7 <= 3 &&
                                 ((qs - G::HEAD_STEP) % 7 == 0 || (qs - G::HEAD_STEP) % 7 == 3);
      if constexpr (kHeadStep) {
        constexpr int p = (qs - G::HEAD_STEP) / 7;
        const int li = (t + 2) * G::S + hrow;
        if constexpr ((qs - G::HEAD_STEP) % 7 == 0) {
          if (li < G::IN_ROWS) hfrag = head_gather(li, p);
        } else {
          if (li < G::IN_ROWS) head_finish(geo, (t + 2) % G::NST, li, p, hfrag);
        }
      }
      if constexpr (qs == 0 || (G::SBUF == 1 && qs == 1) || qs == 2 || qs == 3 || kHeadStep)
        __builtin_amdgcn_sched_barrier(0);

      const half8 b = ring[q % kAhead];
      if constexpr (q + kAhead < G::READS) ring[q % kAhead] = read_b(q + kAhead);
      if constexpr (v == 0 && h == 0 && i < G::UR) acc[i & 3] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int o = i - u;
        if (o >= 0 && o < G::UR) {
          const int ks = G::NH * (3 * u + v) + h;
          acc[o & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[ks], b, acc[o & 3], 0, 0, 0);
        }
      }
      // The last read of input row i completes output row i - 2: bias, ReLU,
      // fp16 (nearest even), into stage t's staging rows.
      if constexpr (v == 2 && h == G::NH - 1 && i >= 2 && i - 2 < G::UR) {
        constexpr int o = i - 2;
        _Float16 hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float r = acc[o & 3][e] + bias[e];
          if constexpr (RELU) r = fmaxf(r, 0.f);
          hv[e] = (_Float16)r;
        }
        if constexpr (D2S) {
          // Channels 4g .. 4g + 3 of pixel wpx into their planes (the first 9).
          char *row = lds + d2s_w + ((t % G::SBUF) * G::S + (i % G::S)) * G::OUT_ROW_BYTES;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * g + e < 9) *reinterpret_cast<_Float16 *>(row + (4 * g + e) * kD2sPlane) = hv[e];
        } else {
          *reinterpret_cast<uint2v *>(lds + soff_w + ((t % G::SBUF) * G::S + (i % G::S)) * G::OUT_ROW_BYTES) =
              __builtin_bit_cast(uint2v, hv);
        }
      }
      // End of stage t: stage t + 2 (read from the next stage's last steps on,
      // through the read-ahead ring) must have landed; the barrier publishes it,
      // frees stage t's ring slot and completes stage t's staged rows.
      if constexpr (qs == G::READS_PER_STAGE - 1 || q == G::READS - 1) {
        if constexpr (!HEAD && t + 2 < G::STAGES) __builtin_amdgcn_s_waitcnt(waitcnt_vm(vm_after<G>(t + 2, t)));
        lds_barrier();
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    read_staged(G::STAGES - 1, sv);
    store_stage(G::STAGES - 1, sv);

    unit += step;
    if (unit >= hi) break;
    // The next unit's first D stages go out now: their ring slots were freed
    // by this unit's last barrier, and the next unit's first barrier comes
    // after this unit's last staging reads.
    geo = unit_geo(unit);
    unit_start(geo, unit, 0);
  }
}

// (C, K) pairs with a kernel: the layers of the pages' upscaling network.
bool shape_supported(int c, int k) {
  return (c == 64 && (k == 64 || k == 32)) || (c == 32 && (k == 32 || k == 16));
}

template <int C, int K, int URX = 0>
void fill_geometry(Plan &p) {
  using G = K4Cfg<C, K, URX>;
  p.nseg = (p.d.w + G::TC - 1) / G::TC;
  p.nstrip = (p.d.h + G::UR - 1) / G::UR;
  p.lds = G::LDS_BYTES;
  p.tile_w = G::TC;
  p.tile_h = G::UR;
}

// The layer's ReLU is a compile-time choice: a run-time flag costs a select
// per output value in the row epilogue (1.5% of the 64 -> 64 layer's time).
template <int SWZ, int C, int K, int D2S = 0, int URX = 0, int HEAD = 0>
hipError_t launch_k4(const MfmaArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  return a.relu ? launch_kernel(is_k4_mfma<SWZ, C, K, D2S, URX, HEAD, true>, grid, block, 0, s, a)
                : launch_kernel(is_k4_mfma<SWZ, C, K, D2S, URX, HEAD, false>, grid, block, 0, s, a);
}

}  // namespace

bool configure_mfma(Plan &p, int param) {
  const conv2d_desc &d = p.d;
  if (d.layout != IS_NHWC || d.in_dtype != IS_F16 || d.out_dtype != IS_F16) return false;
  if (!shape_supported(d.c, d.k) || d.r != 3 || d.s != 3) return false;
  if (2.0 * d.h * (double)d.w * d.c >= 4.0e9 || 2.0 * d.h * (double)d.w * d.k >= 4.0e9)
    return false;   // 32-bit offsets per image
  // Unit height: 64 rows (32 for 16 output channels), or 60 (30) when that
  // computes fewer rows past the image's last one. A 720-row frame: 12 units
  // of 60 rows against 12 of 64, a twelfth of them below the image; with 16
  // output channels 24 units of 30 rows, 32 input rows = 8 whole stages each,
  // against 23 units of 32 rows, 34 input rows = 9 stages, the last one half
  // used, and 16 rows below the image.
  const bool ur60 = (d.h + 59) / 60 * 60 < (d.h + 63) / 64 * 64;
  const bool ur30 = (d.h + 29) / 30 * 30 < (d.h + 31) / 32 * 32;
  if (d.c == 64 && d.k == 64) {
    if (ur60) fill_geometry<64, 64, 60>(p);
    else fill_geometry<64, 64>(p);
  } else if (d.c == 64) {
    if (ur60) fill_geometry<64, 32, 60>(p);
    else fill_geometry<64, 32>(p);
  } else if (d.k == 32) {
    if (ur60) fill_geometry<32, 32, 60>(p);
    else fill_geometry<32, 32>(p);
  } else {
    if (ur30) fill_geometry<32, 16, 30>(p);
    else fill_geometry<32, 16>(p);
  }
  const long long units = (long long)p.nseg * p.nstrip * d.n;
  if (units > (1LL << 31) - 1) return false;
  p.kid = kMfmaNhwcF16;
  p.name = "is_k4_mfma";
  p.ntiles = (int)units;
  p.kvalid = d.k;
  // Persistent: one workgroup per CU (its LDS and registers fill the CU);
  // fewer when there are fewer units.
  p.grid_x = persistent_grid(p.ntiles, 256);
  p.grid_y = p.grid_z = 1;
  p.block = kThreads;
  // Swizzle row bytes: 128 gives the fewest SQ_LDS_BANK_CONFLICT cycles of 0,
  // 128 and 256 on the 64 -> 64 layer; the other two are tuning variants.
  p.vec = 128;
  if (param != 0) {   // a tuning variant: swizzle row bytes (-1 = none); 64 -> 64 only has all three
    const int v = param < 0 ? 0 : param;
    if (v != 128 && !(d.c == 64 && d.k == 64 && (v == 0 || v == 256))) return false;
    p.vec = v;
  }
  // The 60-row units are built with the 128-byte swizzle only.
  if (p.vec != 128 && p.tile_h == 60) {
    if (d.c == 64 && d.k == 64) fill_geometry<64, 64>(p);
    else fill_geometry<64, 32>(p);
    const long long u64 = (long long)p.nseg * p.nstrip * d.n;
    p.ntiles = (int)u64;
    p.grid_x = persistent_grid(p.ntiles, 256);
  }
  return true;
}

bool mfma_d2s3_supported(const Plan &p) {
  const conv2d_desc &d = p.d;
  return p.kid == kMfmaNhwcF16 && d.c == 32 && d.k == 16 && p.vec == 128 && p.kvalid == 9 && d.w % 2 == 0 &&
         18.0 * d.h * (double)d.w < 2.0e9;
}

hipError_t launch_mfma_d2s3(const Plan &p, const _Float16 *x, const _Float16 *w, const float *b, _Float16 *y,
                            hipStream_t s) {
  if (!mfma_d2s3_supported(p)) return hipErrorInvalidValue;
  MfmaArgs a;
  a.x = x;
  a.w = w;
  a.bias = b;
  a.y = y;
  a.N = p.d.n;
  a.H = p.d.h;
  a.W = p.d.w;
  a.relu = p.d.relu;
  a.kvalid = p.kvalid;
  a.units_x = p.nseg;
  a.units_y = p.nstrip;
  a.nunits = p.ntiles;
  a.wh = nullptr;
  a.bh = nullptr;
  a.relu_h = 0;
  const dim3 grid(persistent_grid(p.ntiles, device_cu_count())), block(p.block);
  return p.tile_h == 30 ? launch_k4<128, 32, 16, 3, 30>(a, grid, block, s)
                        : launch_k4<128, 32, 16, 3>(a, grid, block, s);
}

bool mfma_head_supported(const Plan &p, int head_r) {
  const conv2d_desc &d = p.d;
  return p.kid == kMfmaNhwcF16 && d.c == 64 && d.k == 64 && p.vec == 128 && p.kvalid == d.k &&
         (head_r == 3 || head_r == 5) && (p.tile_h == 64 || p.tile_h == 60);
}

hipError_t launch_mfma_head(const Plan &p, const _Float16 *x1, const _Float16 *wh, const float *bh, int relu_h,
                            int head_r, const _Float16 *w, const float *b, _Float16 *y, hipStream_t s) {
  if (!mfma_head_supported(p, head_r)) return hipErrorInvalidValue;
  MfmaArgs a;
  a.x = x1;
  a.w = w;
  a.bias = b;
  a.y = y;
  a.N = p.d.n;
  a.H = p.d.h;
  a.W = p.d.w;
  a.relu = p.d.relu;
  a.kvalid = p.kvalid;
  a.units_x = p.nseg;
  a.units_y = p.nstrip;
  a.nunits = p.ntiles;
  a.wh = wh;
  a.bh = bh;
  a.relu_h = relu_h;
  const dim3 grid(persistent_grid(p.ntiles, device_cu_count())), block(p.block);
  const bool u60 = p.tile_h == 60;
  if (head_r == 5)
    return u60 ? launch_k4<128, 64, 64, 0, 60, 5>(a, grid, block, s)
               : launch_k4<128, 64, 64, 0, 0, 5>(a, grid, block, s);
  return u60 ? launch_k4<128, 64, 64, 0, 60, 3>(a, grid, block, s)
             : launch_k4<128, 64, 64, 0, 0, 3>(a, grid, block, s);
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
  a.kvalid = p.kvalid;
  a.units_x = p.nseg;
  a.units_y = p.nstrip;
  a.nunits = p.ntiles;
  a.wh = nullptr;
  a.bh = nullptr;
  a.relu_h = 0;
  const dim3 grid(persistent_grid(p.ntiles, device_cu_count())), block(p.block);
  if (p.d.c == 64 && p.d.k == 64) {
    if (p.tile_h == 60) return launch_k4<128, 64, 64, 0, 60>(a, grid, block, s);
    switch (p.vec) {
      case 0: return launch_k4<0, 64, 64>(a, grid, block, s);
      case 128: return launch_k4<128, 64, 64>(a, grid, block, s);
      default: return launch_k4<256, 64, 64>(a, grid, block, s);
    }
  }
  if (p.d.c == 64 && p.d.k == 32) {
    if (p.tile_h == 60) return launch_k4<128, 64, 32, 0, 60>(a, grid, block, s);
    return launch_k4<128, 64, 32>(a, grid, block, s);
  }
  if (p.d.c == 32 && p.d.k == 32) {
    if (p.tile_h == 60) return launch_k4<128, 32, 32, 0, 60>(a, grid, block, s);
    return launch_k4<128, 32, 32>(a, grid, block, s);
  }
  if (p.d.c == 32 && p.d.k == 16) {
    if (p.tile_h == 30) return launch_k4<128, 32, 16, 0, 30>(a, grid, block, s);
    return launch_k4<128, 32, 16>(a, grid, block, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace is
