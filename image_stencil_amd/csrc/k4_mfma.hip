// k4_mfma.hip -- fp16 NHWC 3x3 layer with 64 input and 64 output channels as an
// implicit GEMM on the gfx950 matrix cores, fp32 accumulation, fp16 output.
//
// For output pixel p and output channel o the layer is
//   y[p][o] = b[o] + sum_k W[o][k] * X[k][p],  k = (tap t = 3u + v, channel c),
// a dense contraction of length 9 * 64 = 576 (the "blocked GEMM" view of a
// convolution that "Optimizing Memory Efficiency for Convolution Kernels on
// Kepler GPUs" contrasts with its direct method; here the wide-channel layer
// really is that contraction, so it runs on MFMA). The layer sits at the fp16
// ridge point of the chip (288 FLOP per byte of compulsory HBM traffic against
// 312 for 2.5 PFLOP/s over 8 TB/s), so the design keeps the memory streams
// running at full rate under the matrix work:
//  * a workgroup owns a unit: a strip 32 pixels wide and 64 output rows high of
//    one image (one unit per CU at 8 x 256 x 256; units of one XCD are
//    neighbours so that halo rows and columns hit that XCD's L2). It walks
//    the 66 input rows of its unit top to bottom in stages of 4 rows;
//  * input rows stream HBM -> LDS by buffer_load ... lds into a ring of 6
//    stages, 5 stages (20 rows) ahead of the stage being read: no tile-sized
//    double buffer that must be complete at a tile boundary. A row is 32
//    pixels x 128 bytes, with its two halo pixels stored after them; each wave
//    moves half a row per stage plus the row's halo pixels. Pixels outside the
//    image read as 0 through the buffer range check;
//  * LDS holds each pixel's 64 channels as eight 16-byte chunks, permuted by the
//    XOR swizzle of "CUDA shared memory swizzling" (its formula, with 16-byte
//    elements and chunks) over rows of SWZ bytes, so that 16 lanes reading the
//    same chunk of 16 consecutive pixels hit distinct banks;
//  * 8 waves, 2 per SIMD: wave w owns the 16 output channels 16*(w%4) .. +16
//    (one A block) for the 16 columns 16*(w/4) .. +16 of every row; its 18
//    weight fragments (all 576 k) stay in registers;
//  * v_mfma_f32_16x16x32_f16: A = 16 output channels x 32 k (weights), B = 32 k
//    x 16 pixels (one 16-byte LDS read per lane), D = 4 consecutive output
//    channels of one pixel per lane;
//  * rolling rows: the B fragment of input row i (tap column v, channel half h)
//    is read once and feeds output rows i, i-1 and i-2 through filter rows 0,
//    1 and 2, so only three rows of accumulators are live;
//  * an output row is final once input row +2 has been read: it gets the fp32
//    bias, the optional ReLU and fp16 rounding (nearest even) and goes to an
//    LDS staging area; after the stage's barrier every wave copies its share
//    of the stage's rows to HBM as whole 128-byte pixel lines (16 bytes per
//    lane, non-temporal), while the matrix cores work on the next stage.
#include "common.hpp"
#include "internal.hpp"

#include <stdlib.h>

namespace is {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));

constexpr int kC = 64;                        // input channels
constexpr int kK = 64;                        // output channels
constexpr int kTC = 32;                       // unit width (output pixels)
constexpr int kUR = 64;                       // unit height (output rows)
constexpr int kInRows = kUR + 2;              // input rows of a unit, halo included
constexpr int kS = 4;                         // input rows per stage
constexpr int kStages = (kInRows + kS - 1) / kS;
constexpr int kD = 5;                         // stages in flight ahead of the one read
constexpr int kNst = kD + 1;                  // ring slots
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowSlots = kTC * 8 + 16;       // 16-byte slots of an input row: 32 pixels, 2 halo pixels
constexpr int kHaloSlot = kTC * 8;            // left halo pixel; the right one follows
constexpr int kRowBytes = kRowSlots * 16;
constexpr int kStageBytes = kS * kRowBytes;
constexpr int kRingBytes = kNst * kStageBytes;
constexpr int kOutRowBytes = kTC * kK * 2;    // one output row of the unit, fp16
constexpr int kStagingBytes = 2 * kS * kOutRowBytes;
constexpr int kLdsBytes = kRingBytes + kStagingBytes;
constexpr int kReads = kInRows * 6;           // B reads per wave and unit
constexpr int kReadsPerStage = kS * 6;
constexpr unsigned kOob = 0xFFFFFFF0u;
// Cache policy of the input DMA and the output stores: non-temporal (gfx950 nt
// bit). Every byte is moved once; measured faster than the default policy.
constexpr int kNonTemporal = 2;

static_assert(kWaves == 2 * kS, "each wave moves half of one row of a stage");
static_assert(kS * kOutRowBytes == kWaves * 2 * 1024, "each wave stores two 1 KB pieces of a stage");

// Weights are staged once, in ring slots kPreStages.. and the staging area,
// while the DMA of the first unit's first kPreStages stages fills the slots
// before them.
constexpr int kPreStages = 3;
constexpr int kWRow = kC * 9 * 2 + 16;        // bytes per padded weight row
constexpr int kWStage = kPreStages * kStageBytes;
static_assert(kWStage + kK * kWRow <= kLdsBytes, "weights fit beside the first stages");

// ---- VMEM operations of one wave, in program order, per unit:
//   prologue: DMA of stages 0 .. kD-1 (3 operations each, nothing in between);
//   stage s:  2 stores of stage s-1's rows (s >= 1), then 3 DMA operations of
//             stage s + kD (if it exists).
// vmcnt counts both kinds and they retire in issue order, so "stage `target`'s
// DMA is complete" is "at most vm_after(target, s) operations are outstanding"
// at the end of stage s (s = -1: at the end of the prologue).
constexpr int ops_in_stage(int s) { return (s >= 1 ? 2 : 0) + (s + kD < kStages ? 3 : 0); }
constexpr int vm_after(int target, int s) {
  int n = 0;
  int from = target - kD;                      // stage in which target's DMA was issued
  if (from < 0) {
    n += 3 * (kD - 1 - target);                // later prologue DMAs
    from = -1;
  }
  for (int k = from + 1; k <= s; ++k) n += ops_in_stage(k);
  return n;
}
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
static_assert(vm_after(kD + 2, kD) < 64 && vm_after(0, 0) < 64, "vmcnt field");

// Slot of chunk c (0..7) of pixel px (0..31) inside one input row. Each row is
// its own swizzled array: rows of SWZ bytes (one pixel for 128, a pixel pair
// for 256) whose 16-byte chunks are permuted by XOR with the row index, the
// formula of "CUDA shared memory swizzling" with 16-byte elements and chunks.
// SWZ = 0 keeps the plain layout.
template <int SWZ>
__device__ __forceinline__ int slot_in_row(int px, int c) {
  if constexpr (SWZ == 0) {
    return px * 8 + c;
  } else {
    constexpr int NX = SWZ / 16;           // chunks per swizzle row
    constexpr int PPR = NX / 8;            // pixels per swizzle row
    const int y = px / PPR;
    const int x = (px % PPR) * 8 + c;
    return y * NX + swizzle_col(y, x, NX, 16, 16);
  }
}

// Inverse: pixel and chunk stored at slot si (< 256) of a row. The XOR
// swizzle is an involution inside each swizzle row, so the same map undoes it.
template <int SWZ>
__device__ __forceinline__ void chunk_at(int si, int &px, int &c) {
  if constexpr (SWZ == 0) {
    px = si >> 3;
    c = si & 7;
  } else {
    constexpr int NX = SWZ / 16;
    constexpr int PPR = NX / 8;
    const int y = si / NX;
    const int x = swizzle_col(y, si % NX, NX, 16, 16);
    px = y * PPR + x / 8;
    c = x % 8;
  }
}

struct MfmaArgs {
  const _Float16 *x;
  const _Float16 *w;
  const float *bias;
  _Float16 *y;
  int N, H, W, relu;
  int units_x, units_y, nunits;
};

// Where one unit's bytes live: the image's buffer resources, the unit origin,
// and the column parts of this lane's DMA and store offsets (kOob outside).
struct UnitGeo {
  __amdgpu_buffer_rsrc_t rx, ry;
  int y0, x0;
  unsigned dcol[2], hcol;
  unsigned scol[2];
};

template <int SWZ>
__global__ __launch_bounds__(kThreads, 1) void is_k4_mfma(MfmaArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;      // pixel (B, D) or output channel (A) inside a 16-block
  const int g = lane >> 4;        // k group of 8 (A, B) or channel group of 4 (D)
  const int og = wave & 3;        // output channels 16*og .. +16
  const int ch = wave >> 2;       // unit-column half: columns 16*ch .. 16*ch+15

  // ---- Unit schedule: XCD x (= blockIdx mod 8) walks its own contiguous range.
  const int xcd = blockIdx.x & 7;
  const int per_xcd = (a.nunits + 7) / 8;
  const int hi = min(a.nunits, xcd * per_xcd + per_xcd);
  const int step = gridDim.x >> 3;
  int unit = xcd * per_xcd + (blockIdx.x >> 3);
  if (unit >= hi) return;

  const size_t img = (size_t)a.H * a.W * kC;   // halves per image
  const unsigned pix_row_bytes = (unsigned)a.W * kC * 2u;

  // ---- DMA of one stage: wave w moves row w/2 of the stage, pixels
  // 16*(w%2) .. +16 (two 1 KB operations, 64 slots each), and the row's two
  // halo pixels (one 4-byte-per-lane operation: 64 x 4 bytes = both 128-byte
  // pixels, the whole halo part of the row). Both waves of a row load its halo:
  // they write the same bytes to the same place, which keeps every wave's
  // operation count equal and the instruction stream free of branches.
  // Offsets are branch-free 32-bit arithmetic (the plan keeps an image under
  // 4 GB).
  const int drow = wave >> 1;
  const int dhalf = wave & 1;
  int dpx[2], dc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) chunk_at<SWZ>(128 * dhalf + 64 * j + lane, dpx[j], dc[j]);
  const int hpx = (lane >> 5) ? kTC : -1;   // halo DMA: lanes 0-31 left pixel, 32-63 right
  // Stores: wave w copies row w/2 of a stage's staged rows, pixels
  // 16*(w%2) + 8j + lane/8 (j = 0, 1), chunk lane%8: whole 128-byte lines.
  const int sr = wave >> 1;
  const int spx = 16 * (wave & 1) + (lane >> 3);
  const int sc = lane & 7;

  auto unit_geo = [&](int u) -> UnitGeo {
    UnitGeo q;
    const int tx = u % a.units_x;
    const int ty = (u / a.units_x) % a.units_y;
    const int n = u / (a.units_x * a.units_y);
    q.y0 = ty * kUR;
    q.x0 = tx * kTC;
    q.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16 *>(a.x + (size_t)n * img), (short)0,
                                             (int)(img * 2), kBufferFlags);
    q.ry = __builtin_amdgcn_make_buffer_rsrc(a.y + (size_t)n * img, (short)0, (int)(img * 2), kBufferFlags);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gx = q.x0 + dpx[j];
      q.dcol[j] = gx < a.W ? (unsigned)((gx * kC + dc[j] * 8) * 2) : kOob;
      const int sx = q.x0 + spx + 8 * j;
      q.scol[j] = sx < a.W ? (unsigned)((sx * kK + sc * 8) * 2) : kOob;
    }
    const int hx = q.x0 + hpx;
    q.hcol = ((unsigned)hx < (unsigned)a.W) ? (unsigned)(hx * kC * 2 + 4 * (lane & 31)) : kOob;
    return q;
  };
  auto issue_stage = [&](const UnitGeo &q, int t) {
    const int li = t * kS + drow;                        // input row of the unit
    const int gy = q.y0 - 1 + li;
    const bool row_in = (li < kInRows) & ((unsigned)gy < (unsigned)a.H);
    const unsigned roff = (unsigned)gy * pix_row_bytes;
    char *dst = lds + (t % kNst) * kStageBytes + drow * kRowBytes;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const unsigned off = (row_in & (q.dcol[j] != kOob)) ? roff + q.dcol[j] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          q.rx, (__attribute__((address_space(3))) void *)(dst + (128 * dhalf + 64 * j) * 16), 16, off, 0, 0,
          kNonTemporal);
    }
    {
      const unsigned off = (row_in & (q.hcol != kOob)) ? roff + q.hcol : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          q.rx, (__attribute__((address_space(3))) void *)(dst + kHaloSlot * 16), 4, off, 0, 0, kNonTemporal);
    }
  };

  // ---- Weights and bias: coalesced loads first, then the DMA of the first
  // unit's first kPreStages stages, then the weights' trip through LDS, so
  // that the DMA latency overlaps it. Each output channel's 576 halves go on
  // a row of 1168 bytes (16 bytes of padding put the rows of 8 consecutive
  // channels on distinct banks). Fragment ks = 2t + h of lane (n16, g) holds
  // channels c0 .. c0+8 (c0 = 32h + 8g) of tap t for output channel
  // o = 16*og + n16: halves 9jj + t (jj = 0..7) of the 72 halves
  // w[o][c0 .. c0+8][0..3][0..3], 144 contiguous bytes of o's row, read as 9
  // 16-byte vectors per channel half and sorted in registers.
  UnitGeo geo = unit_geo(unit);
  half8 wa[18];
  float4v bias;
  {
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16 *>(a.w), (short)0, kK * kC * 9 * 2, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.bias), (short)0, a.bias ? kK * 4 : 0, kBufferFlags);
    constexpr int kVecRow = kC * 9 * 2 / 16;   // 72 vectors per output channel
    constexpr int kVecPerThread = kK * kVecRow / kThreads;
    static_assert(kVecPerThread * kThreads == kK * kVecRow, "whole vectors per thread");
    // The bias goes first: the waits for the weights then cover it, and no
    // wait for it is left to the loop (which would also wait for the DMA).
    bias = __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(rb, (16 * og + 4 * g) * 4, 0, 0));
    uint4v t[kVecPerThread];
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j)
      t[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, (j * kThreads + tid) * 16, 0, 0);
#pragma unroll
    for (int st = 0; st < kPreStages; ++st) issue_stage(geo, st);
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j) {
      const int v = j * kThreads + tid;
      const int o = v / kVecRow, r = v - o * kVecRow;
      *reinterpret_cast<uint4v *>(lds + kWStage + o * kWRow + r * 16) = t[j];
    }
  }
  lds_barrier();
  {
    const int o = 16 * og + n16;
    half8 raw[2][9];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 9; ++j)
        raw[h][j] = *reinterpret_cast<const half8 *>(lds + kWStage + o * kWRow + (32 * h + 8 * g) * 18 + 16 * j);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const int t = ks >> 1, h = ks & 1;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) wa[ks][jj] = raw[h][(9 * jj + t) / 8][(9 * jj + t) % 8];
    }
  }
  lds_barrier();   // the weights' LDS is ring space from here on
#pragma unroll
  for (int st = kPreStages; st < kD; ++st) issue_stage(geo, st);

  // Byte offsets (inside a row) of this lane's B reads for filter column v and
  // channel half h: pixel 16*ch + n16 + v - 1 of the row, chunk 4h + g.
  int boff[3][2];
#pragma unroll
  for (int v = 0; v < 3; ++v)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int px = 16 * ch + n16 + v - 1;
      const int c = 4 * h + g;
      const int slot = px < 0 ? kHaloSlot + c : (px >= kTC ? kHaloSlot + 8 + c : slot_in_row<SWZ>(px, c));
      boff[v][h] = slot * 16;
    }
  // Staging: output row r of a stage holds pixel px's 64 channels as 8 chunks,
  // chunk c at position c ^ (px % 8) so that both the fragment writes and the
  // line reads spread over the banks. This lane writes channels 16*og + 4g ..
  // +4 of pixel 16*ch + n16; it reads chunk sc of pixels spx and spx + 8.
  const int wpx = 16 * ch + n16;
  const int soff_w = kRingBytes + wpx * 128 + (((2 * og + (g >> 1)) ^ (wpx & 7)) * 16) + (g & 1) * 8;
  const int soff_r = kRingBytes + sr * kOutRowBytes + spx * 128 + ((sc ^ (spx & 7)) * 16);

  while (true) {
    // ---- Unit prologue: stages 0 .. kD-1 are in flight; the first two must
    // have landed before the first read.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(vm_after(1, -1)));
    lds_barrier();

    auto read_b = [&](int q) -> half8 {
      const int i = q / 6, v = (q % 6) >> 1, h = q & 1;
      const char *p = lds + ((i / kS) % kNst) * kStageBytes + (i % kS) * kRowBytes + boff[v][h];
      return *reinterpret_cast<const half8 *>(p);
    };
    // This wave's two 1 KB pieces of staged row sr of stage t, to registers
    // and then to HBM (output row t*kS + sr - 2 of the unit).
    auto read_staged = [&](int t, uint4v (&sv)[2]) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        sv[j] = *reinterpret_cast<const uint4v *>(lds + soff_r + (t & 1) * kS * kOutRowBytes + 8 * j * 128);
    };
    auto store_stage = [&](int t, const uint4v (&sv)[2]) {
      const int o = t * kS + sr - 2;
      const int gy = geo.y0 + o;
      const bool row_out = (o >= 0) & (o < kUR) & (gy < a.H);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const unsigned off =
            (row_out & (geo.scol[j] != kOob)) ? (unsigned)gy * pix_row_bytes + geo.scol[j] : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(sv[j], geo.ry, off, 0, kNonTemporal);
      }
    };

    constexpr int kAhead = 8;
    half8 ring[kAhead];
#pragma unroll
    for (int q = 0; q < kAhead; ++q) ring[q] = read_b(q);
    float4v acc[4];
    uint4v sv[2];
    static_for<kReads>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      constexpr int i = q / 6, v = (q % 6) >> 1, h = q & 1;
      constexpr int t = i / kS;                            // stage of input row i
      constexpr int qs = q % kReadsPerStage;               // read step inside the stage
      // Stage t - 1's rows leave for HBM; stage t + kD's rows start their DMA.
      if constexpr (t >= 1 && qs == 0) read_staged(t - 1, sv);
      if constexpr (t >= 1 && qs == 2) store_stage(t - 1, sv);
      if constexpr (t + kD < kStages && qs == 3) issue_stage(geo, t + kD);
      if constexpr (qs == 0 || qs == 2 || qs == 3) __builtin_amdgcn_sched_barrier(0);

      const half8 b = ring[q % kAhead];
      if constexpr (q + kAhead < kReads) ring[q % kAhead] = read_b(q + kAhead);
      if constexpr (v == 0 && h == 0 && i < kUR) acc[i & 3] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int o = i - u;
        if (o >= 0 && o < kUR) {
          const int ks = 2 * (3 * u + v) + h;
          acc[o & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[ks], b, acc[o & 3], 0, 0, 0);
        }
      }
      // The last read of input row i completes output row i - 2: bias, ReLU,
      // fp16 (nearest even), into stage t's staging rows.
      if constexpr (v == 2 && h == 1 && i >= 2 && i - 2 < kUR) {
        constexpr int o = i - 2;
        _Float16 hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float r = acc[o & 3][e] + bias[e];
          if (a.relu) r = fmaxf(r, 0.f);
          hv[e] = (_Float16)r;
        }
        *reinterpret_cast<uint2v *>(lds + soff_w + ((t & 1) * kS + (i % kS)) * kOutRowBytes) =
            __builtin_bit_cast(uint2v, hv);
      }
      // End of stage t: stage t + 2 (read from the next stage's last steps on,
      // through the read-ahead ring) must have landed; the barrier publishes it,
      // frees stage t's ring slot and completes stage t's staged rows.
      if constexpr (qs == kReadsPerStage - 1 || q == kReads - 1) {
        if constexpr (t + 2 < kStages) __builtin_amdgcn_s_waitcnt(waitcnt_vm(vm_after(t + 2, t)));
        lds_barrier();
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    read_staged(kStages - 1, sv);
    store_stage(kStages - 1, sv);

    unit += step;
    if (unit >= hi) break;
    // The next unit's first kD stages go out now: their ring slots were freed
    // by this unit's last barrier, and the next unit's first barrier comes
    // after this unit's last staging reads.
    geo = unit_geo(unit);
#pragma unroll
    for (int t = 0; t < kD; ++t) issue_stage(geo, t);
  }
}

}  // namespace

bool configure_mfma(Plan &p) {
  const conv2d_desc &d = p.d;
  if (d.layout != IS_NHWC || d.in_dtype != IS_F16 || d.out_dtype != IS_F16) return false;
  if (d.c != kC || d.k != kK || d.r != 3 || d.s != 3) return false;
  if (2.0 * d.h * (double)d.w * kC >= 4.0e9) return false;   // 32-bit offsets per image
  const long long units = (long long)((d.w + kTC - 1) / kTC) * ((d.h + kUR - 1) / kUR) * d.n;
  if (units > (1LL << 31) - 1) return false;
  p.kid = kMfmaNhwcF16;
  p.name = "is_k4_mfma";
  p.nseg = (d.w + kTC - 1) / kTC;
  p.nstrip = (d.h + kUR - 1) / kUR;
  p.ntiles = (int)units;
  // Persistent: one workgroup per CU (its LDS and registers fill the CU),
  // 8 XCDs x 32 CUs; fewer when there are fewer units (kept a multiple of 8).
  int g = 256;
  while (g > 8 && g / 2 >= p.ntiles) g /= 2;
  p.grid_x = g;
  p.grid_y = p.grid_z = 1;
  p.block = kThreads;
  p.lds = kLdsBytes;
  p.tile_w = kTC;
  p.tile_h = kUR;
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
  a.units_x = p.nseg;
  a.units_y = p.nstrip;
  a.nunits = p.ntiles;
  switch (p.vec) {
    case 0: return launch_kernel(is_k4_mfma<0>, dim3(p.grid_x), dim3(p.block), 0, s, a);
    case 128: return launch_kernel(is_k4_mfma<128>, dim3(p.grid_x), dim3(p.block), 0, s, a);
    default: return launch_kernel(is_k4_mfma<256>, dim3(p.grid_x), dim3(p.block), 0, s, a);
  }
}

}  // namespace is
