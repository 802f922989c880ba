// k3_chain.hip -- the upscaling chain fused into one kernel:
//   conv 5x5 1->32, conv 3x3 32->32, conv 3x3 32->32, conv 3x3 32->4 (fp32,
//   ReLU as requested per layer), then depth-to-space x2.
//
// The network is the one of "Optimizing convolution kernels - CNNs in Vulkan
// Part 2/3" (StreamHPC; introduction and the layer table of "Reducing memory
// traffic"), scaled to 32 channels. The fusion follows "Model-Based Warp
// Overlapped Tiling for Image Processing Programs on GPUs" (arXiv 1909.07190,
// abstract): overlapped tiles, loop fusion across the stages, intermediates kept
// on chip in a mix of registers and shared memory. Here:
//  * a workgroup owns a 64-column window and sweeps a block of rows down the
//    image four rows at a time. Every layer is evaluated on all 64 columns;
//    validity shrinks by the filter radius per layer, and the 56 middle columns
//    are kept, so neighbouring windows overlap by 8 columns (the recomputed
//    halo). There is no vertical recomputation except a two-step warm-up at the
//    top of each block: each intermediate layer keeps a ring of its last six
//    output rows (all 32 channels, fp32) in LDS, which is all that the next
//    layer's 3x3 window needs for four new rows;
//  * the two 32 -> 32 layers (90% of the FLOPs) run on the fp32 matrix cores
//    (v_mfma_f32_16x16x4_f32, as in the fp32 MFMA layer kernel): each wave owns
//    16 output channels of one of the four step rows, reads one LDS float per
//    lane per (tap, channel quad, 16-column block) and keeps the weights of both
//    layers in registers;
//  * the 5x5 1 -> 32 layer and the 3x3 32 -> 4 layer stay on the vector ALUs:
//    a lane holds 4 contiguous pixels x 4 channels of one row, reads one
//    16-byte LDS vector per input channel and filter row and takes its
//    left/right neighbours by DPP row shifts, as in the multi-channel kernel;
//  * only the input frame is read from HBM and only the depth-to-space output
//    is written: two 16-byte stores per lane and output row pair.
#include "common.hpp"
#include "internal.hpp"

namespace is {
namespace {

constexpr int kWin = 64;            // columns evaluated per window
constexpr int kKeep = 56;           // columns kept: window columns [4, 60)
constexpr int kRows = 4;            // rows per pipeline step
constexpr int kThreads = 512;       // 8 waves
constexpr int kCh = 32;             // channels of the intermediate layers
constexpr int kRing = 6;            // rows held per intermediate ring
constexpr int kInRing = 12;         // input rows held: 8 in use + 4 arriving
constexpr int kInG = kWin / 4 + 2;  // 16-byte vectors per input row: x0-4 .. x0+67
constexpr int kG = kWin / 4;        // 16-byte vectors per intermediate row
constexpr unsigned kOob = 0xFFFFFFF0u;

constexpr int kDppRowShr1 = 0x111;  // lane reads lane-1 inside its row of 16
constexpr int kDppRowShl1 = 0x101;  // lane reads lane+1 inside its row of 16

__device__ __forceinline__ float row_prev(float src, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), kDppRowShr1,
                                                    0xf, 0xf, false));
}
__device__ __forceinline__ float row_next(float src, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), kDppRowShl1,
                                                    0xf, 0xf, false));
}

typedef float float4v __attribute__((ext_vector_type(4)));

// Intermediate rings hold, per row slot and channel, the 64 window columns as
// 16 float4 vectors (one channel row = 256 bytes = the 64 LDS banks of 4
// bytes); channel c is stored rotated by 4 * (c mod 4) vectors (16 floats) so
// that the four channels of a quad, which one MFMA operand load reads 16
// floats each, land on four disjoint quarters of the banks. Vector lc of
// channel c:
__device__ __forceinline__ int rot4(int c, int lc) { return (lc + 4 * (c & 3)) & 15; }

// The input ring: per row slot, the window's own 16 vectors (x0 .. x0+63,
// rows 256 bytes apart, so that the 4 rows of a read are served without bank
// conflicts) and, after all of those, the slot's 2 halo vectors (x0-4 .. x0-1
// and x0+64 .. x0+67). Vector g of slot s, g = 0 .. kInG-1 counting from x0-4:
constexpr int kInMain = kWin / 4;
constexpr int kInHaloBase = kInRing * kInMain;
__device__ __forceinline__ int in_idx(int s, int g) {
  return (g >= 1 && g <= kInMain) ? s * kInMain + g - 1 : kInHaloBase + 2 * s + (g != 0);
}

struct ChainArgs {
  const float *x;
  const float *w[4];
  const float *b[4];
  float *y;
  int H, W, relu_mask;
  int nstrip, nblock, block_rows, ntiles;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const float *p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), (short)0, (int)bytes, kBufferFlags);
}

__device__ __forceinline__ float4 ld4(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// The 9 taps of one (output channel, input channel) pair: 36 contiguous bytes
// starting 4*s bytes past a 16-byte boundary `base`. Three aligned 16-byte loads
// cover them (the last may run past the weights and then reads 0); s folds to a
// constant at every call once the channel loop is unrolled.
__device__ __forceinline__ void load_taps9(__amdgpu_buffer_rsrc_t r, unsigned base, int s, float *t) {
  float v[12];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const float4 q = ld4(r, base + 16 * i);
    v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
  }
#pragma unroll
  for (int i = 0; i < 9; ++i) t[i] = v[s + i];
}

// 16-byte aligned byte offset of the taps of (output channel o, input channel c)
// in a K x 32 x 3 x 3 weight tensor; the taps start (c mod 4) floats later.
__device__ __forceinline__ unsigned taps_base(int o, int c) {
  return (unsigned)(o * kCh * 36 + 36 * c - 4 * (c & 3));
}

// 3x3 window rows of input channel c for the lane's 4 pixels: one LDS vector
// per filter row, neighbours by DPP (zero beyond the window edge).
__device__ __forceinline__ void window3(const float4 *src, const int (&slot)[3], int c, int lc,
                                        float (&win)[3][6]) {
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const float4 o = src[(slot[u] * kCh + c) * kG + rot4(c, lc)];
    win[u][1] = o.x; win[u][2] = o.y; win[u][3] = o.z; win[u][4] = o.w;
    win[u][0] = row_prev(o.w, 0.f);
    win[u][5] = row_next(o.x, 0.f);
  }
}

__global__ __launch_bounds__(kThreads) void is_k3_chain(ChainArgs a) {
  __shared__ float4 in_ring[kInRing * kInG];
  __shared__ float4 ring[3][kRing * kCh * kG];
  __shared__ float l4buf[4 * kRows * kWin];
  lds_poison(in_ring, sizeof(in_ring));
  lds_poison(ring, sizeof(ring));
  lds_poison(l4buf, sizeof(l4buf));

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int lr = lane >> 4;   // row inside a 4-row step
  const int lc = lane & 15;   // 4-column group inside the window

  const int tile = xcd_remap(blockIdx.x, a.ntiles);
  const int sx = tile % a.nstrip;
  const int by = (tile / a.nstrip) % a.nblock;
  const int n = tile / (a.nstrip * a.nblock);
  const int H = a.H, W = a.W;
  const int xw = sx * kKeep - 4;                // window column 0
  const int y0 = by * a.block_rows;
  const int yend = min(y0 + a.block_rows, H);
  const int t0 = y0 - 8;                        // two warm-up steps
  const int nsteps = 2 + (yend - y0 + kRows - 1) / kRows;
  const size_t HW = (size_t)H * W;

  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x + (size_t)n * HW, (unsigned)(HW * 4));
  const __amdgpu_buffer_rsrc_t ry = rsrc(a.y + (size_t)n * 4 * HW, (unsigned)(4 * HW * 4));
  const __attribute__((address_space(4))) float *w0c = (const __attribute__((address_space(4))) float *)a.w[0];
  const __amdgpu_buffer_rsrc_t rw3 = rsrc(a.w[3], 4 * 32 * 9 * 4);

  // Byte offset of input vector q (row slot q/kInG of a 4- or 8-row batch
  // starting at image row r0, 16-byte group q%kInG of the window).
  auto in_off = [&](int r0, int q) -> unsigned {
    const int r = r0 + q / kInG;
    const int col = xw - 4 + 4 * (q % kInG);
    const bool in = r >= 0 && r < H && col >= 0 && col < W;
    return in ? (unsigned)(((size_t)r * W + col) * 4) : kOob;
  };
  auto in_slot = [&](int r) { return (r - t0 - 1) % kInRing; };

  // Input rows t0+1 .. t0+8 before the first step.
  for (int q = tid; q < 8 * kInG; q += kThreads) in_ring[in_idx(q / kInG, q % kInG)] = ld4(rx, in_off(t0 + 1, q));

  // MFMA layers: lane (g4, n16) holds, for filter tap t and channel quad cq,
  // the weight of output channel 16*mob + n16 and input channel 4*cq + g4.
  const int mob = wave & 1, mrow = wave >> 1;
  const int n16 = lane & 15, g4 = lane >> 4;
  float wm[2][9 * (kCh / 4)];
  float bm[2];
#pragma unroll
  for (int l = 0; l < 2; ++l) {
    const float *wp = a.w[l + 1] + ((size_t)(16 * mob + n16) * kCh + g4) * 9;
#pragma unroll
    for (int tp = 0; tp < 9; ++tp)
#pragma unroll
      for (int cq = 0; cq < kCh / 4; ++cq) wm[l][tp * (kCh / 4) + cq] = wp[cq * 4 * 9 + tp];
    bm[l] = a.b[l + 1] ? a.b[l + 1][16 * mob + n16] : 0.f;
  }

  const int gcol = xw + 4 * lc;                 // first image column of the lane's pixels
  const bool col_in = gcol >= 0 && gcol < W;
  const int f0 = wave * 4;                      // first output channel of this wave
  __syncthreads();

  for (int k = 0; k < nsteps; ++k) {
    const int t = t0 + kRows * k;

    // Input rows for the next step, written to the ring at the end of this one.
    float4 pre = make_float4(0.f, 0.f, 0.f, 0.f);
    const bool do_pre = tid < 4 * kInG && k + 1 < nsteps;
    if (do_pre) pre = ld4(rx, in_off(t + 9, tid));

    // ---- Layer 1: 5x5, 1 -> 32, rows t+3 .. t+6, channels f0 .. f0+3.
    {
      const int row = t + 3 + lr;
      float acc[4][4];
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[f][p] = 0.f;
#pragma unroll
      for (int u = 0; u < 5; ++u) {
        const int rs = in_slot(row + u - 2);
        const float4 o = in_ring[in_idx(rs, lc + 1)];
        const float4 h = in_ring[in_idx(rs, lc == 15 ? kInG - 1 : 0)];
        float win[8];
        win[2] = o.x; win[3] = o.y; win[4] = o.z; win[5] = o.w;
        win[1] = row_prev(o.w, h.w);
        win[0] = row_prev(o.z, h.z);
        win[6] = row_next(o.x, h.x);
        win[7] = row_next(o.y, h.y);
        // Taps of this filter row for the wave's 4 channels: scalar loads (the
        // empty asm keeps them from being hoisted out of the u loop).
        float tap[4][5];
        int toff = f0 * 25 + u * 5;
        asm volatile("" : "+s"(toff));
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
          for (int v = 0; v < 5; ++v) tap[f][v] = w0c[toff + f * 25 + v];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
          for (int v = 0; v < 5; ++v)
#pragma unroll
            for (int p = 0; p < 4; ++p) acc[f][p] = __builtin_fmaf(tap[f][v], win[p + v], acc[f][p]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool keep = col_in && row >= 0 && row < H;
      const bool relu = a.relu_mask & 1;
      float4 *dst = ring[0] + ((row - t0) % kRing) * kCh * kG;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const float bb = a.b[0] ? a.b[0][f0 + f] : 0.f;
        float o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          o[p] = acc[f][p] + bb;
          if (relu) o[p] = fmaxf(o[p], 0.f);
          if (!keep) o[p] = 0.f;
        }
        dst[(f0 + f) * kG + rot4(f0 + f, lc)] = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
    __syncthreads();

    // ---- Layers 2 and 3: 3x3, 32 -> 32 (rows t+2.. and t+1..) on the fp32
    // matrix cores, skipped while their inputs are still warming up. Wave w
    // computes output channels 16*(w&1) .. +16 of step row w>>1 for the four
    // 16-column blocks of the window: A = 16 pixels x 4 channels of one tap
    // (one LDS float per lane), B = 4 channels x 16 output channels (weights in
    // registers), D = 4 consecutive pixels of one output channel per lane,
    // written back to the next ring as one float4. The window's edge columns
    // read a neighbouring column of the same ring row instead of 0; they only
    // reach window columns 0..2 and 61..63 of the last layer, outside the kept
    // 4..59.
    for (int l = 1; l <= 2; ++l) {
      if (k >= 1) {
        const float *src = reinterpret_cast<const float *>(ring[l - 1]);
        const float *wl = wm[l - 1];
        const int row = t + 3 - l + mrow;
        float4v acc[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[cb] = float4v{0.f, 0.f, 0.f, 0.f};
        // Float offset of the lane's A element for filter row u, tap column v
        // and column block cb (channel quad 0); quad cq adds 4 * kWin * cq.
        int aoff[3][3][4];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          const int base = ((row - 1 + u - t0) % kRing * kCh + g4) * kWin;
#pragma unroll
          for (int v = 0; v < 3; ++v)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) aoff[u][v][cb] = base + ((16 * cb + n16 + v - 1 + 16 * g4) & 63);
        }
        constexpr int kSteps = 9 * (kCh / 4) * 4;   // (tap, channel quad, column block)
        constexpr int kAhead = 16;
        auto read_a = [&](int q) -> float {
          const int tq = q / 4, cb = q % 4, tp = tq / 8, cq = tq % 8;
          return src[aoff[tp / 3][tp % 3][cb] + cq * 4 * kWin];
        };
        float ra[kAhead];
#pragma unroll
        for (int q = 0; q < kAhead; ++q) ra[q] = read_a(q);
        static_for<kSteps>([&](auto qc) __attribute__((always_inline)) {
          constexpr int q = decltype(qc)::value;
          const float av = ra[q % kAhead];
          if constexpr (q + kAhead < kSteps) ra[q % kAhead] = read_a(q + kAhead);
          constexpr int tq = q / 4, cb = q % 4;
          acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, wl[tq], acc[cb], 0, 0, 0);
        });
        const bool row_in = row >= 0 && row < H;
        const bool relu = (a.relu_mask >> l) & 1;
        const int c = 16 * mob + n16;
        float4 *dst = ring[l] + ((row - t0) % kRing) * kCh * kG + c * kG;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int gc = xw + 16 * cb + 4 * g4;   // image column of the lane's first pixel
          const bool keep = row_in && gc >= 0 && gc < W;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = acc[cb][e] + bm[l - 1];
            if (relu) o[e] = fmaxf(o[e], 0.f);
            if (!keep) o[e] = 0.f;
          }
          dst[rot4(c, 4 * cb + g4)] = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
      __syncthreads();
    }

    // ---- Layer 4: 3x3, 32 -> 4, rows t .. t+3; wave w < 4 computes channel w.
    if (k >= 2 && wave < 4) {
      const int o = wave;
      const int row = t + lr;
      int slot[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) slot[u] = (row - 1 + u - t0) % kRing;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int c4 = 0; c4 < kCh; c4 += 4) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const int c = c4 + cc;
          float tap[9];
          load_taps9(rw3, taps_base(o, c), cc, tap);
          float win[3][6];
          window3(ring[2], slot, c, lc, win);
#pragma unroll
          for (int u = 0; u < 3; ++u)
#pragma unroll
            for (int v = 0; v < 3; ++v)
#pragma unroll
              for (int p = 0; p < 4; ++p) acc[p] = __builtin_fmaf(tap[u * 3 + v], win[u][p + v], acc[p]);
        }
      }
      const float bb = a.b[3] ? a.b[3][o] : 0.f;
      const bool relu = (a.relu_mask >> 3) & 1;
      float out[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        out[p] = acc[p] + bb;
        if (relu) out[p] = fmaxf(out[p], 0.f);
      }
      *reinterpret_cast<float4 *>(&l4buf[(o * kRows + lr) * kWin + 4 * lc]) =
          make_float4(out[0], out[1], out[2], out[3]);
    }
    __syncthreads();

    // ---- Depth-to-space x2: wave w writes output row 2*(t + w/2) + w%2; lane
    // q < 28 writes the 16 bytes of pixel pair (4 + 2q, 5 + 2q) of the window.
    if (k >= 2) {
      const int i = t + (wave >> 1);
      const int dy = wave & 1;
      const int q = lane;
      if (q < kKeep / 2 && i >= y0 && i < yend) {
        const int j0 = 4 + 2 * q;                 // window column of the pair
        const int gj = xw + j0;                   // image column (even)
        const float *z0 = &l4buf[((2 * dy) * kRows + (wave >> 1)) * kWin];
        const float *z1 = &l4buf[((2 * dy + 1) * kRows + (wave >> 1)) * kWin];
        const float4 v = make_float4(z0[j0], z1[j0], z0[j0 + 1], z1[j0 + 1]);
        const unsigned off =
            gj < W ? (unsigned)(((size_t)(2 * i + dy) * (2 * W) + 2 * gj) * 4) : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v),
                                               ry, off, 0, 0);
      }
    }

    if (do_pre) in_ring[in_idx(in_slot(t + 9) + tid / kInG, tid % kInG)] = pre;
    __syncthreads();
  }
}

}  // namespace

bool chain_fused_supported(const conv_chain_desc *d) {
  if (!d || d->n_layers != 4 || d->depth_to_space != 2 || d->dtype != IS_F32) return false;
  const conv_layer_desc *L = d->layer;
  if (!(L[0].c == 1 && L[0].k == 32 && L[0].r == 5 && L[0].s == 5)) return false;
  for (int l = 1; l <= 2; ++l)
    if (!(L[l].c == 32 && L[l].k == 32 && L[l].r == 3 && L[l].s == 3)) return false;
  if (!(L[3].c == 32 && L[3].k == 4 && L[3].r == 3 && L[3].s == 3)) return false;
  if (d->w % 4 != 0 || d->h < 1 || d->w < 1 || d->n < 1) return false;
  // 32-bit buffer offsets: one output image (4 H W floats) under 4 GB.
  if (16.0 * d->h * (double)d->w >= 4.0e9) return false;
  return true;
}

hipError_t launch_chain_fused(const conv_chain_desc *d, const float *x, const float *const *w,
                              const float *const *b, float *y, hipStream_t s) {
  ChainArgs a;
  a.x = x;
  for (int l = 0; l < 4; ++l) {
    a.w[l] = w[l];
    a.b[l] = b ? b[l] : nullptr;
  }
  a.y = y;
  a.H = d->h;
  a.W = d->w;
  a.relu_mask = 0;
  for (int l = 0; l < 4; ++l) a.relu_mask |= (d->layer[l].relu ? 1 : 0) << l;
  a.nstrip = (d->w + kKeep - 1) / kKeep;
  // About one workgroup per CU: split each strip into blocks of rows so that
  // strips x blocks x images fills the device's CUs once.
  const int cus = device_cu_count();
  const int per_img = a.nstrip * d->n;
  int nb = per_img >= cus ? 1 : cus / per_img;
  if (nb < 1) nb = 1;
  int rows = (d->h + nb - 1) / nb;
  rows = (rows + kRows - 1) / kRows * kRows;
  a.block_rows = rows;
  a.nblock = (d->h + rows - 1) / rows;
  const long long tiles = (long long)a.nstrip * a.nblock * d->n;
  if (tiles > (1LL << 31) - 1) return hipErrorInvalidValue;
  a.ntiles = (int)tiles;
  return launch_kernel(is_k3_chain, dim3(a.ntiles), dim3(kThreads), 0, s, a);
}

}  // namespace is
