// k2_multi.hip -- multi-channel fp32 NCHW layer, square odd filters r = s in {1, 3, 5}
// (and 7 in the matrix-core form at the end of the file).
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

typedef float float4v __attribute__((ext_vector_type(4)));

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (and nothing else).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

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

// Per-lane byte offsets of this lane's DMA vectors inside a slab (the same
// for every slab: the resource base moves instead). Vectors outside the image
// and the padding past the slab read 0.
template <int R, int CS>
__device__ __forceinline__ void slab_offsets(unsigned *voff, int wave, int lane, int x0, int y0, int H, int W,
                                             size_t HW) {
  using G = Geo<R, CS>;
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
    const int gy = y0 - G::P + lrow;
    const int gx = x0 - 4 + 4 * g;
    const bool in = q < G::V4 && gy >= 0 && gy < H && gx >= 0 && gx < W;
    voff[j] = in ? (unsigned)(((size_t)c * HW + (size_t)gy * W + gx) * 4) : kOob;
  }
}

// Epilogue: bias, ReLU, 16-byte stores (dropped outside the image). acc[f][p]
// is this lane's sum for filter kg * FT + f at output pixel (oy, ox + p);
// filters from K on (a last group of the matrix-core form that K does not
// fill) have no bias and their stores fall outside the output's range.
template <int FT, bool RELU, bool D2S, bool VEC = true>
__device__ __forceinline__ void store_tile(const float (&acc)[FT][4], const float *bias, float *y, int n,
                                           int kg, int K, int H, int W, int oy, int ox) {
  const size_t HW = (size_t)H * W;
  const bool in = oy < H && ox < W;
  const int kv = min(FT, K - kg * FT);   // filters of this group that exist
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
      yn, (short)0, (int)(kv * HW * 4), kBufferFlags);
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    const float b = (bias && f < kv) ? bias[kg * FT + f] : 0.f;
    float o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      o[p] = acc[f][p] + b;
      if constexpr (RELU) o[p] = fmaxf(o[p], 0.f);
    }
    if constexpr (VEC) {
      const unsigned off = in ? (unsigned)(((size_t)f * HW + (size_t)oy * W + ox) * 4) : kOob;
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, make_float4(o[0], o[1], o[2], o[3])),
          rs_o, off, 0, kNonTemporalStore);
    } else {
      // Rows that are not whole vectors: one dword per pixel inside the row.
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const unsigned off =
            (oy < H && ox + p < W) ? (unsigned)(((size_t)f * HW + (size_t)oy * W + ox + p) * 4) : kOob;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, o[p]), rs_o, off, 0,
                                              kNonTemporalStore);
      }
    }
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

  unsigned voff[G::ROUNDS];
  slab_offsets<R, CS>(voff, wave, lane, x0, y0, H, W, HW);

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

  store_tile<FT, RELU, D2S>(acc, bias, y, n, kg, K, H, W, y0 + row0, x0 + 4 * lc);
}

// ---- The matrix-core path --------------------------------------------------
//
// The same tiles, slabs and row windows with the products on the fp32 matrix
// cores, for 4 filters per workgroup. v_mfma_f32_4x4x1_16b_f32 multiplies, in
// each of 16 blocks of 4 lanes, a 4-vector A by a 4-vector B into a 4 x 4
// accumulator: lane 4b + i gives A[b][i] and B[b][i] and holds D[b][0..3][i].
// A is one tap of the 4 filters (lane i gives filter i mod 4's tap) and B the
// pixel the lane owns, so every lane accumulates its own pixel for all 4
// filters: one instruction per input channel, tap and pixel column of the
// lane's 4, each accumulation a single-rounding fma, in the vector path's
// order (channel, then filter row, then column), so both paths give the same
// bits. Per tap it issues at the matrix cores' full fp32 rate, twice the
// vector ALUs' fma rate.
//
// The layer moves 36 bytes per output pixel for 288 fmas, so once the products
// are this cheap the input stream decides the time, and one slab in flight per
// workgroup (the vector path's double buffer) leaves HBM idle between slabs.
// Here slabs of CS channels go through a ring of NB LDS buffers with NB - 1
// slabs in flight and one workgroup barrier per slab. Each slab brings its taps
// after its pixels ([channel][filter][tap], rows of TP taps padded with zeros
// to 16 bytes), by dword DMA. Every wave issues the same number of DMA
// instructions per slab (chunks past the data write zeros into the padding),
// so a slab's arrival is a fixed count of outstanding vector-memory operations.
template <int R, int CS>
struct MGeo {
  using G = Geo<R, CS>;
  static constexpr int TP = (R * R + 3) / 4 * 4;        // taps per (channel, filter)
  static constexpr int WUSED = CS * 4 * TP;             // tap dwords of a slab
  static constexpr int WROUNDS = (WUSED + 255) / 256;   // dword chunks per wave
  static constexpr int PIXV4 = G::PADV4;                // pixel vectors per buffer
  static constexpr int BUFV4 = PIXV4 + WROUNDS * 64;    // + WROUNDS x 4 x 64 dwords
  static constexpr int IPW = G::ROUNDS + WROUNDS;       // DMA instructions per wave per slab
  // Rows that are not whole 16-byte vectors (W % 4 != 0): the pixels move one
  // dword per lane, so that each pixel outside the image reads 0 on its own.
  // Instruction i writes LDS floats 64 i .. 64 i + 63: first one per staged
  // row (its 64 own columns), then the halo area (8 floats per row) in pieces
  // of 64; every wave issues DROUNDS of them (the last ones into padding).
  static constexpr int DMAIN = CS * G::LH;                       // one per staged row
  static constexpr int DHALO = (CS * G::LH * 8 + 63) / 64;
  static constexpr int DROUNDS = (DMAIN + DHALO + 3) / 4;
  static constexpr int IPW_D = DROUNDS + WROUNDS;
  static_assert(DROUNDS * 4 * 16 <= PIXV4, "the dword DMA stays in the pixel area");
};

// One slab into one ring buffer: every wave issues G::ROUNDS pixel chunks and
// WROUNDS tap chunks.
template <int R, int CS>
__device__ __forceinline__ void issue_ring_slab(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rw, float4 *buf,
                                                int wave, const unsigned *voff, const unsigned *wvoff) {
  using G = Geo<R, CS>;
  using M = MGeo<R, CS>;
#pragma unroll
  for (int j = 0; j < G::ROUNDS; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(buf + (j * 4 + wave) * 64),
                                             16, voff[j], 0, 0, 0);
#pragma unroll
  for (int j = 0; j < M::WROUNDS; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rw, (__attribute__((address_space(3))) void *)((float *)(buf + M::PIXV4) + (j * 4 + wave) * 64), 4,
        wvoff[j], 0, 0, 0);
}

// NSL: the slab count C / CS when known at compile time (0: any).
// The same with the pixels as dwords (rows that are not whole vectors).
template <int R, int CS>
__device__ __forceinline__ void issue_ring_slab_d(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rw,
                                                  float4 *buf, int wave, const unsigned *doff,
                                                  const unsigned *wvoff) {
  using M = MGeo<R, CS>;
#pragma unroll
  for (int j = 0; j < M::DROUNDS; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void *)((float *)buf + (j * 4 + wave) * 64), 4, doff[j], 0, 0, 0);
#pragma unroll
  for (int j = 0; j < M::WROUNDS; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rw, (__attribute__((address_space(3))) void *)((float *)(buf + M::PIXV4) + (j * 4 + wave) * 64), 4,
        wvoff[j], 0, 0, 0);
}

// VEC: W % 4 == 0 (16-byte pixel groups and stores); else dwords.
template <int R, int CS, int NB, int NSL, bool RELU, bool D2S, bool VEC = true>
__global__ __launch_bounds__(kThreads) void is_k2_multi_mfma(const float *__restrict__ x,
                                                             const float *__restrict__ w,
                                                             const float *__restrict__ bias,
                                                             float *__restrict__ y, int C, int H, int W, int K,
                                                             int ntx, int nty, int nkg, int ntiles) {
  using G = Geo<R, CS>;
  using M = MGeo<R, CS>;
  constexpr int P = G::P;
  constexpr int TQ = M::TP / 4;
  constexpr int PD = NB - 1;   // slabs in flight ahead of the one computed
  // The ring's buffers are separate arrays so that the compiler can tell a
  // slab's LDS reads from the DMA still writing the other buffers (one array
  // indexed by slab would make every LDS read wait for all DMA in flight).
  static_assert(NB == 4, "four ring buffers");
  __shared__ float4 ring0[M::BUFV4], ring1[M::BUFV4], ring2[M::BUFV4], ring3[M::BUFV4];
  lds_poison(ring0, sizeof(ring0));
  lds_poison(ring1, sizeof(ring1));
  lds_poison(ring2, sizeof(ring2));
  lds_poison(ring3, sizeof(ring3));

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane >> 4;
  const int lc = lane & 15;

  const int tile = xcd_remap(blockIdx.x, ntiles);
  const int tx = tile % ntx;
  const int ty = (tile / ntx) % nty;
  const int kg = (tile / (ntx * nty)) % nkg;
  const int n = tile / (ntx * nty * nkg);
  const int x0 = tx * kTW, y0 = ty * kTH;
  const size_t HW = (size_t)H * W;

  static_assert(VEC || !D2S, "the depth-to-space stores are 16-byte vectors");
  constexpr int IPW = VEC ? M::IPW : M::IPW_D;   // DMA operations per wave and slab
  static_assert((PD - 1) * IPW < 64, "vmcnt field");
  unsigned voff[VEC ? G::ROUNDS : M::DROUNDS];
  if constexpr (VEC) {
    slab_offsets<R, CS>(voff, wave, lane, x0, y0, H, W, HW);
  } else {
#pragma unroll
    for (int j = 0; j < M::DROUNDS; ++j) {
      const int ins = j * 4 + wave;
      int c = 0, lrow = 0, gx = -1;
      if (ins < M::DMAIN) {
        c = ins / G::LH;
        lrow = ins - c * G::LH;
        gx = x0 + lane;
      } else {
        const int h = (ins - M::DMAIN) * 64 + lane;   // float of the halo area
        if (h < CS * G::LH * 8) {
          const int crow = h >> 3, j8 = h & 7;
          c = crow / G::LH;
          lrow = crow - c * G::LH;
          gx = j8 < 4 ? x0 - 4 + j8 : x0 + kTW + j8 - 4;
        }
      }
      const int gy = y0 - P + lrow;
      const bool in = gx >= 0 && gx < W && gy >= 0 && gy < H;
      voff[j] = in ? (unsigned)(((size_t)c * HW + (size_t)gy * W + gx) * 4) : kOob;
    }
  }
  // This lane's tap dwords in a slab: filter f of the group, channel c of the
  // slab, tap t; relative to the slab's first channel of the group's first
  // filter. Padding taps and chunks read 0.
  unsigned wvoff[M::WROUNDS];
#pragma unroll
  for (int j = 0; j < M::WROUNDS; ++j) {
    const int e = (j * 4 + wave) * 64 + lane;
    const int c = e / (4 * M::TP), f = (e / M::TP) % 4, t = e % M::TP;
    wvoff[j] = (e < M::WUSED && t < R * R) ? (unsigned)((((size_t)f * C + c) * R * R + t) * 4) : kOob;
  }

  const float *xn = x + (size_t)n * C * HW;
  const float *wg = w + (size_t)kg * 4 * C * R * R;
  const size_t w_left = (size_t)(K - kg * 4) * C * R * R;   // dwords from wg to the end of w
  auto issue = [&](int s, float4 *buf) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(xn + (size_t)s * CS * HW), (short)0, (int)(CS * HW * 4), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(wg + (size_t)s * CS * R * R), (short)0,
        (int)((w_left - (size_t)s * CS * R * R) * 4), kBufferFlags);
    if constexpr (VEC)
      issue_ring_slab<R, CS>(rs, rw, buf, wave, voff, wvoff);
    else
      issue_ring_slab_d<R, CS>(rs, rw, buf, wave, voff, wvoff);
  };

  const int row0 = wave * 4 + lr;
  const int halo_g = lc == 15 ? 1 : 0;
  float4v macc[4];   // macc[p][f]: pixel column p, filter f
#pragma unroll
  for (int p = 0; p < 4; ++p) macc[p] = float4v{0.f, 0.f, 0.f, 0.f};

  // One slab: per channel, the R row windows as on the vector path and the
  // taps of filter lane mod 4 (16-byte reads); the next channel's LDS reads
  // are issued before this channel's products.
  auto compute = [&](const float4 *bf) __attribute__((always_inline)) {
    const float4 *wl = bf + M::PIXV4 + (lane & 3) * TQ;
    float4 raw_o[2][R], raw_h[2][R], raw_w[2][TQ];
    auto read_raw = [&](int c, int b) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int crow = c * G::LH + row0 + u;
        raw_o[b][u] = bf[crow * kMainG + lc];
        if constexpr (P > 0) raw_h[b][u] = bf[G::MAINV4 + crow * 2 + halo_g];
      }
#pragma unroll
      for (int q = 0; q < TQ; ++q) raw_w[b][q] = wl[c * 4 * TQ + q];
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
      float tap[4 * TQ];
#pragma unroll
      for (int q = 0; q < TQ; ++q) {
        const float4 t4 = raw_w[c & 1][q];
        tap[4 * q] = t4.x; tap[4 * q + 1] = t4.y; tap[4 * q + 2] = t4.z; tap[4 * q + 3] = t4.w;
      }
      if (c + 1 < CS) read_raw(c + 1, (c + 1) & 1);
#pragma unroll
      for (int u = 0; u < R; ++u)
#pragma unroll
        for (int v = 0; v < R; ++v)
#pragma unroll
          for (int p = 0; p < 4; ++p)
            macc[p] = __builtin_amdgcn_mfma_f32_4x4x1f32(tap[u * R + v], win[u][p + v], macc[p], 0, 0, 0);
    }
  };

  // Wait until this wave's part of slab s has landed, with `ahead` later slabs
  // still allowed in flight.
  static_assert(PD <= 4, "wait_slab's cases");
  auto wait_slab = [&](int ahead) __attribute__((always_inline)) {
    if (ahead == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if constexpr (PD > 1) if (ahead == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(1 * IPW));
    if constexpr (PD > 2) if (ahead == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * IPW));
    if constexpr (PD > 3) if (ahead == 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * IPW));
  };

  const int nslab = NSL > 0 ? NSL : C / CS;
  float4 *const bufs[4] = {ring0, ring1, ring2, ring3};
  if (nslab > 0) issue(0, ring0);
  if (nslab > 1) issue(1, ring1);
  if (nslab > 2) issue(2, ring2);
  // Slab s sits in buffer s mod 4; slab s + 3 goes into the buffer of slab s - 1.
  auto step = [&](int s, float4 *cur, float4 *next) __attribute__((always_inline)) {
    wait_slab(min(PD - 1, nslab - 1 - s));
    // Every wave's part of slab s is in LDS, and every wave is done with slab
    // s - 1, whose buffer slab s + PD takes next; the later slabs' DMA stays
    // in flight across the barrier.
    lds_barrier();
    if (s + PD < nslab) issue(s + PD, next);
    compute(cur);
  };
  if constexpr (NSL > 0) {
    // A known slab count unrolls the whole channel loop. The compiler then sees
    // which buffer every LDS read and DMA touches and waits only for the slab a
    // read needs; around a loop's back edge it would wait for all DMA in flight.
#pragma unroll
    for (int s = 0; s < NSL; ++s) step(s, bufs[s & 3], bufs[(s + 3) & 3]);
  } else {
    for (int s = 0; s < nslab; s += 4) {
      step(s, ring0, ring3);
      if (s + 1 < nslab) step(s + 1, ring1, ring0);
      if (s + 2 < nslab) step(s + 2, ring2, ring1);
      if (s + 3 < nslab) step(s + 3, ring3, ring2);
    }
  }

  float acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[f][p] = macc[p][f];
  store_tile<4, RELU, D2S, VEC>(acc, bias, y, n, kg, K, H, W, y0 + row0, x0 + 4 * lc);
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

// The matrix-core path: slabs of 2 channels in a ring of 4 buffers (3 slabs in
// flight; 53 KB of LDS, so 3 workgroups per CU), or of 1 channel for odd
// channel counts (37 KB).
constexpr int kMfCS = 2;
constexpr int kMfNB = 4;
// Channels per slab: 2, or 1 for odd channel counts and for 7x7 filters (whose
// 2-channel slabs need 181 VGPRs and 72 KB of LDS: 2 workgroups per CU against 4).
int mf_slab_channels(int r, int c) { return (c % kMfCS == 0 && r != 7) ? kMfCS : 1; }
template <bool RELU, bool D2S, bool VEC>
K2Fn pick_mf_v(int r, int c) {
  if (mf_slab_channels(r, c) == kMfCS) {
    if (r == 3) {
      if constexpr (VEC)
        if (c == 32) return is_k2_multi_mfma<3, kMfCS, kMfNB, 32 / kMfCS, RELU, D2S, VEC>;
      return is_k2_multi_mfma<3, kMfCS, kMfNB, 0, RELU, D2S, VEC>;
    }
    if constexpr (!D2S)
      if (r == 5) return is_k2_multi_mfma<5, kMfCS, kMfNB, 0, RELU, D2S, VEC>;
    return nullptr;
  }
  if (r == 3) return is_k2_multi_mfma<3, 1, kMfNB, 0, RELU, D2S, VEC>;
  if constexpr (!D2S) {
    if (r == 5) return is_k2_multi_mfma<5, 1, kMfNB, 0, RELU, D2S, VEC>;
    if (r == 7) return is_k2_multi_mfma<7, 1, kMfNB, 0, RELU, D2S, VEC>;
  }
  return nullptr;
}
// w % 4 == 0: 16-byte pixel groups and stores; else dwords (no depth-to-space).
template <bool RELU, bool D2S>
K2Fn pick_mf(int r, int c, int w) {
  if (w % 4 == 0) return pick_mf_v<RELU, D2S, true>(r, c);
  if constexpr (D2S) return nullptr;
  return pick_mf_v<RELU, false, false>(r, c);
}

}  // namespace

bool configure_multi(Plan &p, int param) {
  const conv2d_desc &d = p.d;
  if (d.layout != IS_NCHW || d.in_dtype != IS_F32 || d.r != d.s) return false;
  if (d.w % 4 != 0) return false;
  const int cs = (d.c % 4 == 0) ? 4 : 1;
  // Output channels per workgroup: as many as divide K, up to 16 (up to 32 for
  // one channel with K not a multiple of 16). With one input channel there is a
  // single slab, so a workgroup loads, computes and stores in sequence; 16
  // channels give twice the workgroups to overlap those phases (the 1 -> 32 5x5
  // layer of a 1280x720 frame: 35.5 against 38.5 us). With more channels 32 per
  // workgroup was the slowest choice but one at every shape the tuner timed
  // (3 -> 32 3x3: 40.2 us against 36.4 with 16; 3 -> 64: 72.5 against 64.0-65.2
  // with 8 or 16; 2 -> 32: 32.8 against 27.8-28.1).
  int ft = 0;
  for (int f : {32, 16, 8, 4, 2})
    if (d.k % f == 0 && !(f == 32 && d.k % 16 == 0 && pick<false>(d.r, 16, cs))) {
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

bool configure_multi_mf(Plan &p, int use) {
  const conv2d_desc &d = p.d;
  if (d.layout != IS_NCHW || d.in_dtype != IS_F32 || d.r != d.s || d.separable) return false;
  // The default plan for an even channel count from 4 on: measured on 1280x720
  // it beats the vector form at every such shape tried (32 -> 8 3x3: 61 against
  // 84 us; 64 -> 16: 228 against 284-344; 32 -> 64: 432 against 505-635; 5x5
  // layers, which the vector form takes only for some channel groups, 144-146
  // us), and loses only with 2 channels, one slab per tile (11.5 against 9.2
  // us). Odd and smaller channel counts keep the vector form (which reads the
  // input once for all its filters), with this form among the variants from 2
  // channels on; the plan falls back to it for the shapes that no other kernel
  // but the one-thread-per-output fallback takes.
  // 5x5 and 7x7 layers take it from 2 channels on whatever their parity (3 -> 32
  // 5x5: 59.6 against 74-87 us; 7 -> 16: 64 against 88-94; 2 -> 16: 28.2
  // against 30-35; the vector form has no 7x7).
  if (use == kMfPlan && (d.c < 4 || d.c % kMfCS != 0) && !(d.r >= 5 && d.c >= 2)) return false;
  if (use == kMfVariant && d.c < 2) return false;
  if (pick_mf<false, false>(d.r, d.c, d.w) == nullptr) return false;
  // 32-bit buffer offsets: one image's input and output planes, and the weights.
  const double img_bytes = 4.0 * d.c * (double)d.h * d.w;
  const double out_bytes = 4.0 * d.k * (double)d.h * d.w;
  const double w_bytes = 4.0 * d.k * d.c * d.r * d.s;
  if (img_bytes >= 4.0e9 || out_bytes >= 4.0e9 || w_bytes >= 2.0e9) return false;
  p.kid = kMultiMfmaF32;
  p.name = "is_k2_multi_mfma";
  p.nseg = (d.w + kTW - 1) / kTW;
  p.nstrip = (d.h + kTH - 1) / kTH;
  p.strip_rows = 4;      // output channels per workgroup
  const int cs = mf_slab_channels(d.r, d.c);
  p.vec = cs;            // input channels per LDS slab
  const long long tiles = (long long)p.nseg * p.nstrip * ((d.k + 3) / 4) * d.n;
  if (tiles > (1LL << 31) - 1) return false;
  p.ntiles = (int)tiles;
  p.grid_x = p.ntiles;
  p.grid_y = p.grid_z = 1;
  p.block = kThreads;
  p.lds = kMfNB * 16 * (cs == kMfCS ? (d.r == 3 ? MGeo<3, kMfCS>::BUFV4 : MGeo<5, kMfCS>::BUFV4)
                                    : (d.r == 3 ? MGeo<3, 1>::BUFV4
                                                : (d.r == 5 ? MGeo<5, 1>::BUFV4 : MGeo<7, 1>::BUFV4)));
  p.tile_w = kTW;
  p.tile_h = kTH;
  return true;
}

hipError_t launch_multi_mf(const Plan &p, const float *x, const float *w, const float *b, float *y,
                           hipStream_t s) {
  const conv2d_desc &d = p.d;
  const K2Fn fn = d.relu ? pick_mf<true, false>(d.r, d.c, d.w) : pick_mf<false, false>(d.r, d.c, d.w);
  if (p.kid != kMultiMfmaF32 || !fn) return hipErrorInvalidValue;
  return launch_kernel(fn, dim3(p.grid_x), dim3(p.block), 0, s, x, w, b, y, d.c, d.h, d.w, d.k, p.nseg,
                       p.nstrip, (d.k + 3) / 4, p.ntiles);
}

bool multi_d2s_supported(const Plan &p) {
  if (p.d.k != 4) return false;
  if (p.kid == kMultiMfmaF32) return pick_mf<false, true>(p.d.r, p.d.c, p.d.w) != nullptr;
  return p.kid == kMultiChannel && pick_d2s<false>(p.d.r, p.strip_rows, p.vec) != nullptr;
}

hipError_t launch_multi_d2s(const Plan &p, const float *x, const float *w, const float *b, float *y,
                            hipStream_t s) {
  const conv2d_desc &d = p.d;
  if (!multi_d2s_supported(p)) return hipErrorInvalidValue;
  const int ft = p.strip_rows, cs = p.vec;
  K2Fn fn;
  if (p.kid == kMultiMfmaF32)
    fn = d.relu ? pick_mf<true, true>(d.r, d.c, d.w) : pick_mf<false, true>(d.r, d.c, d.w);
  else
    fn = d.relu ? pick_d2s<true>(d.r, ft, cs) : pick_d2s<false>(d.r, ft, cs);
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
