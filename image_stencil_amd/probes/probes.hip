// probes.hip -- measurement kernels for the benchmark (not part of the
// convolution library): the rate that back-to-back matrix-core instructions
// sustain on this chip, with the shader clock during the run, and the LDS
// bank behaviour of the access widths the convolution kernels use.
//
// Every kernel stays inside its own buffers: `stamps` holds two values per
// wave, `sink` one per thread, and LDS addresses stay below kLdsBytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;   // 4 waves: one per SIMD of a CU
constexpr int kMaxChains = 8;   // independent accumulators per wave (at most)

__device__ __forceinline__ unsigned hash32(unsigned v) {
  v ^= v >> 16;
  v *= 0x7feb352dU;
  v ^= v >> 15;
  v *= 0x846ca68bU;
  v ^= v >> 16;
  return v;
}

template <typename Fn, int... I>
__device__ __forceinline__ void static_for_seq(Fn &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <typename Fn>
__device__ __forceinline__ void static_for_steps(Fn &&f) {
  static_for_seq(f, std::make_integer_sequence<int, 24>{});
}

// Back-to-back MFMAs: every wave issues kChains independent accumulations per
// step (so no instruction waits for the previous one's result) for `iters`
// steps, on operands that differ from one instruction to the next (random
// values in [-1, 1), as the convolution's data would). F16: the fp16 layer's
// v_mfma_f32_16x16x32_f16 (16384 FLOP each); else v_mfma_f32_16x16x4_f32
// (2048 FLOP each). Each wave's lane 0 records its shader-clock cycles
// (s_memtime) and 100 MHz real-time ticks (s_memrealtime) over the loop.
template <bool F16, int kChains = 8>
__global__ __launch_bounds__(kThreads) void isp_mfma_rate(int iters, unsigned long long *stamps, float *sink) {
  const int tid = threadIdx.x;
  const unsigned gid = blockIdx.x * kThreads + tid;
  float4v acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = float4v{0.f, 0.f, 0.f, 0.f};
  unsigned long long c0 = 0, r0 = 0;
  if constexpr (F16) {
    half8 a[kMaxChains], b[kMaxChains];
#pragma unroll
    for (int j = 0; j < kMaxChains; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[j][e] = (_Float16)((int)(hash32(gid * 64 + j * 8 + e) & 0xFFFF) / 32768.f - 1.f);
        b[j][e] = (_Float16)((int)(hash32(gid * 64 + j * 8 + e + 0x9E3779B9u) & 0xFFFF) / 32768.f - 1.f);
      }
    c0 = clock64();
    r0 = wall_clock64();
    // kMaxChains MFMAs per step in any case (the host's count), spread over
    // kChains accumulators: each accumulator's next product depends on its
    // previous one kChains instructions earlier.
    for (int i = 0; i < iters; i += kMaxChains) {   // the host rounds iters to a multiple of 8
#pragma unroll
      for (int ii = 0; ii < kMaxChains; ++ii)
#pragma unroll
        for (int j = 0; j < kMaxChains; ++j)
          acc[j % kChains] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], b[(j + ii) % kMaxChains],
                                                                     acc[j % kChains], 0, 0, 0);
    }
  } else {
    float a[kMaxChains], b[kMaxChains];
#pragma unroll
    for (int j = 0; j < kMaxChains; ++j) {
      a[j] = (int)(hash32(gid * 16 + j) & 0xFFFF) / 32768.f - 1.f;
      b[j] = (int)(hash32(gid * 16 + j + 0x9E3779B9u) & 0xFFFF) / 32768.f - 1.f;
    }
    c0 = clock64();
    r0 = wall_clock64();
    for (int i = 0; i < iters; i += kMaxChains) {
#pragma unroll
      for (int ii = 0; ii < kMaxChains; ++ii)
#pragma unroll
        for (int j = 0; j < kMaxChains; ++j)
          acc[j % kChains] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[(j + ii) % kMaxChains],
                                                                  acc[j % kChains], 0, 0, 0);
    }
  }
  const unsigned long long c1 = clock64(), r1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sink[gid] = s;
  if ((tid & 63) == 0) {
    const unsigned wave = gid >> 6;
    stamps[2 * wave] = c1 - c0;
    stamps[2 * wave + 1] = r1 - r0;
  }
}

// LDS bank probe: one wave per workgroup repeats one LDS access `iters`
// times, every lane at the byte address pattern(lane) (alternating with a copy
// of the pattern 8 KB higher, which keeps the banks and stops the compiler from
// merging the accesses). OP: 0 read 16 B, 1 write 16 B, 2 read 8 B, 3 write
// 8 B. PAT: 0 contiguous (lane x width); 1 every lane in one 16-byte bank
// group, rows 128 B apart; 2 groups of 8 consecutive lanes each covering the
// 128 bytes of one row (rows 256 B apart); 3 groups of 16 consecutive lanes
// covering 256 bytes, but lanes l and l + 1 of an even pair share a 16-byte
// bank group in the 128-byte view; 4 pixel-row reads of the fp16 layer: lane
// l reads 16-byte chunk c = l / 16 of pixel l mod 16 under the 128-byte XOR
// swizzle (chunk position c ^ (pixel mod 8)); 5 every lane at one address
// (broadcast); 6 in each group of 16 lanes, lanes 0-14 share one address and
// lane 15 reads another (a row's left and right halo vectors, rows 288 bytes
// apart, as the multi-channel kernel reads them); 7 the same rows, every lane
// its own vector (that kernel's main read).
constexpr int kLdsBytes = 32 * 1024;

template <int PAT, int WIDTH>
__device__ __forceinline__ int probe_addr(int lane) {
  if constexpr (PAT == 0) return lane * WIDTH;
  if constexpr (PAT == 1) return lane * 128;
  if constexpr (PAT == 2) return (lane % 8) * 16 + (lane / 8) * 256;
  if constexpr (PAT == 3) return ((lane % 16) % 2 * 8 + (lane % 16) / 2) * 16 + (lane / 16) * 256;
  if constexpr (PAT == 5) return 0;
  if constexpr (PAT == 6) return (lane / 16) * 288 + ((lane % 16) == 15 ? 17 * 16 : 0);
  if constexpr (PAT == 7) return (lane / 16) * 288 + ((lane % 16) + 1) * 16;
  const int px = lane % 16, c = lane / 16;
  return px * 128 + ((c ^ (px % 8)) * 16);
}

template <int OP, int PAT>
__global__ __launch_bounds__(64) void isp_lds_probe(int iters, float *sink) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int lane = threadIdx.x;
  constexpr int WIDTH = (OP <= 1) ? 16 : 8;
  const int base = probe_addr<PAT, WIDTH>(lane);
  for (int i = lane; i < kLdsBytes / 4; i += 64) reinterpret_cast<float *>(lds)[i] = (float)i;
  __syncthreads();
  uint4v acc = {0u, 0u, 0u, 0u};
  for (int i = 0; i < iters; ++i) {
    const int addr = base + (i & 1) * 8192;
    if constexpr (OP == 0) {
      const uint4v v = *reinterpret_cast<const uint4v *>(lds + addr);
      acc ^= v;
    } else if constexpr (OP == 1) {
      *reinterpret_cast<uint4v *>(lds + addr) = uint4v{(unsigned)i, (unsigned)lane, acc.x, 1u};
    } else if constexpr (OP == 2) {
      const uint2v v = *reinterpret_cast<const uint2v *>(lds + addr);
      acc.x ^= v.x;
      acc.y ^= v.y;
    } else {
      *reinterpret_cast<uint2v *>(lds + addr) = uint2v{(unsigned)i, (unsigned)lane};
    }
    __asm__ volatile("" ::: "memory");
  }
  __syncthreads();
  sink[blockIdx.x * 64 + lane] = (float)(acc.x ^ acc.y ^ acc.z ^ acc.w) + lds[(lane * 16) % kLdsBytes];
}

// Lane-pair probe: every lane accesses lane x width (contiguous, conflict-
// free) except lane `partner`, which accesses lane 0's bank position
// `offset` bytes higher (offset a multiple of 256, past the contiguous block).
// A conflict then means that lane 0 and `partner` are served in the same LDS
// pass. OP as above.
template <int OP>
__global__ __launch_bounds__(64) void isp_lds_pair_probe(int partner, int offset, int iters, float *sink) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int lane = threadIdx.x;
  constexpr int WIDTH = (OP <= 1) ? 16 : 8;
  const int base = lane == partner ? offset : lane * WIDTH;
  for (int i = lane; i < kLdsBytes / 4; i += 64) reinterpret_cast<float *>(lds)[i] = (float)i;
  __syncthreads();
  uint4v acc = {0u, 0u, 0u, 0u};
  for (int i = 0; i < iters; ++i) {
    const int addr = base + (i & 1) * 8192;
    if constexpr (OP == 0) {
      acc ^= *reinterpret_cast<const uint4v *>(lds + addr);
    } else if constexpr (OP == 1) {
      *reinterpret_cast<uint4v *>(lds + addr) = uint4v{(unsigned)i, (unsigned)lane, acc.x, 1u};
    } else if constexpr (OP == 2) {
      const uint2v v = *reinterpret_cast<const uint2v *>(lds + addr);
      acc.x ^= v.x;
      acc.y ^= v.y;
    } else {
      *reinterpret_cast<uint2v *>(lds + addr) = uint2v{(unsigned)i, (unsigned)lane};
    }
    __asm__ volatile("" ::: "memory");
  }
  __syncthreads();
  sink[blockIdx.x * 64 + lane] = (float)(acc.x ^ acc.y ^ acc.z ^ acc.w) + lds[(lane * 16) % kLdsBytes];
}

// Stride probe: lane l accesses (l mod group) x width + (l / group) x stride,
// so groups of `group` consecutive lanes cover contiguous bytes and the groups
// lie `stride` bytes apart. Whether two groups served in the same pass
// conflict at a given stride shows how the bank index depends on the address.
constexpr int kStrideLdsBytes = 64 * 1024;

template <int OP>
__global__ __launch_bounds__(64) void isp_lds_stride_probe(int group, int stride, int offset, int iters,
                                                           float *sink) {
  __shared__ __attribute__((aligned(16))) char lds[kStrideLdsBytes];
  const int lane = threadIdx.x;
  constexpr int WIDTH = (OP <= 1) ? 16 : 8;
  const int base = offset + (lane % group) * WIDTH + (lane / group) * stride;
  for (int i = lane; i < kStrideLdsBytes / 4; i += 64) reinterpret_cast<float *>(lds)[i] = (float)i;
  __syncthreads();
  uint4v acc = {0u, 0u, 0u, 0u};
  for (int i = 0; i < iters; ++i) {
    const int addr = base + (i & 1) * (kStrideLdsBytes / 2);
    if constexpr (OP == 0) {
      acc ^= *reinterpret_cast<const uint4v *>(lds + addr);
    } else if constexpr (OP == 1) {
      *reinterpret_cast<uint4v *>(lds + addr) = uint4v{(unsigned)i, (unsigned)lane, acc.x, 1u};
    } else if constexpr (OP == 2) {
      const uint2v v = *reinterpret_cast<const uint2v *>(lds + addr);
      acc.x ^= v.x;
      acc.y ^= v.y;
    } else {
      *reinterpret_cast<uint2v *>(lds + addr) = uint2v{(unsigned)i, (unsigned)lane};
    }
    __asm__ volatile("" ::: "memory");
  }
  __syncthreads();
  sink[blockIdx.x * 64 + lane] = (float)(acc.x ^ acc.y ^ acc.z ^ acc.w) + lds[(lane * 16) % kStrideLdsBytes];
}

template <typename... KArgs, typename... Args>
hipError_t launch(void (*k)(KArgs...), int grid, int block, hipStream_t s, Args... args) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k, dim3(grid), dim3(block), 0, s, static_cast<KArgs>(args)...);
  return hipGetLastError();
}

// LDS throughput: one workgroup of `waves` waves per CU; every wave issues
// steps of 8 independent, conflict-free accesses (each wave 8 whole 64-lane
// blocks of its own; OP 0 read 16 B, 1 write 16 B, 2 read 8 B) for `iters`
// steps. Lane 0 of each wave records its cycles and real-time ticks over the
// loop, as the MFMA probe does.
constexpr int kRateLdsBytes = 64 * 1024;

template <int OP>
__global__ __launch_bounds__(1024) void isp_lds_rate(int iters, unsigned long long *stamps, float *sink) {
  __shared__ __attribute__((aligned(16))) char lds[kRateLdsBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int WIDTH = (OP == 2) ? 8 : 16;
  for (int i = tid; i < kRateLdsBytes / 4; i += blockDim.x) reinterpret_cast<float *>(lds)[i] = (float)i;
  __syncthreads();
  uint4v acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = uint4v{0u, 0u, 0u, 0u};
  const unsigned long long c0 = clock64(), r0 = wall_clock64();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // 64 x WIDTH bytes per block; blocks wrap within the 64 KB array
      const int addr = ((wave * 8 + j) * 64 * WIDTH + lane * WIDTH) & (kRateLdsBytes - 1);
      if constexpr (OP == 0) {
        acc[j] ^= *reinterpret_cast<const uint4v *>(lds + addr);
      } else if constexpr (OP == 1) {
        *reinterpret_cast<uint4v *>(lds + addr) = uint4v{(unsigned)i, (unsigned)lane, (unsigned)j, 1u};
      } else {
        const uint2v v = *reinterpret_cast<const uint2v *>(lds + addr);
        acc[j].x ^= v.x;
        acc[j].y ^= v.y;
      }
    }
    __asm__ volatile("" ::: "memory");
  }
  const unsigned long long c1 = clock64(), r1 = wall_clock64();
  __syncthreads();
  unsigned x = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) x ^= acc[j].x ^ acc[j].y ^ acc[j].z ^ acc[j].w;
  sink[blockIdx.x * blockDim.x + tid] = (float)x + lds[(tid * 16) % kRateLdsBytes];
  if (lane == 0) {
    const unsigned gw = blockIdx.x * (blockDim.x >> 6) + wave;
    stamps[2 * gw] = c1 - c0;
    stamps[2 * gw + 1] = r1 - r0;
  }
}

// The fp16 layer's instruction mix, piece by piece: 8 waves per CU (2 per
// SIMD), each holding 18 A fragments in registers and stepping through 24
// operand slots of 1 KB per round (a stage of 4 input rows x 3 tap columns x
// 2 channel halves): every step reads the operand 8 steps ahead from LDS into a
// register ring and issues 3 v_mfma_f32_16x16x32_f16 that use the current one,
// into 3 of 4 rotating accumulators; every 6 steps one accumulator is finished
// (fp16, 8 bytes per lane). MIX bits switch the parts on: 1 the LDS operand
// reads (else the ring keeps its first values), 2 the MFMAs (else one VALU add
// per product), 4 the finished rows' LDS writes, 8 a workgroup barrier (LDS
// drained) per round, 16 two 16-byte global stores per wave per round, 32 three
// 16-byte global-to-LDS loads per wave per round (each round's waited for at
// the barrier 3 rounds later, as the layer waits for its row DMA), 64 the
// stores and loads split by wave (even waves store, odd waves load). gbuf holds
// 64 KB per workgroup; LDS addresses stay below 128 KB.
constexpr int kMixLdsBytes = 128 * 1024;
// s_waitcnt immediate: at most n vector memory operations outstanding (expcnt
// and lgkmcnt not waited for).
constexpr int mix_vm_wait(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kMixSteps = 24;

template <int MIX>
__global__ __launch_bounds__(512, 1) void isp_mix_rate(int iters, unsigned long long *stamps, float *sink,
                                                       char *gbuf) {
  __shared__ __attribute__((aligned(16))) char lds[kMixLdsBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(gbuf + (size_t)blockIdx.x * 65536, (short)0, 65536, 0x00020000);
  for (int i = tid; i < kMixLdsBytes / 4; i += blockDim.x)
    reinterpret_cast<float *>(lds)[i] = (float)(i & 255) * (1.f / 256);
  __syncthreads();
  half8 wa[18];
#pragma unroll
  for (int k = 0; k < 18; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) wa[k][e] = (_Float16)((int)(hash32(tid * 256 + k * 8 + e) & 255) / 256.f);
  // Waves 0, 2, 4, 6 and 1, 3, 5, 7 read the same 24 KB (the four output-channel
  // waves of a pixel block share their operand rows in the layer).
  const int rbase = (wave & 1) * kMixSteps * 1024 + lane * 16;   // < 48 KB + 24 KB
  const int wbase = 64 * 1024 + wave * 4096 + lane * 8;          // < 96 KB
  half8 ring[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) ring[q] = *reinterpret_cast<const half8 *>(lds + rbase + q * 1024);
  float4v acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = float4v{0.f, 0.f, 0.f, 0.f};
  const unsigned long long c0 = clock64(), r0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
    static_for_steps([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      if constexpr ((MIX & 16) && !(MIX & 64) && (q == 2 || q == 14))
        __builtin_amdgcn_raw_buffer_store_b128(uint4v{(unsigned)it, (unsigned)lane, (unsigned)q, 1u}, rs,
                                               (wave * 2 + q / 12) * 1024 + lane * 16, 0, 2);
      if constexpr ((MIX & 32) && !(MIX & 64) && (q == 3 || q == 11 || q == 19))
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void *)(lds + 96 * 1024 + (wave * 3 + q / 8) * 1024), 16,
            32768 + (wave * 3 + q / 8) * 1024 + lane * 16, 0, 0, 2);
      // 64: the same stores and loads per workgroup, split by wave: the even
      // waves issue all the stores (4 each), the odd ones all the loads (6 each).
      if constexpr ((MIX & 16) && (MIX & 64) && q % 6 == 2)
        if ((wave & 1) == 0)
          __builtin_amdgcn_raw_buffer_store_b128(uint4v{(unsigned)it, (unsigned)lane, (unsigned)q, 1u}, rs,
                                                 (wave * 4 + q / 6) * 1024 + lane * 16, 0, 2);
      if constexpr ((MIX & 32) && (MIX & 64) && q % 4 == 3)
        if (wave & 1)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void *)(lds + 96 * 1024 + ((wave * 6 + q / 4) % 32) * 1024),
              16, 32768 + ((wave * 6 + q / 4) % 32) * 1024 + lane * 16, 0, 0, 2);
      const half8 b = ring[q % 8];
      if constexpr (MIX & 1)   // moving by 16 bytes a round keeps the reads conflict-free and live
        ring[q % 8] = *reinterpret_cast<const half8 *>(lds + rbase + ((q + 8) % kMixSteps) * 1024 + (it & 7) * 16);
      constexpr int i = q / 6, v = (q % 6) / 2, h = q % 2;
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int ks = 2 * (3 * u + v) + h;
        if constexpr (MIX & 2)
          acc[(i - u) & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[ks], b, acc[(i - u) & 3], 0, 0, 0);
        else
          acc[(i - u) & 3][0] += (float)b[0];
      }
      if constexpr (q % 6 == 5) {
        _Float16 hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = (_Float16)(acc[(i - 2) & 3][e] + 0.5f);
        acc[(i - 2) & 3] = float4v{0.f, 0.f, 0.f, 0.f};
        if constexpr (MIX & 4)
          *reinterpret_cast<uint2v *>(lds + wbase + i * 512 + (it & 1) * 2048) = __builtin_bit_cast(uint2v, hv);
        else
          acc[(i + 1) & 3][1] += (float)hv[0] + (float)hv[3];
      }
    });
    __asm__ volatile("" ::: "memory");
    if constexpr (MIX & 8) {
      // As in the layer (5 stages of DMA ahead, each waited for 3 stages
      // after it was issued): the loads of the round 3 rounds back have
      // landed; this round's and the 2 before it may still be in flight.
      if constexpr ((MIX & 32) && !(MIX & 64)) __builtin_amdgcn_s_waitcnt(mix_vm_wait(3 * ((MIX & 16 ? 2 : 0) + 3)));
      if constexpr ((MIX & 32) && (MIX & 64)) {
        if (wave & 1) __builtin_amdgcn_s_waitcnt(mix_vm_wait(3 * 6));
        else __builtin_amdgcn_s_waitcnt(mix_vm_wait(3 * 4));
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);                            // lgkmcnt 0
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    }
  }
  const unsigned long long c1 = clock64(), r1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
#pragma unroll
  for (int q = 0; q < 8; ++q) s += (float)ring[q][0];
  __syncthreads();
  sink[blockIdx.x * blockDim.x + tid] = s + lds[(tid * 16) % kMixLdsBytes];
  if (lane == 0) {
    const unsigned gw = blockIdx.x * 8 + wave;
    stamps[2 * gw] = c1 - c0;
    stamps[2 * gw + 1] = r1 - r0;
  }
}

// The same stage on another data flow, for comparison: 4 waves per CU (one per
// SIMD), each holding 64 output channels x half the k range (input channels
// 32*kh .. +32 of all 9 taps: 36 A fragments), so one 16-byte operand read
// feeds 12 MFMAs (4 channel blocks x 3 accumulating rows) instead of 3. The two
// k halves of an output row are summed through LDS: when a row is final the
// kh = 1 waves write their fp32 partial sums (4 x 16 bytes per lane) and the
// kh = 0 waves read and add them before rounding to fp16 and staging the row.
// MIX bits as above (4: the partial-sum exchange with the staging writes); per
// round (4 input rows) each wave makes 12 operand reads and 144 MFMAs, so a
// CU does 576 MFMAs per round as in isp_mix_rate. gbuf holds 64 KB per
// workgroup; LDS addresses stay below 128 KB.
template <int MIX>
__global__ __launch_bounds__(256, 1) void isp_mix4_rate(int iters, unsigned long long *stamps, float *sink,
                                                        char *gbuf) {
  constexpr int kSteps4 = 12;   // 4 input rows x 3 filter columns
  __shared__ __attribute__((aligned(16))) char lds[kMixLdsBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int kh = wave >> 1;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(gbuf + (size_t)blockIdx.x * 65536, (short)0, 65536, 0x00020000);
  for (int i = tid; i < kMixLdsBytes / 4; i += blockDim.x)
    reinterpret_cast<float *>(lds)[i] = (float)(i & 255) * (1.f / 256);
  __syncthreads();
  half8 wa[36];
#pragma unroll
  for (int k = 0; k < 36; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) wa[k][e] = (_Float16)((int)(hash32(tid * 512 + k * 8 + e) & 255) / 256.f);
  const int rbase = wave * kSteps4 * 1024 + lane * 16;            // reads below 48 KB + 1.1 KB
  const int pbase = 50 * 1024 + (wave & 1) * 4096 + lane * 16;    // partial sums below 68 KB
  const int sbase = 72 * 1024 + wave * 2048 + lane * 8;           // staging below 80 KB
  half8 ring[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ring[q] = *reinterpret_cast<const half8 *>(lds + rbase + q * 1024);
  float4v acc[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[b][j] = float4v{0.f, 0.f, 0.f, 0.f};
  const unsigned long long c0 = clock64(), r0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
    static_for_seq([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      if constexpr ((MIX & 16) && q % 3 == 1)
        __builtin_amdgcn_raw_buffer_store_b128(uint4v{(unsigned)it, (unsigned)lane, (unsigned)q, 1u}, rs,
                                               (wave * 4 + q / 3) * 1024 + lane * 16, 0, 2);
      if constexpr ((MIX & 32) && q % 3 == 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void *)(lds + 96 * 1024 + (wave * 4 + q / 3) * 1024), 16,
            32768 + (wave * 4 + q / 3) * 1024 + lane * 16, 0, 0, 2);
      const half8 b = ring[q % 4];
      if constexpr (MIX & 1)
        ring[q % 4] = *reinterpret_cast<const half8 *>(lds + rbase + ((q + 4) % kSteps4) * 1024 + (it & 7) * 16);
      constexpr int i = q / 3, v = q % 3;
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          if constexpr (MIX & 2)
            acc[blk][(i - u) & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[blk * 9 + 3 * u + v], b,
                                                                            acc[blk][(i - u) & 3], 0, 0, 0);
          else
            acc[blk][(i - u) & 3][0] += (float)b[0];
        }
      if constexpr (v == 2) {   // output row i - 2 is final in every block
        constexpr int o = (i - 2) & 3;
        if constexpr (MIX & 4) {
          char *pp = lds + pbase + (it & 1) * 8192;
          if (kh) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) *reinterpret_cast<float4v *>(pp + blk * 1024) = acc[blk][o];
          } else {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
              const float4v pv = *reinterpret_cast<const float4v *>(pp + blk * 1024 + 2048);
              _Float16 hv[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) hv[e] = (_Float16)(acc[blk][o][e] + pv[e]);
              *reinterpret_cast<uint2v *>(lds + sbase + blk * 512 + (it & 1) * 256) = __builtin_bit_cast(uint2v, hv);
            }
          }
        } else {
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) acc[blk][(o + 1) & 3][1] += acc[blk][o][2];
        }
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) acc[blk][o] = float4v{0.f, 0.f, 0.f, 0.f};
      }
    }, std::make_integer_sequence<int, kSteps4>{});
    __asm__ volatile("" ::: "memory");
    if constexpr (MIX & 8) {
      if constexpr (MIX & 32) __builtin_amdgcn_s_waitcnt(mix_vm_wait(3 * ((MIX & 16 ? 4 : 0) + 4)));   // as above
      __builtin_amdgcn_s_waitcnt(0xC07F);                            // lgkmcnt 0
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    }
  }
  const unsigned long long c1 = clock64(), r1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[b][j][0] + acc[b][j][1] + acc[b][j][2] + acc[b][j][3];
#pragma unroll
  for (int q = 0; q < 4; ++q) s += (float)ring[q][0];
  __syncthreads();
  sink[blockIdx.x * blockDim.x + tid] = s + lds[(tid * 16) % kMixLdsBytes];
  if (lane == 0) {
    const unsigned gw = blockIdx.x * 4 + wave;
    stamps[2 * gw] = c1 - c0;
    stamps[2 * gw + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Back-to-back MFMA rate: `grid` workgroups of 256 threads; stamps holds
// 2 x (grid x 4) values, sink grid x 256 floats. kind 0: fp16 16x16x32, 1: fp32
// 16x16x4. iters is rounded up to a multiple of 8 (steps of 8 MFMAs per wave
// each). Returns a hipError_t.
int isp_mfma_rate(int kind, int grid, int iters, unsigned long long *stamps, float *sink, hipStream_t s) {
  if (grid < 1 || iters < 1 || !stamps || !sink) return (int)hipErrorInvalidValue;
  iters = (iters + kMaxChains - 1) / kMaxChains * kMaxChains;
  if (kind == 0) return (int)launch(isp_mfma_rate<true>, grid, kThreads, s, iters, stamps, sink);
  if (kind == 1) return (int)launch(isp_mfma_rate<false>, grid, kThreads, s, iters, stamps, sink);
  return (int)hipErrorInvalidValue;
}

// The fp16 rate with `chains` independent accumulators per wave (1, 2, 3, 4,
// 6 or 8; 8 MFMAs per step in every case): how far apart dependent products
// must be to keep the matrix unit busy.
int isp_mfma_chain_rate(int chains, int grid, int iters, unsigned long long *stamps, float *sink, hipStream_t s) {
  if (grid < 1 || iters < 1 || !stamps || !sink) return (int)hipErrorInvalidValue;
  iters = (iters + kMaxChains - 1) / kMaxChains * kMaxChains;
  switch (chains) {
    case 1: return (int)launch(isp_mfma_rate<true, 1>, grid, kThreads, s, iters, stamps, sink);
    case 2: return (int)launch(isp_mfma_rate<true, 2>, grid, kThreads, s, iters, stamps, sink);
    case 3: return (int)launch(isp_mfma_rate<true, 3>, grid, kThreads, s, iters, stamps, sink);
    case 4: return (int)launch(isp_mfma_rate<true, 4>, grid, kThreads, s, iters, stamps, sink);
    case 6: return (int)launch(isp_mfma_rate<true, 6>, grid, kThreads, s, iters, stamps, sink);
    case 8: return (int)launch(isp_mfma_rate<true, 8>, grid, kThreads, s, iters, stamps, sink);
    default: return (int)hipErrorInvalidValue;
  }
}

// LDS probe of access `op` and address pattern `pat` (see above): `grid`
// one-wave workgroups; sink holds grid x 64 floats.
int isp_lds_probe(int op, int pat, int grid, int iters, float *sink, hipStream_t s) {
  if (grid < 1 || iters < 1 || !sink) return (int)hipErrorInvalidValue;
#define ISP_CASE(O, P) \
  if (op == O && pat == P) return (int)launch(isp_lds_probe<O, P>, grid, 64, s, iters, sink);
#define ISP_OP(O) \
  ISP_CASE(O, 0) ISP_CASE(O, 1) ISP_CASE(O, 2) ISP_CASE(O, 3) ISP_CASE(O, 4) ISP_CASE(O, 5) ISP_CASE(O, 6) ISP_CASE(O, 7)
  ISP_OP(0) ISP_OP(1) ISP_OP(2) ISP_OP(3)
#undef ISP_OP
#undef ISP_CASE
  return (int)hipErrorInvalidValue;
}

// Stride probe (see above), every address moved up by `offset` bytes: group
// in {4, 8, 16, 32}; stride and offset multiples of 16; the highest address,
// offset + (63 / group) x stride + group x width, must stay within half the
// 64 KB.
int isp_lds_stride_probe(int op, int group, int stride, int offset, int grid, int iters, float *sink,
                         hipStream_t s) {
  if (grid < 1 || iters < 1 || !sink || (group != 4 && group != 8 && group != 16 && group != 32) || stride < 0 ||
      stride % 16 != 0 || offset < 0 || offset % 16 != 0 ||
      offset + (63 / group) * stride + group * 16 > kStrideLdsBytes / 2)
    return (int)hipErrorInvalidValue;
  switch (op) {
    case 0: return (int)launch(isp_lds_stride_probe<0>, grid, 64, s, group, stride, offset, iters, sink);
    case 1: return (int)launch(isp_lds_stride_probe<1>, grid, 64, s, group, stride, offset, iters, sink);
    case 2: return (int)launch(isp_lds_stride_probe<2>, grid, 64, s, group, stride, offset, iters, sink);
    case 3: return (int)launch(isp_lds_stride_probe<3>, grid, 64, s, group, stride, offset, iters, sink);
    default: return (int)hipErrorInvalidValue;
  }
}

// LDS throughput probe (see above): `grid` workgroups of `waves` waves (4, 8
// or 16); stamps holds 2 x grid x waves values, sink grid x waves x 64 floats.
int isp_lds_rate(int op, int waves, int grid, int iters, unsigned long long *stamps, float *sink, hipStream_t s) {
  if (grid < 1 || iters < 1 || !stamps || !sink || (waves != 4 && waves != 8 && waves != 16))
    return (int)hipErrorInvalidValue;
  switch (op) {
    case 0: return (int)launch(isp_lds_rate<0>, grid, 64 * waves, s, iters, stamps, sink);
    case 1: return (int)launch(isp_lds_rate<1>, grid, 64 * waves, s, iters, stamps, sink);
    case 2: return (int)launch(isp_lds_rate<2>, grid, 64 * waves, s, iters, stamps, sink);
    default: return (int)hipErrorInvalidValue;
  }
}

// Instruction-mix probe (see above): `grid` workgroups of 8 waves; mix is an
// OR of the part bits (1 .. 63); stamps holds 2 x grid x 8 values, sink
// grid x 512 floats, gbuf grid x 64 KB.
int isp_mix_rate(int mix, int grid, int iters, unsigned long long *stamps, float *sink, char *gbuf, hipStream_t s) {
  if (grid < 1 || iters < 1 || !stamps || !sink || !gbuf) return (int)hipErrorInvalidValue;
  switch (mix) {
#define ISP_MIX(M) \
  case M: return (int)launch(isp_mix_rate<M>, grid, 512, s, iters, stamps, sink, gbuf);
    ISP_MIX(2) ISP_MIX(3) ISP_MIX(7) ISP_MIX(10) ISP_MIX(11) ISP_MIX(15) ISP_MIX(31) ISP_MIX(47) ISP_MIX(63)
    ISP_MIX(5) ISP_MIX(61) ISP_MIX(127) ISP_MIX(125)
#undef ISP_MIX
    default: return (int)hipErrorInvalidValue;
  }
}

// The 4-wave data flow (isp_mix4_rate): `grid` workgroups of 256 threads;
// stamps 2 x (grid x 4) values, sink grid x 256 floats, gbuf grid x 64 KB.
int isp_mix4_rate(int mix, int grid, int iters, unsigned long long *stamps, float *sink, char *gbuf, hipStream_t s) {
  if (grid < 1 || iters < 1 || !stamps || !sink || !gbuf) return (int)hipErrorInvalidValue;
  switch (mix) {
#define IS_MIX4_CASE(M) \
  case M: return (int)launch(isp_mix4_rate<M>, grid, 256, s, iters, stamps, sink, gbuf);
    IS_MIX4_CASE(2) IS_MIX4_CASE(3) IS_MIX4_CASE(7) IS_MIX4_CASE(15) IS_MIX4_CASE(10) IS_MIX4_CASE(11)
    IS_MIX4_CASE(31) IS_MIX4_CASE(47) IS_MIX4_CASE(63) IS_MIX4_CASE(5) IS_MIX4_CASE(61)
#undef IS_MIX4_CASE
    default: return (int)hipErrorInvalidValue;
  }
}

// Lane-pair probe (see above): offset must be a multiple of 256 in
// [1024, 8192]; `grid` one-wave workgroups; sink holds grid x 64 floats.
int isp_lds_pair_probe(int op, int partner, int offset, int grid, int iters, float *sink, hipStream_t s) {
  if (grid < 1 || iters < 1 || !sink || partner < 0 || partner > 63 || offset < 1024 || offset > 8192 ||
      offset % 256 != 0)
    return (int)hipErrorInvalidValue;
  switch (op) {
    case 0: return (int)launch(isp_lds_pair_probe<0>, grid, 64, s, partner, offset, iters, sink);
    case 1: return (int)launch(isp_lds_pair_probe<1>, grid, 64, s, partner, offset, iters, sink);
    case 2: return (int)launch(isp_lds_pair_probe<2>, grid, 64, s, partner, offset, iters, sink);
    case 3: return (int)launch(isp_lds_pair_probe<3>, grid, 64, s, partner, offset, iters, sink);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // extern "C"
