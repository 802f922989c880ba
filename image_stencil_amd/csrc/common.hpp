// common.hpp -- device helpers shared by the gfx950 convolution kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <utility>

namespace is {

constexpr int kWave = 64;   // CDNA wavefront width

// Word 3 of a raw (unswizzled, stride 0) gfx9 buffer resource: 32-bit data
// format so that range checking is in bytes against num_records.
constexpr int kBufferFlags = 0x00020000;

// GFX9 DPP wavefront shifts: every lane reads the register of its neighbour
// inside the whole 64-lane wave (row_mask and bank_mask all on). A lane whose
// source lies outside the wave keeps `old` (bound_ctrl off).
constexpr int kDppWaveShl1 = 0x130;   // lane l reads lane l+1
constexpr int kDppWaveShr1 = 0x138;   // lane l reads lane l-1

__device__ __forceinline__ float from_prev_lane(float src, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src),
                                                    kDppWaveShr1, 0xf, 0xf, false));
}
__device__ __forceinline__ float from_next_lane(float src, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src),
                                                    kDppWaveShl1, 0xf, 0xf, false));
}

// Debug builds (-DIMGSTENCIL_LDS_POISON) fill a kernel's LDS with a pattern
// that is NaN both as fp32 and as each fp16 half before the kernel stages
// anything, so that a read of LDS that was never written (a missing wait or
// barrier, an unwritten halo) turns into NaN in the output, which the parity
// tests reject. Release builds compile it to nothing.
__device__ __forceinline__ void lds_poison(void *lds, int bytes) {
#ifdef IMGSTENCIL_LDS_POISON
  unsigned *p = static_cast<unsigned *>(lds);
  for (int i = threadIdx.x; i < bytes / 4; i += blockDim.x) p[i] = 0x7FC07FC0u;
  __syncthreads();
#else
  (void)lds;
  (void)bytes;
#endif
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations
// (lgkmcnt 0) but not for its vector-memory operations, so that loads into
// another LDS buffer stay in flight across it (__syncthreads() waits for
// those too). The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Workgroups are dealt to the 8 XCDs of the chip round-robin in launch order,
// and each XCD has its own L2. Renumber launch index b so that XCD k receives
// the contiguous logical range [k*T/8, (k+1)*T/8) of the first 8*floor(T/8)
// tiles; neighbouring tiles then share an L2 and their halo rows/columns hit
// there. The last T mod 8 tiles keep their own index. A bijection on [0, T).
__device__ __forceinline__ int xcd_remap(int b, int T) {
  const int per = T >> 3;
  if (b >= (per << 3)) return b;
  return (b & 7) * per + (b >> 3);
}

// XOR swizzle of a column index inside an LDS array T a[][nx] whose rows are
// nx * elem_bytes bytes (a power of two >= 32), permuting chunks of chunk_bytes:
// chunk index i = (y*nx + x)*eb/cb, row-of-chunks yc = i / (nx*eb/cb),
// column-of-chunks xc = i mod (nx*eb/cb), swizzled chunk xc ^ yc, then back to an
// element column keeping the element's offset inside its chunk. Used for the
// NHWC fp16 tiles; a bijection on x for every fixed y.
__host__ __device__ constexpr int swizzle_col(int y, int x, int nx, int eb, int cb) {
  const int per_chunk = cb / eb;                  // elements per chunk
  const int chunks_per_row = (nx * eb) / cb;      // chunks in one swizzle row
  const long long i_chunk = ((long long)y * nx + x) * eb / cb;
  const long long y_chunk = i_chunk / chunks_per_row;
  const long long x_chunk = i_chunk % chunks_per_row;
  const long long x_chunk_swz = y_chunk ^ x_chunk;
  return (int)((x_chunk_swz * per_chunk) % nx) + x % per_chunk;
}

// Launch and report this launch's error. hipGetLastError() is per-thread state
// that earlier calls of the host program (not ours) may have left set; it is
// cleared first so that only a failure of this launch is returned.
// Calls f(std::integral_constant<int, 0>{}), ..., f(<N-1>) in order: a loop
// whose index is a compile-time constant in every step, for bodies too large
// for the unroller's size limit (a partially unrolled loop would index
// register arrays dynamically).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, unsigned lds, hipStream_t s,
                         Args &&...args) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(kernel, grid, block, lds, s, static_cast<KArgs>(args)...);
  return hipGetLastError();
}

}  // namespace is
