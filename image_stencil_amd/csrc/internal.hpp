// internal.hpp -- plan structure and kernel launchers behind the C ABI.
#pragma once

#include "imgstencil.h"

namespace is {

enum KernelId {
  kGenericNchwF32 = 0,   // one thread per output, any shape (fallback)
  kGenericNhwcF16 = 1,   // one thread per output, any shape (fallback)
  kSingleChannel = 2,    // C = 1, fp32 NCHW: K = 1 with r, s <= 7, or K = 2, 4, 8 filters
  kMultiChannel = 3,     // fp32 NCHW register-blocked, C, K multiples of the block
  kMfmaNhwcF16 = 4,      // fp16 NHWC implicit GEMM on MFMA
  kMfmaNchwF32 = 5,      // fp32 NCHW 32 -> 32 3x3 implicit GEMM on the fp32 MFMA
  kHeadNhwcF16 = 6,      // fp16 NHWC first layer, 1 -> K, one MFMA k step over the taps
  kPointwise = 7,        // fp32 NCHW 1x1 filters over several channels
  kHeadNchwF32 = 8,      // fp32 NCHW first layer, 1 -> K, fp32 MFMA k steps over the taps
  kMultiMfmaF32 = 9      // fp32 NCHW, 4 filters per workgroup on the fp32 4x4x1 MFMA
};

struct Plan {
  conv2d_desc d;
  KernelId kid;
  const char *name;
  int grid_x, grid_y, grid_z;
  int block;
  int lds;
  int tile_w, tile_h;
  // Kernel-specific geometry.
  int nseg, nstrip, ntiles;   // column segments, row strips, total tiles
  int strip_rows;             // output rows per strip
  int vec;                    // 1 = 16-byte vector path
  int kvalid;                 // fp16 MFMA layer: output channels with weights (the rest are 0)
};

// Workgroups of a persistent kernel that walks `units` work units with one
// workgroup per CU: the CU count rounded down to a multiple of 8 (the kernels
// deal their units to 8 groups of workgroups, one group per XCD on a whole
// MI355X, so the grid must stay a multiple of 8), or fewer when the units
// need fewer: units rounded up to a multiple of 8; at least 8. Plans record it
// for 256 CUs; the launchers recompute it for the current device.
int persistent_grid(int units, int cus);
// Compute units of the current device, cached per device (256 when the runtime
// cannot tell).
int device_cu_count();

// conv_chain_forward with the caller's workspace (the whole entry point: checks
// and launches); shared by the entry points that bring their own workspace.
is_status chain_forward(const conv_chain_desc *d, const void *x, const void *const *w, const float *const *b,
                        void *y, void *workspace, size_t workspace_bytes, hipStream_t stream);
// IS_OK for hipSuccess, else IS_ERR_HIP with the error kept for is_last_hip_error.
is_status report_hip(hipError_t e);

// Each kernel family fills the launch geometry of a plan it accepts and
// launches it. configure_* return false when the family cannot run the desc.
// `param` selects one of the family's tile variants (0: the default choice):
// strip rows for the single-channel kernel, output channels per workgroup for
// the multi-channel kernel, LDS swizzle row bytes for the fp16 MFMA kernel;
// a family without variants ignores it.
bool configure_generic(Plan &p);
hipError_t launch_generic(const Plan &p, const void *x, const void *w, const float *b, void *y,
                          hipStream_t s);

bool configure_single(Plan &p, int param = 0);
hipError_t launch_single(const Plan &p, const float *x, const float *w, const float *b, float *y,
                         hipStream_t s);

bool configure_multi(Plan &p, int param = 0);
hipError_t launch_multi(const Plan &p, const float *x, const float *w, const float *b, float *y,
                        hipStream_t s);
// The multi-channel layer's products on the matrix cores, 4 filters per
// workgroup (any C, K and W; 3x3, 5x5 or 7x7). use: kMfPlan
// where it is the plan's first choice (an even channel count from 4 on, or 7x7
// from 2 channels: the vector form has no 7x7), kMfVariant for
// the tuning variants (2 channels or more), kMfLastResort for the plan of
// shapes that no other kernel but the one-thread-per-output fallback takes.
enum { kMfPlan = 0, kMfVariant = 1, kMfLastResort = 2 };
bool configure_multi_mf(Plan &p, int use = kMfPlan);
hipError_t launch_multi_mf(const Plan &p, const float *x, const float *w, const float *b, float *y,
                           hipStream_t s);
// The multi-channel layer (either path) with 4 output channels followed by a
// 2x depth-to-space (y: N x 1 x 2H x 2W), in one launch.
bool multi_d2s_supported(const Plan &p);
hipError_t launch_multi_d2s(const Plan &p, const float *x, const float *w, const float *b, float *y,
                            hipStream_t s);

bool configure_mfma(Plan &p, int param = 0);
hipError_t launch_mfma(const Plan &p, const _Float16 *x, const _Float16 *w, const float *b, _Float16 *y,
                       hipStream_t s);

// The (32 -> 16) layer whose first 9 channels go through a 3x3 depth-to-space
// (y: N x 3H x 3W fp16), in one launch: the last layer of the pages' net.
bool mfma_d2s3_supported(const Plan &p);
hipError_t launch_mfma_d2s3(const Plan &p, const _Float16 *x, const _Float16 *w, const float *b, _Float16 *y,
                            hipStream_t s);

// The fp16 MFMA layer (plan p: 64 -> 64, 3x3) fed by a first layer
// 1 -> 64 with an r x r filter (r = 3 or 5) computed inside the same launch
// from the one-channel image x1 (N x H x W fp16): its weights wh (64 x 1 x r x r
// fp16), bias bh (64 fp32 or null) and ReLU flag. The first layer's output is
// rounded to fp16 as if it were stored, and never leaves the chip.
bool mfma_head_supported(const Plan &p, int head_r);
hipError_t launch_mfma_head(const Plan &p, const _Float16 *x1, const _Float16 *wh, const float *bh, int relu_h,
                            int head_r, const _Float16 *w, const float *b, _Float16 *y, hipStream_t s);

bool configure_head_f32(Plan &p);
hipError_t launch_head_f32(const Plan &p, const float *x, const float *w, const float *b, float *y,
                           hipStream_t s);
bool configure_head_f16(Plan &p);
hipError_t launch_head_f16(const Plan &p, const _Float16 *x, const _Float16 *w, const float *b, _Float16 *y,
                           hipStream_t s);

bool configure_pointwise(Plan &p, int param = 0);
hipError_t launch_pointwise(const Plan &p, const float *x, const float *w, const float *b, float *y,
                            hipStream_t s);

bool configure_mfma_f32(Plan &p);
hipError_t launch_mfma_f32(const Plan &p, const float *x, const float *w, const float *b, float *y,
                           hipStream_t s);

// The fused upscaling chain (1->32 5x5, 32->32 3x3 twice, 32->4 3x3, depth-to-space x2).
bool chain_fused_supported(const conv_chain_desc *d);
hipError_t launch_chain_fused(const conv_chain_desc *d, const float *x, const float *const *w,
                              const float *const *b, float *y, hipStream_t s);

// Two or three consecutive single-channel layers (1 -> 1, r = s in {3, 5, 7}
// with at most one 7, fp32 NCHW, W % 4 == 0) of a chain, fused in one pass: layers
// [first, first + count) of d, reading x and writing y (N x 1 x H x W).
struct FusedStencilGeo {
  bool ok;
  int lanes_off, step;        // overlap lanes per side; output columns per window
  int nseg, nstrip, ntiles;   // windows per row, strips, waves
  int strip_rows;
};
FusedStencilGeo fused_stencil_geometry(const conv_chain_desc *d, int first, int count);
hipError_t launch_fused_stencil(const conv_chain_desc *d, int first, int count, const float *x,
                                const float *const *w, const float *const *b, float *y, hipStream_t s);

// out[n,0,f*i+dy,f*j+dx] = z[n,f*dy+dx,i,j] for z of N x f*f x H x W fp32.
hipError_t launch_depth_to_space(const float *z, float *out, int N, int H, int W, int f, hipStream_t s);
// The same for NHWC fp16: z is N x H x W x zc (channels f*dy+dx among zc >= f*f),
// out is N x f*H x f*W x 1.
hipError_t launch_depth_to_space_f16(const _Float16 *z, _Float16 *out, int N, int H, int W, int f, int zc,
                                     hipStream_t s);

}  // namespace is
