/*
 * imgstencil.h -- C ABI of the MI355X (gfx950) direct 2D convolution library.
 *
 * The operation (every entry point below computes it, or a chain of it):
 *
 *   y[n,k,i,j] = act( sum_{c,u,v} w[k,c,u,v] * x[n,c,i+u-(R-1)/2,j+v-(S-1)/2] + b[k] )
 *
 * with x read as zero outside the HxW image (same-size output, stride 1,
 * centred window, no filter flip) and act = ReLU or identity. This is the
 * per-output-pixel loop nest of "Optimizing convolution kernels - CNNs in
 * Vulkan Part 2/3" (StreamHPC), section "Where we left off": loops over output
 * channel, input channel, kernel row and kernel column; input pixel = output
 * pixel + kernel offset - kernel size / 2; bias added to the finished sum; ReLU
 * by the apply_relu switch of its "Vectorization" section. The single-channel
 * case is the "special case" (one input channel) of "Optimizing Memory
 * Efficiency for Convolution Kernels on Kepler GPUs" (arXiv 1705.10591) and the
 * multi-channel case its "general case".
 *
 * Conventions for every entry point:
 *  - Tensors are caller-owned DEVICE memory, dense and contiguous, with the
 *    base address aligned to 16 bytes (else IS_ERR_MISALIGNED). The library
 *    never allocates device memory on a forward call and keeps no pointer
 *    after the call returns.
 *  - Weights are K,C,R,S (row-major, contiguous) in the input dtype (a
 *    separable filter: its R column taps then its S row taps). Bias is K fp32
 *    values or NULL (no bias).
 *  - Accumulation is always fp32. fp16 outputs are rounded to nearest even.
 *  - Calls only enqueue work on the given stream (0 = the null stream): no host
 *    synchronisation, no allocation. The one exception is conv2d_autotune,
 *    which times on the stream and waits for it. Launch errors return IS_ERR_HIP and
 *    is_last_hip_error() gives the hipError_t. Faults inside a kernel surface
 *    at the caller's next synchronisation.
 *  - No exception crosses this boundary; every function returns a status.
 *  - Input and output must not overlap (IS_ERR_INVALID_ARG when x and y
 *    ranges intersect).
 */
#ifndef IMGSTENCIL_H
#define IMGSTENCIL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IS_VERSION 1
#define IS_MAX_CHAIN 8

typedef enum {
  IS_OK = 0,
  IS_ERR_INVALID_ARG = 1,   /* null pointer, bad size, overlap, bad padding/stride */
  IS_ERR_UNSUPPORTED = 2,   /* valid request this library does not implement (even filters, ...) */
  IS_ERR_MISALIGNED = 3,    /* a tensor base address is not 16-byte aligned */
  IS_ERR_HIP = 4,           /* the HIP runtime reported an error at launch */
  IS_ERR_NO_MEMORY = 5,     /* host allocation of a plan failed */
  IS_ERR_WORKSPACE = 6      /* workspace missing or smaller than required */
} is_status;

typedef enum { IS_F32 = 0, IS_F16 = 1 } is_dtype;
typedef enum { IS_NCHW = 0, IS_NHWC = 1 } is_layout;

/* One convolution layer.
 *  n, c, h, w : input batch, channels, height, width (h, w may be 0: empty, no work)
 *  k, r, s    : output channels, filter height, filter width (r and s odd, >= 1)
 *  pad_h/pad_w: must equal (r-1)/2 and (s-1)/2 (same-size zero padding)
 *  stride_h/w : must be 1
 *  in_dtype / out_dtype: (IS_F32, IS_F32) with layout IS_NCHW, or
 *                        (IS_F16, IS_F16) with layout IS_NHWC
 *  layout     : memory order of x and y: NCHW (x[n][c][i][j]) or NHWC (x[n][i][j][c])
 *  relu       : 0 = identity, 1 = ReLU after the bias
 *  separable  : 0 = a full R x S filter per (k, c); 1 = a separable filter, the
 *               outer product w[i][j] = col[i] * row[j] of a column filter of R
 *               taps and a row filter of S taps, evaluated as a row pass and a
 *               column pass ("Optimizing Memory Efficiency for Convolution
 *               Kernels on Kepler GPUs", arXiv 1705.10591, special case of one
 *               channel): single channel only (c = k = 1, fp32 NCHW, r = s in
 *               {3, 5, 7}); w then holds the R column taps followed by the S
 *               row taps. Other shapes: IS_ERR_UNSUPPORTED.                     */
typedef struct {
  int n, c, h, w;
  int k, r, s;
  int pad_h, pad_w;
  int stride_h, stride_w;
  is_dtype in_dtype, out_dtype;
  is_layout layout;
  int relu;
  int separable;
} conv2d_desc;

typedef struct conv2d_plan_s *conv2d_plan;

/* What a plan will launch (read-only, for tests and measurement). */
typedef struct {
  char kernel[64];        /* device kernel family name, e.g. "is_k1_single" */
  int grid_x, grid_y, grid_z;   /* persistent kernels record their grid for 256 CUs; a
                                   launch sizes it for the device: is_k4_mfma and
                                   is_k5_mfma_f32 is_persistent_grid(units, CUs),
                                   is_k6_head_f16 min(tiles, CUs) */
  int block;              /* threads per workgroup */
  int lds_bytes;          /* LDS per workgroup */
  int tile_w, tile_h;     /* output pixels per wave or workgroup tile */
  double flops;           /* algorithmic: 2*N*K*C*R*S*H*W (separable: 2*N*(R+S)*H*W) */
  double bytes;           /* algorithmic: x + y + w + b, each once */
} conv2d_plan_info;

/* Validate a descriptor and choose a kernel, a tile and a grid. Host only: runs
 * without a GPU. On success *out receives a plan that the caller releases with
 * conv2d_destroy. A plan is immutable and may be used from several threads and
 * streams at once. Errors: IS_ERR_INVALID_ARG (null, negative sizes, c or k < 1,
 * wrong padding, stride != 1), IS_ERR_UNSUPPORTED (even r or s, dtype/layout
 * pair not listed above, r or s > 31), IS_ERR_NO_MEMORY. */
is_status conv2d_create(const conv2d_desc *d, conv2d_plan *out);

/* Enqueue y = act(conv(x, w) + bias) on `stream`.
 *  x: input in the plan's layout and dtype, N*C*H*W elements
 *  w: K*C*R*S weights in the input dtype (separable plans: R + S fp32 values,
 *     the column taps then the row taps)
 *  bias: K fp32 values, or NULL
 *  y: output in the plan's layout and dtype, N*K*H*W elements (written in full)
 * Errors: IS_ERR_INVALID_ARG (null plan/x/w/y, x and y overlap),
 * IS_ERR_MISALIGNED, IS_ERR_HIP. */
is_status conv2d_forward(conv2d_plan plan, const void *x, const void *w,
                         const float *bias, void *y, hipStream_t stream);

/* Release a plan (NULL is ignored). */
void conv2d_destroy(conv2d_plan plan);

/* Describe what a plan launches. */
is_status conv2d_get_plan_info(conv2d_plan plan, conv2d_plan_info *info);

/* Runtime tile tuning. "Optimizing Memory Efficiency for Convolution Kernels on
 * Kepler GPUs" (arXiv 1705.10591, the results of its special-case kernel)
 * picks its block size by a design-space search, and "Optimizing convolution
 * kernels - CNNs in Vulkan Part 2/3" (section "Some notes on workgroup sizes")
 * its workgroup shape by measurement, proposing that an implementation
 * benchmark configurations at run time. Here a descriptor has a list of
 * variants, every kernel configuration that can run it, and conv2d_autotune
 * times them all on the caller's buffers and keeps the fastest. The search is
 * an entry point of its own rather than part of conv2d_create, which runs on
 * the host without a GPU.
 *  kernel     : kernel family, as in conv2d_plan_info
 *  param      : the family's tuning parameter: output rows per strip
 *               (is_k1_single, is_k1_single_separable, is_k1_single_fanout: one
 *               channel, 2, 4 or 8 filters), output channels per
 *               workgroup (is_k2_multi), LDS swizzle row bytes, 0 = none
 *               (is_k4_mfma); 0 for the others
 *  is_default : 1 for the variant conv2d_create chooses (always index 0)
 *  ms         : time per launch measured by conv2d_autotune (0 otherwise)     */
typedef struct {
  char kernel[64];
  int param;
  int is_default;
  float ms;
} conv2d_variant;

/* List the variants of a descriptor, the default first. Host only (no GPU).
 * *count receives the number of variants; the first min(max, *count) are
 * written to out (out may be NULL when max is 0). Errors: those of
 * conv2d_create, IS_ERR_INVALID_ARG (null count, max < 0). */
is_status conv2d_list_variants(const conv2d_desc *d, conv2d_variant *out, int max, int *count);

/* conv2d_create for variant `index` of conv2d_list_variants. Errors: those of
 * conv2d_create, IS_ERR_INVALID_ARG (index out of range). */
is_status conv2d_create_variant(const conv2d_desc *d, int index, conv2d_plan *out);

/* Time every variant of the plan's descriptor on these buffers (one warm-up
 * launch, then `reps` launches between two HIP events on `stream`) and make
 * the plan use the fastest. Arguments as for conv2d_forward; y is overwritten
 * and, when the call returns IS_OK, holds the chosen variant's result (its
 * last launch is enqueued on `stream`). Unlike conv2d_forward this call
 * synchronises with the stream's work (hipEventSynchronize) and creates two
 * events; it allocates no device memory. It changes the plan: do not call it
 * while another thread uses the same plan, nor inside a stream capture.
 * out/max/count: as for conv2d_list_variants, with the measured times (count
 * may be NULL). Errors: those of conv2d_forward, IS_ERR_INVALID_ARG
 * (reps < 1); on error the plan is unchanged. */
is_status conv2d_autotune(conv2d_plan plan, const void *x, const void *w, const float *bias, void *y,
                          hipStream_t stream, int reps, conv2d_variant *out, int max, int *count);

/* A chain of layers applied one after another, each reading the previous
 * layer's output: z_0 = x, z_l = act_l(conv_l(z_{l-1}) + b_l), and finally an
 * optional depth-to-space by f = `depth_to_space` (2 or 3) that turns the last
 * layer's f*f channels of HxW into one channel of fHxfW with
 * out[n,0,f*i+dy,f*j+dx] = z[n,f*dy+dx,i,j]. This is the neural upscaling
 * network of the same StreamHPC page (introduction; layer table of "Reducing
 * memory traffic": 1 -> 64 5x5, 64 -> 64, 64 -> 32, 32 -> 9 3x3, whose 9
 * output channels are taken as a 3x3 sub-pixel upscale), and the fused
 * evaluation follows the warp-sized overlapped tiles with loop fusion of
 * "Model-Based Warp Overlapped Tiling for Image Processing Programs on GPUs"
 * (arXiv 1909.07190, abstract).
 *  Layer l reads layer[l].c channels (layer[0].c = input channels, layer[l].c
 *  = layer[l-1].k), has layer[l].k outputs, odd r == s, and ReLU if relu != 0.
 *  dtype: IS_F32 (NCHW tensors, fp32 weights and biases) or IS_F16 (NHWC
 *  tensors, fp16 weights, fp32 biases; every layer's output is rounded to fp16
 *  as the page's "Reducing memory traffic" step stores it). IS_F16 chains run
 *  layer by layer, except that in IS_CHAIN_AUTO a first layer 1 -> 64 (3x3 or
 *  5x5) followed by a 64 -> 64 3x3 layer runs as one launch in which the first
 *  layer's fp16 output is computed where the second layer reads it and never
 *  written to memory (IS_CHAIN_UNFUSED keeps one launch per layer).
 * Stencil pipelines: a fp32 chain whose layers all map one channel to one
 * (c = k = 1) and has no depth-to-space is an image-processing pipeline of
 * filters, the programs of the same arXiv 1909.07190. It runs in groups of 1
 * to 3 consecutive layers, one launch each: 2 or 3 layers with r = s in
 * {3, 5} and W % 4 == 0 can be fused into one pass over warp-overlapped
 * tiles that keeps the intermediate images on chip. IS_CHAIN_AUTO chooses the
 * groups with a roofline model of each launch (conv_chain_groups reports
 * them), IS_CHAIN_FUSED asks for one group of the whole chain, and
 * IS_CHAIN_UNFUSED for one launch per layer. */
typedef struct { int c, k, r, s, relu; } conv_layer_desc;

typedef enum {
  IS_CHAIN_AUTO = 0,     /* layer by layer when the workspace allows it (the faster path on
                            MI355X), else the fused kernel if the chain has one */
  IS_CHAIN_FUSED = 1,    /* fused only (IS_ERR_UNSUPPORTED if no fused kernel fits) */
  IS_CHAIN_UNFUSED = 2   /* one conv2d launch per layer through the workspace */
} is_chain_mode;

typedef struct {
  int n, h, w, n_layers;
  conv_layer_desc layer[IS_MAX_CHAIN];
  int depth_to_space;    /* 1 = none, f = 2 or 3: x f on the last layer (needs its k == f*f) */
  is_dtype dtype;
  is_chain_mode mode;
} conv_chain_desc;

/* Device bytes of workspace conv_chain_forward wants for this chain and mode:
 * 0 for IS_CHAIN_FUSED; the two intermediate tensors of the layer-by-layer
 * path for IS_CHAIN_UNFUSED and IS_CHAIN_AUTO (with less, AUTO runs the fused
 * kernel when the chain has one, and fails with IS_ERR_WORKSPACE otherwise).
 * Stencil pipelines: one intermediate image per group boundary, at most two
 * (none for a single group); with less, AUTO runs the whole chain as one
 * fused group when it can. */
is_status conv_chain_workspace_size(const conv_chain_desc *d, size_t *bytes);

/* The launch groups of the chain in order, as sizes in layers (host only):
 * *count receives their number and the first min(max, *count) sizes are
 * written to sizes. Stencil pipelines: the grouping of the mode (AUTO: the
 * model's choice, for the workspace conv_chain_workspace_size reports); other
 * chains: one group (IS_CHAIN_FUSED) or one per layer. Errors: those of
 * conv_chain_workspace_size, IS_ERR_INVALID_ARG (null count, max < 0). */
is_status conv_chain_groups(const conv_chain_desc *d, int *sizes, int max, int *count);

/* Enqueue the chain on `stream`.
 *  x: N x layer[0].c x H x W fp32 input (IS_F16: N x H x W x layer[0].c fp16)
 *  w[l], b[l]: host arrays of n_layers device pointers (b[l] may be NULL)
 *  y: N x layer[last].k x H x W, or N x 1 x fH x fW with depth_to_space = f
 *     (IS_F16: N x H x W x layer[last].k, or N x fH x fW x 1)
 *  workspace: device memory of at least conv_chain_workspace_size bytes, or
 *             NULL when that size is 0
 * Errors: as conv2d_forward, plus IS_ERR_WORKSPACE and IS_ERR_UNSUPPORTED. */
is_status conv_chain_forward(const conv_chain_desc *d, const void *x,
                             const void *const *w, const float *const *b,
                             void *y, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Bytes of device workspace the library owns for conv_chain_forward_noalloc:
 * one array of this size on every device the library runs on, held until the
 * process ends (256 MiB, under 0.1% of an MI355X's 288 GB). */
#define IS_NOALLOC_MAX_WORKSPACE ((size_t)256 << 20)

/* conv_chain_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The same chain and the same kernels, with the layer-by-layer
 * intermediates in the library's own workspace of IS_NOALLOC_MAX_WORKSPACE
 * bytes instead of the caller's. Arguments and results as conv_chain_forward
 * without the workspace arguments. It allocates nothing: no hipMalloc, hipFree
 * or allocating library call.
 *  - A chain whose conv_chain_workspace_size exceeds IS_NOALLOC_MAX_WORKSPACE
 *    is rejected with IS_ERR_WORKSPACE, before any GPU call (a 1280x720 frame
 *    through the upscaling chain, fp32 or fp16, needs 225 MiB).
 *  - `stream` must belong to the current device (else IS_ERR_INVALID_ARG): the
 *    workspace's address on a device is looked up once, by the first call on
 *    that device (hipGetSymbolAddress); make that first call outside a stream
 *    capture.
 *  - Every call on one device shares that device's workspace, which keeps the
 *    last call's intermediates; nothing in it needs clearing (each layer writes
 *    its whole output before the next layer reads it). Calls that overlap in
 *    time on one device (on different streams, or from different host
 *    threads) race on it: serialise them, e.g. on one stream.
 * Errors: those of conv_chain_forward, and IS_ERR_WORKSPACE as above. */
is_status conv_chain_forward_noalloc(const conv_chain_desc *d, const void *x,
                                     const void *const *w, const float *const *b,
                                     void *y, hipStream_t stream);

/* Name of the kernel family conv_chain_forward launches for this chain when
 * given the workspace conv_chain_workspace_size reports ("is_k3_chain" when
 * fused, "head_fused" for an fp16 chain whose first two layers run as one
 * launch, "layer_by_layer" otherwise; stencil pipelines: see
 * conv_chain_groups), copied into name[0..len-1]. */
is_status conv_chain_kernel_name(const conv_chain_desc *d, char *name, size_t len);

/* LDS bytes of an input tile that covers tile_w x tile_h outputs of a filter
 * r x s over `channels` channels of `elem_bytes` each: the tile plus its halo,
 * (tile_w + s - 1) * (tile_h + r - 1) * channels * elem_bytes. The sizing rule
 * of the shared-memory table in "Some notes on workgroup sizes" (StreamHPC
 * page). Returns 0 for non-positive arguments. */
size_t is_lds_tile_bytes(int tile_w, int tile_h, int r, int s, int channels, int elem_bytes);

/* XOR swizzle of an LDS index, the formula of "CUDA shared memory swizzling"
 * (section on the swizzling formula): for an array T a[][nx] with
 * nx * elem_bytes a power of two >= 32 and chunks of chunk_bytes (a power of
 * two, elem_bytes <= chunk_bytes <= nx * elem_bytes), element [y][x] is stored
 * at column x_swz of row y. The same function the device code uses.
 * Returns -1 for arguments outside those rules. */
int is_swizzle_col(int y, int x, int nx, int elem_bytes, int chunk_bytes);

/* Workgroups a persistent kernel launches for `units` work units (tiles or
 * strips that the workgroups take in turn) on a device of `cus` compute units:
 * one per CU, the CU count rounded down to a multiple of 8 (units are dealt to
 * 8 groups of workgroups, one group per XCD of a whole MI355X, so the grid
 * stays a multiple of 8), or units rounded up to a multiple of 8 when that is
 * fewer; at least 8. Host only; 0 for non-positive arguments. */
int is_persistent_grid(int units, int cus);

const char *is_status_str(is_status st);
int is_last_hip_error(void);   /* hipError_t of this thread's most recent IS_ERR_HIP */
int is_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IMGSTENCIL_H */
