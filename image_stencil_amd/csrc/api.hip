// api.hip -- the C ABI: descriptor validation, kernel choice and launch.
#include <algorithm>
#include <new>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "common.hpp"
#include "internal.hpp"

struct conv2d_plan_s {
  is::Plan p;
};

namespace {

thread_local int g_last_hip_error = 0;

is_status hip_status(hipError_t e) {
  if (e == hipSuccess) return IS_OK;
  g_last_hip_error = (int)e;
  return IS_ERR_HIP;
}

bool log_enabled() {
  static const int on = [] {
    const char *v = getenv("IMGSTENCIL_LOG");
    return v && v[0] == '1';
  }();
  return on;
}

constexpr int kMaxDevices = 64;
int g_device_cus[kMaxDevices];   // 0 = not read yet

size_t elem_size(is_dtype t) { return t == IS_F16 ? 2 : 4; }

is_status validate(const conv2d_desc *d) {
  if (!d) return IS_ERR_INVALID_ARG;
  if (d->n < 0 || d->h < 0 || d->w < 0 || d->c < 1 || d->k < 1 || d->r < 1 || d->s < 1)
    return IS_ERR_INVALID_ARG;
  if (d->stride_h != 1 || d->stride_w != 1) return IS_ERR_INVALID_ARG;
  if ((d->r % 2) == 0 || (d->s % 2) == 0) return IS_ERR_UNSUPPORTED;
  if (d->pad_h != (d->r - 1) / 2 || d->pad_w != (d->s - 1) / 2) return IS_ERR_INVALID_ARG;
  if (d->r > 31 || d->s > 31) return IS_ERR_UNSUPPORTED;
  if (d->relu != 0 && d->relu != 1) return IS_ERR_INVALID_ARG;
  if (d->separable != 0 && d->separable != 1) return IS_ERR_INVALID_ARG;
  const bool f32 = d->in_dtype == IS_F32 && d->out_dtype == IS_F32 && d->layout == IS_NCHW;
  const bool f16 = d->in_dtype == IS_F16 && d->out_dtype == IS_F16 && d->layout == IS_NHWC;
  if (!f32 && !f16) return IS_ERR_UNSUPPORTED;
  // Separable filters: the single-channel fp32 kernel only.
  if (d->separable && (!f32 || d->c != 1 || d->k != 1 || d->r != d->s || d->r < 3 || d->r > 7))
    return IS_ERR_UNSUPPORTED;
  // Element counts must stay addressable with 64-bit offsets and 32-bit grids.
  const double in_elems = (double)d->n * d->c * d->h * d->w;
  const double out_elems = (double)d->n * d->k * d->h * d->w;
  if (in_elems > 4.0e12 || out_elems > 4.0e12) return IS_ERR_UNSUPPORTED;
  return IS_OK;
}

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return na && nb && a0 < b0 + nb && b0 < a0 + na;
}

void fill_info(const is::Plan &p, conv2d_plan_info *info) {
  memset(info, 0, sizeof(*info));
  snprintf(info->kernel, sizeof(info->kernel), "%s", p.name);
  info->grid_x = p.grid_x;
  info->grid_y = p.grid_y;
  info->grid_z = p.grid_z;
  info->block = p.block;
  info->lds_bytes = p.lds;
  info->tile_w = p.tile_w;
  info->tile_h = p.tile_h;
  const conv2d_desc &d = p.d;
  const double taps = d.separable ? (double)(d.r + d.s) : (double)d.r * d.s;
  info->flops = 2.0 * d.n * d.k * d.c * taps * (double)d.h * d.w;
  const double es = (double)elem_size(d.in_dtype);
  info->bytes = es * ((double)d.n * d.c * d.h * d.w + (double)d.n * d.k * d.h * d.w +
                      (double)d.k * d.c * taps) +
                4.0 * d.k;
}

is_status make_plan(const conv2d_desc *d, is::Plan &p) {
  const is_status st = validate(d);
  if (st != IS_OK) return st;
  memset(&p, 0, sizeof(p));
  p.d = *d;
  if (d->separable) {
    // Only the single-channel kernel evaluates separable filters.
    if (!is::configure_single(p)) return IS_ERR_UNSUPPORTED;
  } else if (!is::configure_single(p) && !is::configure_head_f32(p) && !is::configure_mfma_f32(p) &&
             !is::configure_pointwise(p) && !is::configure_multi_mf(p) &&
             !is::configure_multi(p) && !is::configure_mfma(p) && !is::configure_head_f16(p) &&
             !is::configure_multi_mf(p, is::kMfLastResort)) {
    is::configure_generic(p);
  }
  if (log_enabled())
    fprintf(stderr, "[imgstencil] n=%d c=%d h=%d w=%d k=%d r=%d s=%d -> %s grid=%d block=%d lds=%d\n",
            d->n, d->c, d->h, d->w, d->k, d->r, d->s, p.name, p.grid_x, p.block, p.lds);
  return IS_OK;
}

// ---- Tile variants (runtime tuning) ----------------------------------------
//
// A variant is a kernel family and its tuning parameter as the ABI reports it:
// strip rows (single channel), output channels per workgroup (multi-channel),
// LDS swizzle row bytes with 0 = none (fp16 MFMA), 0 for the others.
struct Variant {
  is::KernelId kid;
  int param;
};

int public_param(const is::Plan &p) {
  switch (p.kid) {
    case is::kSingleChannel:
    case is::kMultiChannel:
    case is::kPointwise: return p.strip_rows;
    case is::kMfmaNhwcF16: return p.vec;
    default: return 0;
  }
}

bool configure_variant(is::Plan &p, const conv2d_desc &d, const Variant &v) {
  memset(&p, 0, sizeof(p));
  p.d = d;
  switch (v.kid) {
    case is::kSingleChannel: return is::configure_single(p, v.param);
    case is::kMultiChannel: return !d.separable && is::configure_multi(p, v.param);
    case is::kMfmaNhwcF16: return !d.separable && is::configure_mfma(p, v.param == 0 ? -1 : v.param);
    case is::kMfmaNchwF32: return !d.separable && is::configure_mfma_f32(p);
    case is::kPointwise: return is::configure_pointwise(p, v.param);
    case is::kHeadNhwcF16: return !d.separable && is::configure_head_f16(p);
    case is::kHeadNchwF32: return is::configure_head_f32(p);
    case is::kMultiMfmaF32: return is::configure_multi_mf(p, is::kMfVariant);
    default:
      if (d.separable) return false;
      is::configure_generic(p);
      return true;
  }
}

// Every configuration that can run the (validated) descriptor, the default
// plan's first, each once. The one-thread-per-output fallback is listed only
// when no other kernel takes the shape (it is never the faster one, and on
// large layers one timing of it would take longer than all the others).
int collect_variants(const conv2d_desc &d, const is::Plan &def, Variant *out, int max) {
  int n = 0;
  auto add = [&](const is::Plan &p) {
    const Variant v{p.kid, public_param(p)};
    for (int i = 0; i < n; ++i)
      if (out[i].kid == v.kid && out[i].param == v.param) return;
    if (n < max) out[n++] = v;
  };
  add(def);
  is::Plan p;
  const Variant tries[] = {
      {is::kSingleChannel, 4}, {is::kSingleChannel, 8}, {is::kSingleChannel, 16},
      {is::kSingleChannel, 32}, {is::kSingleChannel, 64}, {is::kSingleChannel, 128},
      {is::kMfmaNchwF32, 0},
      {is::kPointwise, 32}, {is::kPointwise, 16}, {is::kPointwise, 8}, {is::kPointwise, 4},
      {is::kMultiChannel, 32}, {is::kMultiChannel, 16}, {is::kMultiChannel, 8}, {is::kMultiChannel, 4},
      {is::kMultiChannel, 2},
      {is::kMfmaNhwcF16, 128}, {is::kMfmaNhwcF16, 0}, {is::kMfmaNhwcF16, 256},
      {is::kHeadNhwcF16, 0}, {is::kHeadNchwF32, 0}, {is::kMultiMfmaF32, 0}};
  for (const Variant &v : tries)
    if (configure_variant(p, d, v)) add(p);
  return n;
}

constexpr int kMaxVariants = 32;

// Plan of variant i: the default plan itself for i = 0 (a kernel family can
// take a shape as the plan's last resort that its variant listing leaves out),
// else the family's configuration.
void variant_plan(is::Plan &p, const conv2d_desc &d, const is::Plan &def, const Variant *v, int i) {
  if (i == 0)
    p = def;
  else
    configure_variant(p, d, v[i]);
}

void fill_variant(const is::Plan &p, bool is_default, float ms, conv2d_variant *out) {
  memset(out, 0, sizeof(*out));
  snprintf(out->kernel, sizeof(out->kernel), "%s", p.name);
  out->param = public_param(p);
  out->is_default = is_default ? 1 : 0;
  out->ms = ms;
}

// The argument checks of a forward call (no GPU involved).
is_status check_forward_args(const conv2d_desc &d, const void *x, const void *w, const float *bias,
                             const void *y) {
  if (!x || !w || !y) return IS_ERR_INVALID_ARG;
  if (misaligned(x) || misaligned(w) || misaligned(y) || (bias && misaligned(bias)))
    return IS_ERR_MISALIGNED;
  const size_t es = elem_size(d.in_dtype);
  const size_t xb = es * (size_t)d.n * d.c * d.h * d.w;
  const size_t yb = es * (size_t)d.n * d.k * d.h * d.w;
  if (overlap(x, xb, y, yb)) return IS_ERR_INVALID_ARG;
  return IS_OK;
}

is_status run_plan(const is::Plan &p, const void *x, const void *w, const float *bias, void *y,
                   hipStream_t stream) {
  const conv2d_desc &d = p.d;
  const is_status chk = check_forward_args(d, x, w, bias, y);
  if (chk != IS_OK) return chk;
  const size_t es = elem_size(d.in_dtype);
  const size_t xb = es * (size_t)d.n * d.c * d.h * d.w;
  const size_t yb = es * (size_t)d.n * d.k * d.h * d.w;
  if (xb == 0 || yb == 0) return IS_OK;   // empty image: nothing to compute
  hipError_t e;
  switch (p.kid) {
    case is::kSingleChannel:
      e = is::launch_single(p, static_cast<const float *>(x), static_cast<const float *>(w), bias,
                            static_cast<float *>(y), stream);
      break;
    case is::kMultiChannel:
      e = is::launch_multi(p, static_cast<const float *>(x), static_cast<const float *>(w), bias,
                           static_cast<float *>(y), stream);
      break;
    case is::kMfmaNchwF32:
      e = is::launch_mfma_f32(p, static_cast<const float *>(x), static_cast<const float *>(w), bias,
                              static_cast<float *>(y), stream);
      break;
    case is::kMfmaNhwcF16:
      e = is::launch_mfma(p, static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(w), bias,
                          static_cast<_Float16 *>(y), stream);
      break;
    case is::kPointwise:
      e = is::launch_pointwise(p, static_cast<const float *>(x), static_cast<const float *>(w), bias,
                               static_cast<float *>(y), stream);
      break;
    case is::kHeadNhwcF16:
      e = is::launch_head_f16(p, static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(w), bias,
                              static_cast<_Float16 *>(y), stream);
      break;
    case is::kHeadNchwF32:
      e = is::launch_head_f32(p, static_cast<const float *>(x), static_cast<const float *>(w), bias,
                              static_cast<float *>(y), stream);
      break;
    case is::kMultiMfmaF32:
      e = is::launch_multi_mf(p, static_cast<const float *>(x), static_cast<const float *>(w), bias,
                              static_cast<float *>(y), stream);
      break;
    default:
      e = is::launch_generic(p, x, w, bias, y, stream);
      break;
  }
  return hip_status(e);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Checks a chain descriptor and returns the conv2d_desc of each layer.
is_status chain_layers(const conv_chain_desc *d, conv2d_desc *ld) {
  if (!d) return IS_ERR_INVALID_ARG;
  if (d->n_layers < 1 || d->n_layers > IS_MAX_CHAIN || d->n < 0 || d->h < 0 || d->w < 0)
    return IS_ERR_INVALID_ARG;
  if (d->dtype != IS_F32 && d->dtype != IS_F16) return IS_ERR_UNSUPPORTED;
  if (d->depth_to_space < 1 || d->depth_to_space > 3) return IS_ERR_UNSUPPORTED;
  if (d->mode != IS_CHAIN_AUTO && d->mode != IS_CHAIN_FUSED && d->mode != IS_CHAIN_UNFUSED)
    return IS_ERR_INVALID_ARG;
  for (int l = 0; l < d->n_layers; ++l) {
    const conv_layer_desc &L = d->layer[l];
    if (l > 0 && L.c != d->layer[l - 1].k) return IS_ERR_INVALID_ARG;
    conv2d_desc &c = ld[l];
    memset(&c, 0, sizeof(c));
    c.n = d->n; c.c = L.c; c.h = d->h; c.w = d->w;
    c.k = L.k; c.r = L.r; c.s = L.s;
    c.pad_h = (L.r - 1) / 2; c.pad_w = (L.s - 1) / 2;
    c.stride_h = c.stride_w = 1;
    c.in_dtype = c.out_dtype = d->dtype;
    c.layout = d->dtype == IS_F16 ? IS_NHWC : IS_NCHW;
    c.relu = L.relu;
    const is_status st = validate(&c);
    if (st != IS_OK) return st;
  }
  const int f = d->depth_to_space;
  if (f > 1 && d->layer[d->n_layers - 1].k != f * f) return IS_ERR_UNSUPPORTED;
  return IS_OK;
}

bool chain_fusable(const conv_chain_desc *d, const conv2d_desc *) {
  return d->dtype == IS_F32 && is::chain_fused_supported(d);
}

// fp16 chains: a last layer of fewer than 16 output channels followed by
// depth-to-space runs on the MFMA kernel as 16 channels with zero weights past
// its own (kvalid), into the workspace, when that kernel takes (C, 16).
bool pad_last_f16(const conv_chain_desc *d, const conv2d_desc &last) {
  if (d->dtype != IS_F16 || d->depth_to_space == 1 || last.k >= 16) return false;
  conv2d_desc c = last;
  c.k = 16;
  is::Plan p;
  memset(&p, 0, sizeof(p));
  p.d = c;
  return is::configure_mfma(p);
}

// fp16 chains in IS_CHAIN_AUTO whose first layer is 1 -> 64 (3x3 or 5x5) and
// second 64 -> 64 (3x3) on the MFMA kernel run those two layers as one launch:
// the first layer is computed inside the second layer's units ("Optimizing
// convolution kernels - CNNs in Vulkan Part 2/3", section "Reducing memory
// traffic": its first intermediate never goes to memory).
bool f16_head_fused(const conv_chain_desc *d, const conv2d_desc *ld) {
  if (d->dtype != IS_F16 || d->mode != IS_CHAIN_AUTO || d->n_layers < 2) return false;
  const conv_layer_desc &a = d->layer[0], &b = d->layer[1];
  if (a.c != 1 || a.k != 64 || a.r != a.s || (a.r != 3 && a.r != 5)) return false;
  if (b.c != 64 || b.k != 64 || b.r != 3 || b.s != 3) return false;
  is::Plan p;
  memset(&p, 0, sizeof(p));
  p.d = ld[1];
  return is::configure_mfma(p) && is::mfma_head_supported(p, a.r);
}

size_t chain_buffer_bytes(const conv_chain_desc *d, const conv2d_desc *ld) {
  const size_t es = d->dtype == IS_F16 ? 2 : 4;
  const int last = d->n_layers - 1;
  size_t m = 0;
  for (int l = 0; l < d->n_layers; ++l) {
    const int k = (l == last && pad_last_f16(d, ld[last])) ? 16 : d->layer[l].k;
    const size_t b = es * (size_t)d->n * k * d->h * d->w;
    if (b > m) m = b;
  }
  return align256(m);
}

// Workspace of the layer-by-layer path: ping-pong buffers for the
// intermediates; a single layer without depth-to-space writes straight to y.
size_t unfused_bytes(const conv_chain_desc *d, const conv2d_desc *ld) {
  const int need = (d->n_layers == 1 && d->depth_to_space == 1) ? 0 : (d->n_layers == 1 ? 1 : 2);
  return need * chain_buffer_bytes(d, ld);
}

// ---- Stencil pipelines: chains of single-channel layers --------------------
//
// A chain whose layers all map one channel to one (fp32, no depth-to-space) is
// an image-processing stencil pipeline. Its layers run in groups of 1 to 3
// consecutive layers, each group one launch: a single layer on the
// single-channel kernel, 2 or 3 layers on the fused kernel (warp-overlapped
// tiles, no intermediate image in HBM). IS_CHAIN_AUTO picks the grouping with
// a roofline model of each launch (the model of "Model-Based Warp Overlapped
// Tiling for Image Processing Programs on GPUs", arXiv 1909.07190, reduced to
// its trade-off: fusion saves the intermediate images' HBM traffic and a
// launch, and pays for the recomputed overlap columns and rows).
bool stencil_chain(const conv_chain_desc *d) {
  if (d->dtype != IS_F32 || d->depth_to_space != 1) return false;
  for (int l = 0; l < d->n_layers; ++l)
    if (d->layer[l].c != 1 || d->layer[l].k != 1) return false;
  return true;
}

// Rates measured on MI355X: the single-channel kernel streams 5.6 TB/s and its
// FMA loop reaches about 80% of the 78.6 TFLOP/s fp32 vector peak; the fused
// kernel's loops reach 65-71% (more live registers per wave, and with a 5x5
// or 7x7 filter among 5x5 or 3x3 ones the taps overflow the scalar registers);
// a launch with its ramp costs a few microseconds.
constexpr double kModelHbm = 5.6e12;
constexpr double kModelAlu = 0.8 * 78.6e12;
constexpr double kModelAluFused = 0.65 * 78.6e12;
constexpr double kModelLaunch = 3.0e-6;

// Estimated seconds of one launch of layers [first, first + count).
double model_group_seconds(const conv_chain_desc *d, int first, int count) {
  const double px = (double)d->n * d->h * d->w;
  if (count == 1) {
    const double r = d->layer[first].r, s = d->layer[first].s;
    return std::max(8.0 * px / kModelHbm, 2.0 * r * s * px / kModelAlu) + kModelLaunch;
  }
  const is::FusedStencilGeo g = is::fused_stencil_geometry(d, first, count);
  int ps = 0;
  for (int l = 0; l < count; ++l) ps += (d->layer[first + l].r - 1) / 2;
  // Every stage runs on the whole 256-column window and on the strip's
  // rows plus ps above and below.
  const double hf = 256.0 / g.step;
  const double vf = (g.strip_rows + 2.0 * ps) / g.strip_rows;
  double flops = 0.0;
  for (int l = 0; l < count; ++l) flops += 2.0 * d->layer[first + l].r * d->layer[first + l].s * px * hf * vf;
  const double bytes = 4.0 * px * hf * vf + 4.0 * px;
  return std::max(bytes / kModelHbm, flops / kModelAluFused) + kModelLaunch;
}

// Sizes of the launch groups of a stencil chain, in order; returns their
// number, 0 when the mode cannot be met (IS_CHAIN_FUSED with no fused kernel
// for the whole chain).
int stencil_groups(const conv_chain_desc *d, int *size) {
  const int L = d->n_layers;
  if (d->mode == IS_CHAIN_UNFUSED) {
    for (int l = 0; l < L; ++l) size[l] = 1;
    return L;
  }
  if (d->mode == IS_CHAIN_FUSED) {
    if (L == 1 || !is::fused_stencil_geometry(d, 0, L).ok) return 0;
    size[0] = L;
    return 1;
  }
  double best[IS_MAX_CHAIN + 1];
  int choice[IS_MAX_CHAIN + 1];
  best[0] = 0.0;
  for (int i = 1; i <= L; ++i) {
    best[i] = -1.0;
    choice[i] = 1;
    for (int c = 1; c <= 3 && c <= i; ++c) {
      const int first = i - c;
      if (c > 1 && !is::fused_stencil_geometry(d, first, c).ok) continue;
      const double v = best[first] + model_group_seconds(d, first, c);
      if (best[i] < 0.0 || v < best[i]) {
        best[i] = v;
        choice[i] = c;
      }
    }
  }
  int rev[IS_MAX_CHAIN], n = 0;
  for (int i = L; i > 0; i -= choice[i]) rev[n++] = choice[i];
  for (int g = 0; g < n; ++g) size[g] = rev[n - 1 - g];
  return n;
}

// Intermediate images a grouping needs in the workspace (ping-pong).
int stencil_buffers(int groups) { return groups <= 1 ? 0 : (groups == 2 ? 1 : 2); }

// Workspace that conv_chain_forward wants for the chain and mode: none for the
// fused kernel; IS_CHAIN_AUTO asks for the layer-by-layer workspace, which
// enables the faster path (on MI355X the layer-by-layer chain, with its
// 32 -> 32 layers on the fp32 MFMA kernel, beats the fused kernel, whose
// overlapped windows recompute about a quarter of the work).
is_status chain_workspace(const conv_chain_desc *d, const conv2d_desc *ld, size_t *bytes) {
  if (stencil_chain(d)) {
    int size[IS_MAX_CHAIN];
    const int groups = stencil_groups(d, size);
    if (groups == 0) return IS_ERR_UNSUPPORTED;
    *bytes = stencil_buffers(groups) * chain_buffer_bytes(d, ld);
    return IS_OK;
  }
  if (d->mode == IS_CHAIN_FUSED) {
    if (!chain_fusable(d, ld)) return IS_ERR_UNSUPPORTED;
    *bytes = 0;
    return IS_OK;
  }
  *bytes = unfused_bytes(d, ld);
  return IS_OK;
}

// Whether conv_chain_forward runs the fused kernel: always in IS_CHAIN_FUSED;
// in IS_CHAIN_AUTO when the workspace falls short of the layer-by-layer need
// and the chain has a fused kernel.
bool runs_fused(const conv_chain_desc *d, const conv2d_desc *ld, const void *workspace,
                size_t workspace_bytes) {
  if (stencil_chain(d)) return false;   // grouped launches, see stencil_groups
  if (d->mode == IS_CHAIN_FUSED) return true;
  if (d->mode == IS_CHAIN_UNFUSED || !chain_fusable(d, ld)) return false;
  const size_t need = unfused_bytes(d, ld);
  return need > 0 && (!workspace || workspace_bytes < need);
}

}  // namespace

namespace is {

int persistent_grid(int units, int cus) {
  const int g = cus < 8 ? 8 : cus / 8 * 8;
  const long long need = ((long long)(units < 1 ? 1 : units) + 7) / 8 * 8;   // every group busy
  return need < g ? (int)need : g;
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = __atomic_load_n(&g_device_cus[dev], __ATOMIC_RELAXED);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  __atomic_store_n(&g_device_cus[dev], cus, __ATOMIC_RELAXED);
  return cus;
}

is_status report_hip(hipError_t e) { return hip_status(e); }

is_status chain_forward(const conv_chain_desc *d, const void *x, const void *const *w,
                        const float *const *b, void *y, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  try {
    conv2d_desc ld[IS_MAX_CHAIN];
    is_status st = chain_layers(d, ld);
    if (st != IS_OK) return st;
    if (!x || !w || !y) return IS_ERR_INVALID_ARG;
    for (int l = 0; l < d->n_layers; ++l) {
      if (!w[l]) return IS_ERR_INVALID_ARG;
      if (misaligned(w[l]) || (b && b[l] && misaligned(b[l]))) return IS_ERR_MISALIGNED;
    }
    if (misaligned(x) || misaligned(y)) return IS_ERR_MISALIGNED;
    const size_t es = d->dtype == IS_F16 ? 2 : 4;
    const size_t xb = es * (size_t)d->n * d->layer[0].c * d->h * d->w;
    const size_t yb = es * (size_t)d->n * d->layer[d->n_layers - 1].k * d->h * d->w;
    if (overlap(x, xb, y, yb)) return IS_ERR_INVALID_ARG;
    size_t need = 0;
    st = chain_workspace(d, ld, &need);
    if (st != IS_OK) return st;
    const bool stencil = stencil_chain(d);
    int gsize[IS_MAX_CHAIN];
    int groups = stencil ? stencil_groups(d, gsize) : 0;
    // IS_CHAIN_AUTO without the workspace: one fused launch when it covers
    // the whole stencil chain.
    if (stencil && need > 0 && (!workspace || workspace_bytes < need) && d->mode == IS_CHAIN_AUTO &&
        is::fused_stencil_geometry(d, 0, d->n_layers).ok) {
      groups = 1;
      gsize[0] = d->n_layers;
      need = 0;
    }
    const bool fused = runs_fused(d, ld, workspace, workspace_bytes);
    if (fused) need = 0;
    if (need > 0 && (!workspace || workspace_bytes < need)) return IS_ERR_WORKSPACE;
    if (need > 0 && misaligned(workspace)) return IS_ERR_MISALIGNED;
    if (need > 0 && (overlap(workspace, need, x, xb) || overlap(workspace, need, y, yb)))
      return IS_ERR_INVALID_ARG;
    if (xb == 0 || yb == 0) return IS_OK;

    if (fused)
      return hip_status(is::launch_chain_fused(d, static_cast<const float *>(x),
                                               reinterpret_cast<const float *const *>(w), b,
                                               static_cast<float *>(y), stream));

    const size_t half = chain_buffer_bytes(d, ld);
    char *ws = static_cast<char *>(workspace);
    if (stencil) {
      const float *gsrc = static_cast<const float *>(x);
      const float *const *wf = reinterpret_cast<const float *const *>(w);
      for (int g = 0, first = 0; g < groups; first += gsize[g], ++g) {
        float *dst = g == groups - 1 ? static_cast<float *>(y) : reinterpret_cast<float *>(ws + (g % 2) * half);
        if (gsize[g] == 1) {
          is::Plan p;
          st = make_plan(&ld[first], p);
          if (st == IS_OK) st = run_plan(p, gsrc, w[first], b ? b[first] : nullptr, dst, stream);
        } else {
          st = hip_status(is::launch_fused_stencil(d, first, gsize[g], gsrc, wf, b, dst, stream));
        }
        if (st != IS_OK) return st;
        gsrc = dst;
      }
      return IS_OK;
    }
    const void *src = x;
    int l0 = 0;
    if (f16_head_fused(d, ld)) {   // layers 0 and 1 in one launch, into layer 1's buffer
      is::Plan p;
      st = make_plan(&ld[1], p);
      if (st != IS_OK) return st;
      void *dst = (d->n_layers == 2 && d->depth_to_space == 1) ? y : (void *)(ws + half);
      st = hip_status(is::launch_mfma_head(
          p, static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(w[0]), b ? b[0] : nullptr,
          d->layer[0].relu, d->layer[0].r, static_cast<const _Float16 *>(w[1]), b ? b[1] : nullptr,
          static_cast<_Float16 *>(dst), stream));
      if (st != IS_OK) return st;
      src = dst;
      l0 = 2;
    }
    for (int l = l0; l < d->n_layers; ++l) {
      const bool last = l == d->n_layers - 1;
      void *dst = (last && d->depth_to_space == 1) ? y : (void *)(ws + (l % 2) * half);
      is::Plan p;
      const bool padded = last && pad_last_f16(d, ld[l]);
      if (padded) {
        conv2d_desc c = ld[l];
        c.k = 16;
        st = make_plan(&c, p);
        p.kvalid = ld[l].k;
      } else {
        st = make_plan(&ld[l], p);
      }
      if (st != IS_OK) return st;
      // The last layer writes the depth-to-space output itself when its kernel can.
      if (last && padded && d->depth_to_space == 3 && is::mfma_d2s3_supported(p))
        return hip_status(is::launch_mfma_d2s3(p, static_cast<const _Float16 *>(src),
                                               static_cast<const _Float16 *>(w[l]), b ? b[l] : nullptr,
                                               static_cast<_Float16 *>(y), stream));
      if (last && d->depth_to_space == 2 && is::multi_d2s_supported(p))
        return hip_status(is::launch_multi_d2s(p, static_cast<const float *>(src),
                                               static_cast<const float *>(w[l]), b ? b[l] : nullptr,
                                               static_cast<float *>(y), stream));
      st = run_plan(p, src, w[l], b ? b[l] : nullptr, dst, stream);
      if (st != IS_OK) return st;
      src = dst;
    }
    const int f = d->depth_to_space;
    if (f > 1 && d->dtype == IS_F16) {
      const int k = d->layer[d->n_layers - 1].k;
      const int zc = pad_last_f16(d, ld[d->n_layers - 1]) ? 16 : k;
      return hip_status(is::launch_depth_to_space_f16(static_cast<const _Float16 *>(src),
                                                      static_cast<_Float16 *>(y), d->n, d->h, d->w, f, zc,
                                                      stream));
    }
    if (f > 1)
      return hip_status(is::launch_depth_to_space(static_cast<const float *>(src), static_cast<float *>(y),
                                                  d->n, d->h, d->w, f, stream));
    return IS_OK;
  } catch (...) {
    return IS_ERR_INVALID_ARG;
  }
}


}  // namespace is

extern "C" {

int is_persistent_grid(int units, int cus) {
  if (units < 1 || cus < 1) return 0;
  return is::persistent_grid(units, cus);
}

is_status conv_chain_workspace_size(const conv_chain_desc *d, size_t *bytes) {
  if (!bytes) return IS_ERR_INVALID_ARG;
  conv2d_desc ld[IS_MAX_CHAIN];
  const is_status st = chain_layers(d, ld);
  if (st != IS_OK) return st;
  return chain_workspace(d, ld, bytes);
}

is_status conv_chain_kernel_name(const conv_chain_desc *d, char *name, size_t len) {
  if (!name || len == 0) return IS_ERR_INVALID_ARG;
  conv2d_desc ld[IS_MAX_CHAIN];
  const is_status st = chain_layers(d, ld);
  if (st != IS_OK) return st;
  size_t ws = 0;
  const is_status st2 = chain_workspace(d, ld, &ws);
  if (st2 != IS_OK) return st2;
  // the path taken when the caller passes the workspace reported above
  if (stencil_chain(d)) {
    int size[IS_MAX_CHAIN];
    const int groups = stencil_groups(d, size);
    bool all_single = true;
    for (int g = 0; g < groups; ++g) all_single = all_single && size[g] == 1;
    if (all_single) {
      snprintf(name, len, "%s", "layer_by_layer");
    } else if (groups == 1) {
      snprintf(name, len, "%s", "is_k7_fused_stencil");
    } else {
      char buf[64] = "fused_groups:";
      for (int g = 0; g < groups; ++g) {
        char part[8];
        snprintf(part, sizeof(part), g ? "+%d" : "%d", size[g]);
        strncat(buf, part, sizeof(buf) - strlen(buf) - 1);
      }
      snprintf(name, len, "%s", buf);
    }
    return IS_OK;
  }
  const bool fused = d->mode == IS_CHAIN_FUSED;
  snprintf(name, len, "%s", fused ? "is_k3_chain" : (f16_head_fused(d, ld) ? "head_fused" : "layer_by_layer"));
  return IS_OK;
}

is_status conv_chain_groups(const conv_chain_desc *d, int *sizes, int max, int *count) {
  if (!count || max < 0 || (max > 0 && !sizes)) return IS_ERR_INVALID_ARG;
  conv2d_desc ld[IS_MAX_CHAIN];
  const is_status st = chain_layers(d, ld);
  if (st != IS_OK) return st;
  size_t ws = 0;
  const is_status st2 = chain_workspace(d, ld, &ws);
  if (st2 != IS_OK) return st2;
  int size[IS_MAX_CHAIN];
  int groups;
  if (stencil_chain(d)) {
    groups = stencil_groups(d, size);
  } else if (d->mode == IS_CHAIN_FUSED) {
    groups = 1;
    size[0] = d->n_layers;
  } else if (f16_head_fused(d, ld)) {
    groups = d->n_layers - 1;
    size[0] = 2;
    for (int l = 1; l < groups; ++l) size[l] = 1;
  } else {
    groups = d->n_layers;
    for (int l = 0; l < groups; ++l) size[l] = 1;
  }
  *count = groups;
  for (int g = 0; g < groups && g < max; ++g) sizes[g] = size[g];
  return IS_OK;
}

is_status conv_chain_forward(const conv_chain_desc *d, const void *x, const void *const *w,
                             const float *const *b, void *y, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  return is::chain_forward(d, x, w, b, y, workspace, workspace_bytes, stream);
}

is_status conv2d_create(const conv2d_desc *d, conv2d_plan *out) {
  if (!out) return IS_ERR_INVALID_ARG;
  *out = nullptr;
  try {
    is::Plan p;
    const is_status st = make_plan(d, p);
    if (st != IS_OK) return st;
    conv2d_plan_s *h = new (std::nothrow) conv2d_plan_s;
    if (!h) return IS_ERR_NO_MEMORY;
    h->p = p;
    *out = h;
    return IS_OK;
  } catch (...) {
    return IS_ERR_NO_MEMORY;
  }
}

is_status conv2d_forward(conv2d_plan plan, const void *x, const void *w, const float *bias, void *y,
                         hipStream_t stream) {
  if (!plan) return IS_ERR_INVALID_ARG;
  try {
    return run_plan(plan->p, x, w, bias, y, stream);
  } catch (...) {
    return IS_ERR_INVALID_ARG;
  }
}

void conv2d_destroy(conv2d_plan plan) { delete plan; }

is_status conv2d_list_variants(const conv2d_desc *d, conv2d_variant *out, int max, int *count) {
  if (!count || max < 0 || (max > 0 && !out)) return IS_ERR_INVALID_ARG;
  try {
    is::Plan def;
    const is_status st = make_plan(d, def);
    if (st != IS_OK) return st;
    Variant v[kMaxVariants];
    const int n = collect_variants(*d, def, v, kMaxVariants);
    *count = n;
    for (int i = 0; i < n && i < max; ++i) {
      is::Plan p;
      variant_plan(p, *d, def, v, i);
      fill_variant(p, i == 0, 0.f, &out[i]);
    }
    return IS_OK;
  } catch (...) {
    return IS_ERR_NO_MEMORY;
  }
}

is_status conv2d_create_variant(const conv2d_desc *d, int index, conv2d_plan *out) {
  if (!out) return IS_ERR_INVALID_ARG;
  *out = nullptr;
  try {
    is::Plan def;
    const is_status st = make_plan(d, def);
    if (st != IS_OK) return st;
    Variant v[kMaxVariants];
    const int n = collect_variants(*d, def, v, kMaxVariants);
    if (index < 0 || index >= n) return IS_ERR_INVALID_ARG;
    conv2d_plan_s *h = new (std::nothrow) conv2d_plan_s;
    if (!h) return IS_ERR_NO_MEMORY;
    variant_plan(h->p, *d, def, v, index);
    *out = h;
    return IS_OK;
  } catch (...) {
    return IS_ERR_NO_MEMORY;
  }
}

is_status conv2d_autotune(conv2d_plan plan, const void *x, const void *w, const float *bias, void *y,
                          hipStream_t stream, int reps, conv2d_variant *out, int max, int *count) {
  if (!plan || reps < 1 || max < 0 || (max > 0 && !out)) return IS_ERR_INVALID_ARG;
  try {
    const conv2d_desc d = plan->p.d;
    is::Plan def;
    is_status st = make_plan(&d, def);
    if (st != IS_OK) return st;
    st = check_forward_args(d, x, w, bias, y);   // before any HIP call
    if (st != IS_OK) return st;
    Variant v[kMaxVariants];
    const int n = collect_variants(d, def, v, kMaxVariants);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
      if (e0) (void)hipEventDestroy(e0);
      return hip_status(hipErrorOutOfMemory);
    }
    int best = -1;
    float best_ms = 0.f;
    is::Plan best_plan;
    for (int i = 0; i < n && st == IS_OK; ++i) {
      is::Plan p;
      variant_plan(p, d, def, v, i);
      st = run_plan(p, x, w, bias, y, stream);   // warm-up; also checks the arguments
      if (st != IS_OK) break;
      hipError_t e = hipEventRecord(e0, stream);
      for (int r = 0; r < reps && st == IS_OK; ++r) st = run_plan(p, x, w, bias, y, stream);
      if (st != IS_OK) break;
      if (e == hipSuccess) e = hipEventRecord(e1, stream);
      if (e == hipSuccess) e = hipEventSynchronize(e1);
      float ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
      if (e != hipSuccess) {
        st = hip_status(e);
        break;
      }
      ms /= (float)reps;
      if (i < max) fill_variant(p, i == 0, ms, &out[i]);
      if (best < 0 || ms < best_ms) {
        best = i;
        best_ms = ms;
        best_plan = p;
      }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st != IS_OK) return st;
    if (count) *count = n;
    plan->p = best_plan;
    // y ends up holding the chosen variant's result.
    return run_plan(plan->p, x, w, bias, y, stream);
  } catch (...) {
    return IS_ERR_NO_MEMORY;
  }
}

is_status conv2d_get_plan_info(conv2d_plan plan, conv2d_plan_info *info) {
  if (!plan || !info) return IS_ERR_INVALID_ARG;
  fill_info(plan->p, info);
  return IS_OK;
}

size_t is_lds_tile_bytes(int tile_w, int tile_h, int r, int s, int channels, int elem_bytes) {
  if (tile_w <= 0 || tile_h <= 0 || r <= 0 || s <= 0 || channels <= 0 || elem_bytes <= 0) return 0;
  return (size_t)(tile_w + s - 1) * (size_t)(tile_h + r - 1) * (size_t)channels * (size_t)elem_bytes;
}

int is_swizzle_col(int y, int x, int nx, int elem_bytes, int chunk_bytes) {
  auto pow2 = [](int v) { return v > 0 && (v & (v - 1)) == 0; };
  if (y < 0 || x < 0 || x >= nx || !pow2(nx) || !pow2(elem_bytes) || !pow2(chunk_bytes)) return -1;
  if (chunk_bytes < elem_bytes || chunk_bytes > nx * elem_bytes || nx * elem_bytes < 32) return -1;
  return is::swizzle_col(y, x, nx, elem_bytes, chunk_bytes);
}

const char *is_status_str(is_status st) {
  switch (st) {
    case IS_OK: return "ok";
    case IS_ERR_INVALID_ARG: return "invalid argument";
    case IS_ERR_UNSUPPORTED: return "unsupported";
    case IS_ERR_MISALIGNED: return "tensor base not 16-byte aligned";
    case IS_ERR_HIP: return "HIP runtime error";
    case IS_ERR_NO_MEMORY: return "out of host memory";
    case IS_ERR_WORKSPACE: return "workspace missing or too small";
  }
  return "unknown status";
}

int is_last_hip_error(void) { return g_last_hip_error; }

int is_version(void) { return IS_VERSION; }

}  // extern "C"
