"""Python binding of libimgstencil: direct 2D convolution with small filters on gfx950.

The functions with the C names (conv2d_create, conv2d_forward, conv2d_destroy,
conv2d_get_plan_info, conv2d_list_variants, conv2d_create_variant,
conv2d_autotune, conv_chain_workspace_size, conv_chain_forward, conv_chain_forward_noalloc,
conv_chain_kernel_name, conv_chain_groups, is_lds_tile_bytes, is_swizzle_col,
is_persistent_grid) marshal arguments to
the C ABI of include/imgstencil.h and nothing else. conv2d() and conv_chain()
are conveniences on torch tensors: torch only allocates device memory and
supplies the current HIP stream.
"""
import ctypes

from . import _abi
from ._abi import (IS_F16, IS_F32, IS_NCHW, IS_NHWC, IS_CHAIN_AUTO, IS_CHAIN_FUSED, IS_CHAIN_UNFUSED,
                   ImgStencilError, conv2d_desc, conv_chain_desc, conv2d_plan_info, conv2d_variant)

__all__ = ["conv2d_create", "conv2d_forward", "conv2d_destroy", "conv2d_get_plan_info",
           "conv2d_list_variants", "conv2d_create_variant", "conv2d_autotune",
           "conv_chain_workspace_size", "conv_chain_forward", "conv_chain_forward_noalloc",
           "conv_chain_kernel_name", "conv_chain_groups",
           "is_lds_tile_bytes", "is_swizzle_col", "is_persistent_grid", "is_version", "make_desc", "make_chain_desc",
           "conv2d", "conv2d_separable", "conv_chain", "Plan", "ImgStencilError"]


def load():
    return _abi.load()


def make_desc(n, c, h, w, k, r, s, dtype="f32", relu=False, separable=False):
    """conv2d_desc for a same-padded stride-1 layer; f32 is NCHW, f16 is NHWC.
    separable: the filter is given as R column taps then S row taps."""
    d = conv2d_desc()
    d.n, d.c, d.h, d.w, d.k, d.r, d.s = n, c, h, w, k, r, s
    d.pad_h, d.pad_w = (r - 1) // 2, (s - 1) // 2
    d.stride_h = d.stride_w = 1
    if dtype == "f32":
        d.in_dtype = d.out_dtype = IS_F32
        d.layout = IS_NCHW
    elif dtype == "f16":
        d.in_dtype = d.out_dtype = IS_F16
        d.layout = IS_NHWC
    else:
        raise ValueError("dtype must be 'f32' (NCHW) or 'f16' (NHWC)")
    d.relu = int(bool(relu))
    d.separable = int(bool(separable))
    return d


def conv2d_create(desc):
    """Returns an opaque plan handle (int); raises ImgStencilError on a bad desc."""
    plan = ctypes.c_void_p()
    _abi.check(load().conv2d_create(ctypes.byref(desc), ctypes.byref(plan)), "conv2d_create")
    return plan.value


def conv2d_forward(plan, x_ptr, w_ptr, bias_ptr, y_ptr, stream):
    """Raw pointers (ints, bias may be 0/None) and a hipStream_t (int)."""
    _abi.check(load().conv2d_forward(plan, x_ptr, w_ptr, bias_ptr or None, y_ptr, stream or None),
               "conv2d_forward")


def conv2d_destroy(plan):
    load().conv2d_destroy(plan)


def _variants(arr, n):
    return [{"kernel": arr[i].kernel.decode(), "param": arr[i].param, "is_default": bool(arr[i].is_default),
             "ms": arr[i].ms} for i in range(n)]


def conv2d_list_variants(desc):
    """Every kernel configuration that can run desc, the default first (dicts)."""
    n = ctypes.c_int()
    arr = (conv2d_variant * 32)()
    _abi.check(load().conv2d_list_variants(ctypes.byref(desc), arr, 32, ctypes.byref(n)), "conv2d_list_variants")
    return _variants(arr, min(n.value, 32))


def conv2d_create_variant(desc, index):
    plan = ctypes.c_void_p()
    _abi.check(load().conv2d_create_variant(ctypes.byref(desc), index, ctypes.byref(plan)),
               "conv2d_create_variant")
    return plan.value


def conv2d_autotune(plan, x_ptr, w_ptr, bias_ptr, y_ptr, stream, reps=10):
    """Time every variant on these buffers, keep the fastest in the plan, and
    return the measured variants (dicts with ms)."""
    n = ctypes.c_int()
    arr = (conv2d_variant * 32)()
    _abi.check(load().conv2d_autotune(plan, x_ptr, w_ptr, bias_ptr or None, y_ptr, stream or None, reps, arr, 32,
                                      ctypes.byref(n)), "conv2d_autotune")
    return _variants(arr, min(n.value, 32))


def conv2d_get_plan_info(plan):
    info = conv2d_plan_info()
    _abi.check(load().conv2d_get_plan_info(plan, ctypes.byref(info)), "conv2d_get_plan_info")
    return {"kernel": info.kernel.decode(), "grid": (info.grid_x, info.grid_y, info.grid_z),
            "block": info.block, "lds_bytes": info.lds_bytes, "tile": (info.tile_w, info.tile_h),
            "flops": info.flops, "bytes": info.bytes}


def make_chain_desc(n, h, w, layers, depth_to_space=1, mode=IS_CHAIN_AUTO, dtype="f32"):
    """layers: sequence of (c, k, r, relu) (square filters); dtype "f32" (NCHW)
    or "f16" (NHWC, fp16 storage between layers)."""
    d = conv_chain_desc()
    d.n, d.h, d.w = n, h, w
    if not 1 <= len(layers) <= _abi.IS_MAX_CHAIN:
        raise ValueError("1 to %d layers" % _abi.IS_MAX_CHAIN)
    d.n_layers = len(layers)
    for i, (c, k, r, relu) in enumerate(layers):
        L = d.layer[i]
        L.c, L.k, L.r, L.s, L.relu = c, k, r, r, int(bool(relu))
    d.depth_to_space = depth_to_space
    d.dtype = {"f32": IS_F32, "f16": IS_F16}[dtype]
    d.mode = mode
    return d


def conv_chain_workspace_size(desc):
    n = ctypes.c_size_t()
    _abi.check(load().conv_chain_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
               "conv_chain_workspace_size")
    return n.value


def conv_chain_kernel_name(desc):
    buf = ctypes.create_string_buffer(64)
    _abi.check(load().conv_chain_kernel_name(ctypes.byref(desc), buf, 64), "conv_chain_kernel_name")
    return buf.value.decode()


def conv_chain_groups(desc):
    """Launch groups of the chain, as sizes in layers."""
    n = ctypes.c_int()
    arr = (ctypes.c_int * _abi.IS_MAX_CHAIN)()
    _abi.check(load().conv_chain_groups(ctypes.byref(desc), arr, _abi.IS_MAX_CHAIN, ctypes.byref(n)),
               "conv_chain_groups")
    return [arr[i] for i in range(n.value)]


def conv_chain_forward(desc, x_ptr, w_ptrs, b_ptrs, y_ptr, ws_ptr, ws_bytes, stream):
    n = desc.n_layers
    W = (ctypes.c_void_p * n)(*w_ptrs)
    B = (ctypes.c_void_p * n)(*[p or None for p in b_ptrs]) if b_ptrs is not None else None
    _abi.check(load().conv_chain_forward(ctypes.byref(desc), x_ptr, W, B, y_ptr, ws_ptr or None,
                                         ws_bytes, stream or None), "conv_chain_forward")


def conv_chain_forward_noalloc(desc, x_ptr, w_ptrs, b_ptrs, y_ptr, stream):
    """conv_chain_forward with the library's own workspace (no allocation)."""
    n = desc.n_layers
    W = (ctypes.c_void_p * n)(*w_ptrs)
    B = (ctypes.c_void_p * n)(*[p or None for p in b_ptrs]) if b_ptrs is not None else None
    _abi.check(load().conv_chain_forward_noalloc(ctypes.byref(desc), x_ptr, W, B, y_ptr, stream or None),
               "conv_chain_forward_noalloc")


def is_lds_tile_bytes(tile_w, tile_h, r, s, channels, elem_bytes):
    return load().is_lds_tile_bytes(tile_w, tile_h, r, s, channels, elem_bytes)


def is_swizzle_col(y, x, nx, elem_bytes, chunk_bytes):
    return load().is_swizzle_col(y, x, nx, elem_bytes, chunk_bytes)


def is_persistent_grid(units, cus):
    return load().is_persistent_grid(units, cus)


def is_version():
    return load().is_version()


# ---------------------------------------------------------------- torch helpers
class Plan:
    """Owns a conv2d plan; forward() launches on torch's current stream.
    variant: index into conv2d_list_variants(desc) (None: the default)."""

    def __init__(self, desc, variant=None):
        self.desc = desc
        self.handle = conv2d_create(desc) if variant is None else conv2d_create_variant(desc, variant)
        # Bound now: at interpreter exit the module's globals may already be
        # gone when __del__ runs.
        self._destroy = load().conv2d_destroy

    def info(self):
        return conv2d_get_plan_info(self.handle)

    def forward(self, x, w, b, y, stream=None):
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        conv2d_forward(self.handle, x.data_ptr(), w.data_ptr(), b.data_ptr() if b is not None else None,
                       y.data_ptr(), stream)
        return y

    def autotune(self, x, w, b, y, reps=10, stream=None):
        """Time every variant on these tensors and keep the fastest (y is
        overwritten with its result); returns the measured variants."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        return conv2d_autotune(self.handle, x.data_ptr(), w.data_ptr(), b.data_ptr() if b is not None else None,
                               y.data_ptr(), stream, reps)

    def __del__(self):
        h = getattr(self, "handle", None)
        destroy = getattr(self, "_destroy", None)
        if h and destroy is not None:
            destroy(h)
            self.handle = None


def _check_dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s" % (name, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


# The shape and dtype checks come before the device checks, so that every
# rejected argument is reported the same way with or without a GPU.
def _check_float_input(x):
    import torch
    if not isinstance(x, torch.Tensor) or x.dtype not in (torch.float32, torch.float16):
        raise TypeError("x must be a float32 (NCHW) or float16 (NHWC) tensor")
    if x.dim() != 4:
        raise ValueError("x must have 4 dimensions, got shape %s" % (tuple(x.shape),))


def _check_weights(w, dtype, cin, name):
    import torch
    if not isinstance(w, torch.Tensor) or w.dtype != dtype:
        raise TypeError("%s must be a %s tensor" % (name, dtype))
    if w.dim() != 4:
        raise ValueError("%s must be K,C,R,S, got shape %s" % (name, tuple(w.shape)))
    if w.shape[1] != cin:
        raise ValueError("%s expects %d input channels, the layer receives %d" % (name, w.shape[1], cin))


def _check_bias(b, K, name="b"):
    """b: None or K fp32 values."""
    import torch
    if b is None:
        return
    if not isinstance(b, torch.Tensor) or b.dtype != torch.float32:
        raise TypeError("%s must be a float32 tensor" % name)
    if b.numel() != K:
        raise ValueError("%s must hold one value per output channel (%d), got %d" % (name, K, b.numel()))


def conv2d(x, w, b=None, relu=False):
    """y = act(conv(x, w) + b). fp32: x is N,C,H,W. fp16: x is N,H,W,C. w is K,C,R,S."""
    import torch
    _check_float_input(x)
    f16 = x.dtype == torch.float16
    if f16:
        N, H, W, C = x.shape
    else:
        N, C, H, W = x.shape
    _check_weights(w, x.dtype, C, "w")
    K, _, R, S = w.shape
    _check_bias(b, K)
    _check_dev(x, x.dtype, "x")
    _check_dev(w, x.dtype, "w")
    if b is not None:
        _check_dev(b, torch.float32, "b")
    if f16:
        y = torch.empty((N, H, W, K), dtype=x.dtype, device=x.device)
    else:
        y = torch.empty((N, K, H, W), dtype=x.dtype, device=x.device)
    p = Plan(make_desc(N, C, H, W, K, R, S, "f16" if f16 else "f32", relu))
    return p.forward(x, w, b, y)


def conv2d_separable(x, col, row, b=None, relu=False):
    """Single-channel fp32 filtering with the separable filter w[i][j] =
    col[i] * row[j]: x N,1,H,W; col R taps, row S taps (device tensors)."""
    import torch
    _check_float_input(x)
    if x.dtype != torch.float32 or x.shape[1] != 1:
        raise ValueError("separable filtering takes one fp32 channel, x is %s %s" % (x.dtype, tuple(x.shape)))
    _check_bias(b, 1)
    _check_dev(x, torch.float32, "x")
    _check_dev(col, torch.float32, "col")
    _check_dev(row, torch.float32, "row")
    if b is not None:
        _check_dev(b, torch.float32, "b")
    N, C, H, W = x.shape
    R, S = col.numel(), row.numel()
    w = torch.cat([col.reshape(-1), row.reshape(-1)])
    y = torch.empty((N, 1, H, W), dtype=x.dtype, device=x.device)
    p = Plan(make_desc(N, C, H, W, 1, R, S, "f32", relu, separable=True))
    return p.forward(x, w, b, y)


def conv_chain(x, layers, depth_to_space=1, mode=IS_CHAIN_AUTO):
    """layers: list of (w, b, relu) device tensors. x fp32 NCHW with fp32 weights,
    or x fp16 NHWC with fp16 weights (fp32 biases). Returns the chain output."""
    import torch
    _check_float_input(x)
    f16 = x.dtype == torch.float16
    if f16:
        N, H, W, C = x.shape
    else:
        N, C, H, W = x.shape
    if not 1 <= len(layers) <= _abi.IS_MAX_CHAIN:
        raise ValueError("1 to %d layers" % _abi.IS_MAX_CHAIN)
    spec = []
    for i, (w, b, relu) in enumerate(layers):
        _check_weights(w, x.dtype, C if i == 0 else spec[-1][1], "w[%d]" % i)
        if w.shape[2] != w.shape[3]:
            raise ValueError("w[%d]: chain layers take square filters, got %dx%d" % (i, w.shape[2], w.shape[3]))
        _check_bias(b, w.shape[0], "b[%d]" % i)
        spec.append((w.shape[1], w.shape[0], w.shape[2], relu))
    _check_dev(x, x.dtype, "x")
    for i, (w, b, _) in enumerate(layers):
        _check_dev(w, x.dtype, "w[%d]" % i)
        if b is not None:
            _check_dev(b, torch.float32, "b[%d]" % i)
    d = make_chain_desc(N, H, W, spec, depth_to_space, mode, "f16" if f16 else "f32")
    f = depth_to_space
    if f16:
        shape = (N, f * H, f * W, 1) if f > 1 else (N, H, W, spec[-1][1])
    else:
        shape = (N, 1, f * H, f * W) if f > 1 else (N, spec[-1][1], H, W)
    y = torch.empty(shape, dtype=x.dtype, device=x.device)
    ws_bytes = conv_chain_workspace_size(d)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device) if ws_bytes else None
    conv_chain_forward(d, x.data_ptr(), [w.data_ptr() for (w, _, _) in layers],
                       [b.data_ptr() if b is not None else None for (_, b, _) in layers],
                       y.data_ptr(), ws.data_ptr() if ws is not None else None, ws_bytes,
                       torch.cuda.current_stream().cuda_stream)
    return y
