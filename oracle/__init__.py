"""CPU oracle for direct 2D convolution with small filters (test infrastructure).

ONLY the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The HIP library never calls it and shares no code with it.

Every function returns float64 results computed by the plain definition in
oracle.c (see its header): same-size zero-padded cross-correlation with a centred
window, bias added after the sum, optional ReLU -- the per-pixel loop nest of
"Optimizing convolution kernels - CNNs in Vulkan Part 2/3", section "Where we
left off". Each result comes with its error scale m = sum |w*x| + |b|.

The conv chain is the composition of single layers followed by depth-to-space
(chain of the upscaling network described in the same page's introduction and
its "Reducing memory traffic" table), with the error scale propagated layer by
layer as m_l = conv(|w_l|, m_{l-1}) + |b_l|.

The fp16-storage chain (the same page's "Reducing memory traffic" step, which
stores the data and the weights as fp16) reads every layer's input as the
previous layer's output rounded to fp16, nearest even (numpy's float64 ->
float16 conversion), computes each layer exactly in float64 on those values and
rounds its output the same way; the network input and the weights are fp16
values, the biases are given as fp32.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_LAYOUT = {"NCHW": 0, "NHWC": 1}


def load_library(path):
    """Open an oracle shared library at `path` and declare its signatures."""
    lib = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    lib.oracle_conv2d.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64, i64,
                                  _f64p, _f64p, _f64p, ctypes.c_int, _f64p, _f64p]
    lib.oracle_conv2d.restype = ctypes.c_int
    lib.oracle_conv2d_points.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64, i64,
                                         _f64p, _f64p, _f64p, ctypes.c_int, i64, _i64p,
                                         _f64p, _f64p]
    lib.oracle_conv2d_points.restype = ctypes.c_int
    lib.oracle_depth_to_space.argtypes = [i64, i64, i64, i64, _f64p, _f64p]
    lib.oracle_depth_to_space.restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = load_library(_LIB_PATH)
    return _lib


def threads():
    """Host threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def _f64(a):
    """Exact widening to a contiguous float64 array (fp16/fp32 -> fp64 is exact)."""
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_f64p)


def _dims(x, w, layout):
    if layout == "NCHW":
        N, C, H, W = x.shape
    elif layout == "NHWC":
        N, H, W, C = x.shape
    else:
        raise ValueError("layout must be NCHW or NHWC")
    K, Cw, R, S = w.shape
    if Cw != C:
        raise ValueError("weight channels %d != input channels %d" % (Cw, C))
    return N, C, H, W, K, R, S


def conv2d(x, w, b=None, relu=False, layout="NCHW", lib=None, scale=True):
    """Full output y and error scale m, both float64, in the input's layout.

    x: N,C,H,W (NCHW) or N,H,W,C (NHWC); w: K,C,R,S (odd R, S); b: K or None.
    lib: another build of oracle.c opened with load_library (default: this one).
    scale=False skips the error scale (m is returned as None); y is the same.
    """
    x, w = _f64(x), _f64(w)
    b = None if b is None else _f64(b)
    N, C, H, W, K, R, S = _dims(x, w, layout)
    if b is not None and b.shape != (K,):
        raise ValueError("bias must have shape (K,)")
    shape = (N, K, H, W) if layout == "NCHW" else (N, H, W, K)
    y = np.empty(shape, np.float64)
    m = np.empty(shape, np.float64) if scale else None
    rc = (lib or _load()).oracle_conv2d(_LAYOUT[layout], N, C, H, W, K, R, S, _ptr(x),
                                        _ptr(w), _ptr(b), int(bool(relu)), _ptr(y), _ptr(m))
    if rc != 0:
        raise ValueError("oracle_conv2d rejected the shapes")
    return y, m


def conv2d_separable(x, col, row, b=None, relu=False):
    """Single-channel filtering with a separable filter: by definition the
    filter is the outer product w[i][j] = col[i] * row[j] (R column taps, S row
    taps), applied as any other filter. x: N,1,H,W; returns (y, m) float64."""
    col, row = _f64(col).reshape(-1), _f64(row).reshape(-1)
    w = (col[:, None] * row[None, :])[None, None]
    return conv2d(x, w, b, relu)


def conv2d_points(x, w, b, relu, pts, layout="NCHW"):
    """y and m at selected outputs; pts is an (npts, 4) int array of (n, k, i, j)."""
    x, w = _f64(x), _f64(w)
    b = None if b is None else _f64(b)
    N, C, H, W, K, R, S = _dims(x, w, layout)
    pts = np.ascontiguousarray(pts, dtype=np.int64).reshape(-1, 4)
    y = np.empty(len(pts), np.float64)
    m = np.empty(len(pts), np.float64)
    rc = _load().oracle_conv2d_points(_LAYOUT[layout], N, C, H, W, K, R, S, _ptr(x),
                                      _ptr(w), _ptr(b), int(bool(relu)), len(pts),
                                      pts.ctypes.data_as(_i64p), _ptr(y), _ptr(m))
    if rc != 0:
        raise ValueError("oracle_conv2d_points rejected the shapes or points")
    return y, m


def depth_to_space(z, f):
    """(N, f*f, H, W) -> (N, 1, f*H, f*W), out[n,0,f*i+dy,f*j+dx] = z[n,f*dy+dx,i,j]."""
    z = _f64(z)
    N, C, H, W = z.shape
    if C != f * f:
        raise ValueError("depth_to_space needs f*f channels")
    out = np.empty((N, 1, H * f, W * f), np.float64)
    rc = _load().oracle_depth_to_space(N, H, W, f, _ptr(z), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_depth_to_space rejected the shapes")
    return out


def chain(x, layers, d2s=1):
    """Layer-by-layer chain on NCHW input, then depth-to-space by d2s (1 = none).

    layers: sequence of (w, b, relu). Returns (out, m) in float64.
    """
    z = _f64(x)
    m = np.abs(z)
    for w, b, relu in layers:
        w = _f64(w)
        b = None if b is None else _f64(b)
        z, _ = conv2d(z, w, b, relu, scale=False)
        m, _ = conv2d(m, np.abs(w), None if b is None else np.abs(b), False, scale=False)
    if d2s > 1:
        z = depth_to_space(z, d2s)
        m = depth_to_space(m, d2s)
    return z, m


def _zero_crop(a, r0, r1, c0, c1):
    """Rows [r0,r1) and cols [c0,c1) of an N,C,H,W array; zero where outside."""
    N, C, H, W = a.shape
    out = np.zeros((N, C, r1 - r0, c1 - c0), a.dtype)
    sr0, sr1 = max(r0, 0), min(r1, H)
    sc0, sc1 = max(c0, 0), min(c1, W)
    if sr0 < sr1 and sc0 < sc1:
        out[:, :, sr0 - r0:sr1 - r0, sc0 - c0:sc1 - c0] = a[:, :, sr0:sr1, sc0:sc1]
    return out


def chain_window(x, layers, i0, i1, j0, j1):
    """Chain output (before depth-to-space) on rows [i0,i1) x cols [j0,j1) only.

    Same result as chain(x, layers)[..., i0:i1, j0:j1]: each layer is evaluated on
    its input window grown by its radius, and every intermediate value that falls
    outside the image is set to zero, as the next layer's zero padding demands.
    """
    x = _f64(x)
    N, _, H, W = x.shape
    radii = []
    for w, _, _ in layers:
        R, S = w.shape[2], w.shape[3]
        if R != S:
            raise ValueError("chain_window assumes square filters")
        radii.append((R - 1) // 2)
    halo = sum(radii)
    z = _zero_crop(x, i0 - halo, i1 + halo, j0 - halo, j1 + halo)
    m = np.abs(z)
    for (w, b, relu), p in zip(layers, radii):
        w = _f64(w)
        b = None if b is None else _f64(b)
        zf, _ = conv2d(z, w, b, relu)
        mf, _ = conv2d(m, np.abs(w), None if b is None else np.abs(b), False)
        hh, ww = zf.shape[2], zf.shape[3]
        z = zf[:, :, p:hh - p, p:ww - p]
        m = mf[:, :, p:hh - p, p:ww - p]
        halo -= p
        rows = np.arange(i0 - halo, i1 + halo)
        cols = np.arange(j0 - halo, j1 + halo)
        outside = ((rows < 0) | (rows >= H))[:, None] | ((cols < 0) | (cols >= W))[None, :]
        z = np.where(outside[None, None], 0.0, z)
        m = np.where(outside[None, None], 0.0, m)
    return z, m


def _to_f16(a):
    """Round float64 values to fp16, nearest even, and widen back (exactly)."""
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


def _nhwc_to_nchw(a):
    return np.ascontiguousarray(np.transpose(a, (0, 3, 1, 2)))


def _nchw_to_nhwc(a):
    return np.ascontiguousarray(np.transpose(a, (0, 2, 3, 1)))


def chain_f16(x, layers, d2s=1):
    """fp16-storage chain on NHWC input, then depth-to-space by d2s (1 = none).

    x: N,H,W,C0 fp16 values; layers: sequence of (w, b, relu) with w K,C,R,R
    fp16 values and b fp32 or None. z_0 = x, z_l = f16(act(conv(z_{l-1}) + b)).
    Returns (out, m) in float64, NHWC: (N,H,W,K_last) or (N, d2s*H, d2s*W, 1).
    """
    z = _nhwc_to_nchw(_f64(x))
    m = np.abs(z)
    for w, b, relu in layers:
        w = _f64(w)
        b = None if b is None else _f64(b)
        z, _ = conv2d(z, w, b, relu, scale=False)
        z = _to_f16(z)
        m, _ = conv2d(m, np.abs(w), None if b is None else np.abs(b), False, scale=False)
    if d2s > 1:
        z = depth_to_space(z, d2s)
        m = depth_to_space(m, d2s)
    return _nchw_to_nhwc(z), _nchw_to_nhwc(m)


def chain_f16_window(x, layers, i0, i1, j0, j1):
    """fp16-storage chain output (before depth-to-space, NHWC) on rows [i0,i1) x
    cols [j0,j1) only: as chain_window, with every layer's output rounded to fp16
    inside the image and zero outside it. Same result as
    chain_f16(x, layers)[0][:, i0:i1, j0:j1, :]."""
    x = _nhwc_to_nchw(_f64(x))
    N, _, H, W = x.shape
    radii = []
    for w, _, _ in layers:
        R, S = w.shape[2], w.shape[3]
        if R != S:
            raise ValueError("chain_f16_window assumes square filters")
        radii.append((R - 1) // 2)
    halo = sum(radii)
    z = _zero_crop(x, i0 - halo, i1 + halo, j0 - halo, j1 + halo)
    m = np.abs(z)
    for (w, b, relu), p in zip(layers, radii):
        w = _f64(w)
        b = None if b is None else _f64(b)
        zf, _ = conv2d(z, w, b, relu)
        mf, _ = conv2d(m, np.abs(w), None if b is None else np.abs(b), False)
        hh, ww = zf.shape[2], zf.shape[3]
        z = _to_f16(zf[:, :, p:hh - p, p:ww - p])
        m = mf[:, :, p:hh - p, p:ww - p]
        halo -= p
        rows = np.arange(i0 - halo, i1 + halo)
        cols = np.arange(j0 - halo, j1 + halo)
        outside = ((rows < 0) | (rows >= H))[:, None] | ((cols < 0) | (cols >= W))[None, :]
        z = np.where(outside[None, None], 0.0, z)
        m = np.where(outside[None, None], 0.0, m)
    return _nchw_to_nhwc(z), _nchw_to_nhwc(m)
