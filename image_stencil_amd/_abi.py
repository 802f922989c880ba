"""ctypes declarations of include/imgstencil.h (argument marshalling only).

Every computation happens in libimgstencil.so (HIP kernels for gfx950). If the
library is not built, loading fails loudly: there is no other code path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libimgstencil.so")

IS_OK, IS_ERR_INVALID_ARG, IS_ERR_UNSUPPORTED, IS_ERR_MISALIGNED, IS_ERR_HIP, IS_ERR_NO_MEMORY, \
    IS_ERR_WORKSPACE = range(7)
IS_F32, IS_F16 = 0, 1
IS_NCHW, IS_NHWC = 0, 1
IS_CHAIN_AUTO, IS_CHAIN_FUSED, IS_CHAIN_UNFUSED = 0, 1, 2
IS_MAX_CHAIN = 8
IS_NOALLOC_MAX_WORKSPACE = 256 << 20

STATUS_NAMES = {0: "IS_OK", 1: "IS_ERR_INVALID_ARG", 2: "IS_ERR_UNSUPPORTED", 3: "IS_ERR_MISALIGNED",
                4: "IS_ERR_HIP", 5: "IS_ERR_NO_MEMORY", 6: "IS_ERR_WORKSPACE"}


class conv2d_desc(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in
                ("n", "c", "h", "w", "k", "r", "s", "pad_h", "pad_w", "stride_h", "stride_w",
                 "in_dtype", "out_dtype", "layout", "relu", "separable")]


class conv2d_plan_info(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 64), ("grid_x", ctypes.c_int), ("grid_y", ctypes.c_int),
                ("grid_z", ctypes.c_int), ("block", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("tile_w", ctypes.c_int), ("tile_h", ctypes.c_int), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


class conv2d_variant(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 64), ("param", ctypes.c_int), ("is_default", ctypes.c_int),
                ("ms", ctypes.c_float)]


class conv_layer_desc(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in ("c", "k", "r", "s", "relu")]


class conv_chain_desc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int), ("h", ctypes.c_int), ("w", ctypes.c_int), ("n_layers", ctypes.c_int),
                ("layer", conv_layer_desc * IS_MAX_CHAIN), ("depth_to_space", ctypes.c_int),
                ("dtype", ctypes.c_int), ("mode", ctypes.c_int)]


# (name, restype, argtypes) of every function the header declares.
_vp = ctypes.c_void_p
SIGNATURES = [
    ("conv2d_create", ctypes.c_int, [ctypes.POINTER(conv2d_desc), ctypes.POINTER(_vp)]),
    ("conv2d_forward", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp]),
    ("conv2d_destroy", None, [_vp]),
    ("conv2d_get_plan_info", ctypes.c_int, [_vp, ctypes.POINTER(conv2d_plan_info)]),
    ("conv2d_list_variants", ctypes.c_int, [ctypes.POINTER(conv2d_desc), ctypes.POINTER(conv2d_variant),
                                            ctypes.c_int, ctypes.POINTER(ctypes.c_int)]),
    ("conv2d_create_variant", ctypes.c_int, [ctypes.POINTER(conv2d_desc), ctypes.c_int, ctypes.POINTER(_vp)]),
    ("conv2d_autotune", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int,
                                       ctypes.POINTER(conv2d_variant), ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_int)]),
    ("conv_chain_workspace_size", ctypes.c_int, [ctypes.POINTER(conv_chain_desc), ctypes.POINTER(ctypes.c_size_t)]),
    ("conv_chain_forward", ctypes.c_int, [ctypes.POINTER(conv_chain_desc), _vp, ctypes.POINTER(_vp),
                                          ctypes.POINTER(_vp), _vp, _vp, ctypes.c_size_t, _vp]),
    ("conv_chain_forward_noalloc", ctypes.c_int, [ctypes.POINTER(conv_chain_desc), _vp, ctypes.POINTER(_vp),
                                                  ctypes.POINTER(_vp), _vp, _vp]),
    ("conv_chain_kernel_name", ctypes.c_int, [ctypes.POINTER(conv_chain_desc), ctypes.c_char_p, ctypes.c_size_t]),
    ("conv_chain_groups", ctypes.c_int, [ctypes.POINTER(conv_chain_desc), ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_int)]),
    ("is_lds_tile_bytes", ctypes.c_size_t, [ctypes.c_int] * 6),
    ("is_swizzle_col", ctypes.c_int, [ctypes.c_int] * 5),
    ("is_persistent_grid", ctypes.c_int, [ctypes.c_int, ctypes.c_int]),
    ("is_status_str", ctypes.c_char_p, [ctypes.c_int]),
    ("is_last_hip_error", ctypes.c_int, []),
    ("is_version", ctypes.c_int, []),
]

_lib = None


def load():
    """Open libimgstencil.so and declare every signature; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libimgstencil.so is not built (%s); run __graft_entry__.build() "
                               "or python image_stencil_amd/build.py" % LIB_PATH)
        # Let torch load its HIP runtime first when it is installed: the library
        # then binds to that same libamdhip64.so.7, so that device pointers and
        # streams coming from torch are valid in it. Loaded first, the library
        # would pull in the system runtime, and torch would have to share it.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class ImgStencilError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        lib = load()
        msg = "%s: %s (%s)" % (where, STATUS_NAMES.get(status, status), lib.is_status_str(status).decode())
        if status == IS_ERR_HIP:
            msg += ", hipError_t %d" % lib.is_last_hip_error()
        super().__init__(msg)


def check(status, where):
    if status != IS_OK:
        raise ImgStencilError(status, where)
