"""Parity of the LDS-staging kernels in the LDS-poison debug build.

libimgstencil_ldspoison.so is the same library compiled with
IMGSTENCIL_LDS_POISON: every kernel that stages data in LDS first fills it with
a pattern that is NaN as fp32 and as fp16, so a read of LDS the kernel never
wrote (a missing wait or barrier, an unwritten halo or tail) propagates NaN
into the output, which the tolerance check rejects. Each shape below spans
several tiles with ragged edges for one kernel family.
"""
import ctypes
import os

import numpy as np
import pytest

import image_stencil_amd as isa
import oracle
import synth
from gpu_util import dev, host, say
from image_stencil_amd import _abi
from image_stencil_amd.build import LIB_LDS_POISON
from tolerance import TAU_F16, TAU_F32, check, tau_f16_chain

pytestmark = pytest.mark.gpu

_lib = None


def _poison_lib():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (the library binds to torch's HIP runtime)
        if not os.path.exists(LIB_LDS_POISON):
            raise RuntimeError("%s is not built; run __graft_entry__.build()" % LIB_LDS_POISON)
        lib = ctypes.CDLL(LIB_LDS_POISON)
        for name, res, args in _abi.SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _forward(d, x, w, b, y, variant=None):
    """variant: (kernel, param) of a tuning variant to run instead of the plan."""
    import torch
    lib = _poison_lib()
    plan = ctypes.c_void_p()
    if variant is None:
        assert lib.conv2d_create(ctypes.byref(d), ctypes.byref(plan)) == 0
    else:
        vs = [(v["kernel"], v["param"]) for v in isa.conv2d_list_variants(d)]
        assert lib.conv2d_create_variant(ctypes.byref(d), vs.index(variant), ctypes.byref(plan)) == 0
    info = _abi.conv2d_plan_info()
    assert lib.conv2d_get_plan_info(plan, ctypes.byref(info)) == 0
    st = lib.conv2d_forward(plan, x.data_ptr(), w.data_ptr(), b.data_ptr() if b is not None else None,
                            y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    lib.conv2d_destroy(plan)
    assert st == 0, st
    return info.kernel.decode()


LAYERS = [
    # (N, C, K, H, W, R, dtype, relu, expected kernel)
    (1, 8, 16, 37, 132, 3, "f32", True, "is_k2_multi_mfma"),
    (2, 1, 8, 40, 136, 5, "f32", False, "is_k2_multi"),
    (1, 32, 32, 50, 200, 3, "f32", True, "is_k5_mfma_f32"),
    (1, 16, 8, 33, 132, 1, "f32", False, "is_k8_pointwise"),
    (2, 64, 64, 37, 70, 3, "f16", False, "is_k4_mfma"),
    (1, 64, 32, 125, 96, 3, "f16", True, "is_k4_mfma"),
    (1, 32, 16, 21, 150, 3, "f16", False, "is_k4_mfma"),
    (1, 1, 64, 67, 129, 5, "f16", True, "is_k6_head_f16"),
    (2, 1, 32, 37, 132, 5, "f32", True, "is_k9_head_f32"),
    (1, 1, 16, 19, 68, 3, "f32", False, "is_k9_head_f32"),
    (1, 32, 4, 37, 132, 3, "f32", True, "is_k2_multi_mfma"),
    (2, 6, 4, 21, 72, 5, "f32", False, "is_k2_multi_mfma"),
    (1, 32, 3, 37, 132, 3, "f32", True, "is_k2_multi_mfma"),
    (2, 5, 3, 21, 72, 5, "f32", False, "is_k2_multi_mfma"),
    (1, 6, 5, 21, 72, 7, "f32", True, "is_k2_multi_mfma"),
    (2, 8, 6, 19, 70, 3, "f32", False, "is_k2_multi_mfma"),   # dword pixels (rows of 70)
    (1, 3, 4, 17, 133, 5, "f32", True, "is_k2_multi_mfma"),
]


@pytest.mark.parametrize("N,C,K,H,W,R,dtype,relu,kernel", LAYERS)
def test_layer_in_the_poison_build(N, C, K, H, W, R, dtype, relu, kernel):
    import torch
    say("lds poison", N, C, K, H, W, R, dtype)
    if dtype == "f16":
        x, w, b = synth.cnn_layer_f16_nhwc(N=N, C=C, K=K, H=H, W=W, R=R, seed=C + K + H)
        y = torch.full((N, H, W, K), float("nan"), dtype=torch.float16, device="cuda")
    else:
        x, w, b = synth.cnn_layer_f32(N=N, C=C, K=K, H=H, W=W, R=R, seed=C + K + H)
        y = torch.full((N, K, H, W), float("nan"), dtype=torch.float32, device="cuda")
    d = isa.make_desc(N, C, H, W, K, R, R, dtype, relu)
    assert _forward(d, dev(x), dev(w), dev(b), y) == kernel
    ref, m = oracle.conv2d(x, w, b, relu, "NHWC" if dtype == "f16" else "NCHW")
    check(host(y), ref, m, TAU_F16 if dtype == "f16" else TAU_F32, "poison %s" % kernel)


@pytest.mark.parametrize("N,C,K,H,W,R,relu,variant", [
    (1, 32, 32, 37, 132, 3, True, ("is_k2_multi", 32)),   # 4-channel slabs, 32 filters per workgroup
    (2, 8, 8, 21, 72, 3, False, ("is_k2_multi", 8)),
    (1, 12, 4, 19, 68, 3, True, ("is_k2_multi", 4)),
])
def test_vector_multichannel_variants_in_the_poison_build(N, C, K, H, W, R, relu, variant):
    """The register-blocked kernel's vector form over 4-channel slabs, which the
    plans now leave to its matrix-core form, run as a tuning variant."""
    import torch
    say("lds poison variant", N, C, K, H, W, R, variant)
    x, w, b = synth.cnn_layer_f32(N=N, C=C, K=K, H=H, W=W, R=R, seed=C + K + H)
    y = torch.full((N, K, H, W), float("nan"), dtype=torch.float32, device="cuda")
    d = isa.make_desc(N, C, H, W, K, R, R, "f32", relu)
    assert _forward(d, dev(x), dev(w), dev(b), y, variant) == variant[0]
    ref, m = oracle.conv2d(x, w, b, relu)
    check(host(y), ref, m, TAU_F32, "poison %s/%d" % variant)


def _chain(d, x, layers, y, ws_bytes):
    import torch
    lib = _poison_lib()
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    wl = [(dev(w), dev(b) if b is not None else None) for (w, b, _) in layers]
    W_ = (ctypes.c_void_p * _abi.IS_MAX_CHAIN)(*([w.data_ptr() for (w, _) in wl] +
                                                [None] * (_abi.IS_MAX_CHAIN - len(wl))))
    B_ = (ctypes.c_void_p * _abi.IS_MAX_CHAIN)(*([b.data_ptr() if b is not None else None for (_, b) in wl] +
                                                [None] * (_abi.IS_MAX_CHAIN - len(wl))))
    st = lib.conv_chain_forward(ctypes.byref(d), dev(x).data_ptr(), W_, B_, y.data_ptr(),
                                ws.data_ptr() if ws_bytes else None, ws_bytes,
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    return host(y)


@pytest.mark.parametrize("mode", ["fused", "unfused"])
def test_fp32_chain_in_the_poison_build(mode):
    """The upscaling chain in one launch (FUSED), or layer by layer (UNFUSED:
    the first-layer kernel, two 32 -> 32 MFMA layers and the 4-filter
    matrix-core layer with the depth-to-space in its stores)."""
    import torch
    x, layers = synth.chain_f32(N=1, H=37, W=120, seed=5)
    spec = [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]
    d = isa.make_chain_desc(1, 37, 120, spec, 2, isa.IS_CHAIN_FUSED if mode == "fused" else isa.IS_CHAIN_UNFUSED)
    ws_bytes = 0 if mode == "fused" else isa.conv_chain_workspace_size(d)
    y = torch.full((1, 1, 74, 240), float("nan"), device="cuda")
    got = _chain(d, x, layers, y, ws_bytes)
    ref, m = oracle.chain(x, layers, d2s=2)
    check(got, ref, m, TAU_F32, "poison %s chain" % mode)


@pytest.mark.parametrize("mode", ["auto", "unfused"])
def test_fp16_net_in_the_poison_build(mode):
    """The pages' net: the first two layers in one launch (AUTO: the first
    layer's rows computed into the LDS ring) or the first-layer kernel and an
    MFMA layer (UNFUSED), then two MFMA layers, the last with the
    depth-to-space in its stores."""
    import torch
    x, layers = synth.chain_f16_nhwc(N=1, H=33, W=70, seed=6)
    spec = [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]
    d = isa.make_chain_desc(1, 33, 70, spec, 3, isa.IS_CHAIN_AUTO if mode == "auto" else isa.IS_CHAIN_UNFUSED, "f16")
    ws_bytes = isa.conv_chain_workspace_size(d)
    y = torch.full((1, 99, 210, 1), float("nan"), dtype=torch.float16, device="cuda")
    got = _chain(d, x, layers, y, ws_bytes)
    ref, m = oracle.chain_f16(x, layers, d2s=3)
    check(got, ref, m, tau_f16_chain(len(layers)), "poison fp16 net")
