"""GPU parity of the conv chain (fused kernel and layer-by-layer) against the oracle.

The upscaling chain: 5x5 1->32 + ReLU, 3x3 32->32 + ReLU (twice), 3x3 32->4,
depth-to-space x2. The oracle chains its fp64 layers and propagates the error
scale m_l = conv(|w_l|, m_{l-1}) + |b_l|; both GPU paths must stay within
1e-5 * m of it. Small frames cover many row blocks, partial strips and image
borders; the 1280x720 frame is compared in full.
"""
import functools

import numpy as np
import pytest

import image_stencil_amd as isa
import oracle
import synth
from gpu_util import dev, host, say
from tolerance import TAU_F32, check

pytestmark = pytest.mark.gpu


def _gpu_chain(x, layers, mode, d2s=2):
    import torch
    dl = [(dev(w), dev(b), relu) for (w, b, relu) in layers]
    y = isa.conv_chain(dev(x), dl, depth_to_space=d2s, mode=mode)
    return host(y)


def _spec(layers):
    return [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]


@pytest.mark.parametrize("N,H,W", [(1, 37, 120), (2, 20, 60), (1, 1, 4), (1, 70, 200), (1, 9, 56), (1, 130, 116)])
@pytest.mark.parametrize("mode", ["fused", "unfused"])
def test_upscale_chain_small(N, H, W, mode):
    x, layers = synth.chain_f32(N=N, H=H, W=W, seed=H + W)
    m_ = isa.IS_CHAIN_FUSED if mode == "fused" else isa.IS_CHAIN_UNFUSED
    d = isa.make_chain_desc(N, H, W, _spec(layers), 2, m_)
    assert isa.conv_chain_kernel_name(d) == ("is_k3_chain" if mode == "fused" else "layer_by_layer")
    say("chain", mode, N, H, W)
    y = _gpu_chain(x, layers, m_)
    ref, m = oracle.chain(x, layers, d2s=2)
    assert y.shape == ref.shape == (N, 1, 2 * H, 2 * W)
    ratio = check(y, ref, m, TAU_F32, "chain %s %dx%dx%d" % (mode, N, H, W))
    say("max err/bound %.3g" % ratio)


def test_fused_matches_unfused():
    x, layers = synth.chain_f32(N=1, H=90, W=340, seed=9)
    yf = _gpu_chain(x, layers, isa.IS_CHAIN_FUSED)
    yu = _gpu_chain(x, layers, isa.IS_CHAIN_UNFUSED)
    ref, m = oracle.chain(x, layers, d2s=2)
    check(yf, ref, m, TAU_F32, "fused")
    check(yu, ref, m, TAU_F32, "unfused")
    # the two GPU paths agree to twice the tolerance of each against the oracle
    assert np.all(np.abs(yf.astype(np.float64) - yu) <= 2 * TAU_F32 * m)


def test_relu_flags_and_no_bias():
    x, layers = synth.chain_f32(N=1, H=24, W=64, seed=10)
    layers = [(w, None if i == 2 else b, (i % 2 == 0)) for i, (w, b, _) in enumerate(layers)]
    import torch
    dl = [(dev(w), dev(b) if b is not None else None, relu) for (w, b, relu) in layers]
    y = host(isa.conv_chain(dev(x), dl, depth_to_space=2, mode=isa.IS_CHAIN_FUSED))
    ref, m = oracle.chain(x, layers, d2s=2)
    check(y, ref, m, TAU_F32, "relu flags")


def test_other_chains_run_layer_by_layer():
    spec = ((3, 8, 3, True), (8, 4, 5, False))
    x, layers = synth.chain_f32(N=1, H=21, W=40, spec=spec, seed=11)
    d = isa.make_chain_desc(1, 21, 40, _spec(layers), 1, isa.IS_CHAIN_AUTO)
    assert isa.conv_chain_kernel_name(d) == "layer_by_layer"
    with pytest.raises(isa.ImgStencilError):
        isa.conv_chain_workspace_size(isa.make_chain_desc(1, 21, 40, _spec(layers), 1, isa.IS_CHAIN_FUSED))
    y = _gpu_chain(x, layers, isa.IS_CHAIN_AUTO, d2s=1)
    ref, m = oracle.chain(x, layers, d2s=1)
    check(y, ref, m, TAU_F32, "2-layer chain")


def test_unfused_depth_to_space_pass_when_widths_are_ragged():
    """W = 30 (not a multiple of 4): the last layer runs on the fallback kernel
    and the depth-to-space is its own pass; W = 32 takes the 4-channel layer
    with the depth-to-space epilogue. Both against the oracle."""
    for W in (30, 32):
        x, layers = synth.chain_f32(N=1, H=13, W=W, seed=12)
        say("chain unfused", W)
        y = _gpu_chain(x, layers, isa.IS_CHAIN_UNFUSED)
        ref, m = oracle.chain(x, layers, d2s=2)
        check(y, ref, m, TAU_F32, "unfused chain W=%d" % W)


def test_auto_mode_uses_workspace_when_given():
    """AUTO runs layer by layer with the workspace it reports and falls back to
    the fused kernel without one; both match the oracle."""
    import torch
    x, layers = synth.chain_f32(N=1, H=30, W=72, seed=12)
    d = isa.make_chain_desc(1, 30, 72, _spec(layers), 2, isa.IS_CHAIN_AUTO)
    ws = isa.conv_chain_workspace_size(d)
    assert ws >= 2 * 4 * 32 * 30 * 72
    assert isa.conv_chain_kernel_name(d) == "layer_by_layer"
    ref, m = oracle.chain(x, layers, d2s=2)
    xd = dev(x)
    wl = [(dev(w), dev(b)) for (w, b, _) in layers]
    for ws_given in (ws, 0):
        y = torch.full((1, 1, 60, 144), float("nan"), dtype=torch.float32, device="cuda")
        buf = torch.empty(max(ws_given, 1), dtype=torch.uint8, device="cuda")
        isa.conv_chain_forward(d, xd.data_ptr(), [w.data_ptr() for (w, _) in wl], [b.data_ptr() for (_, b) in wl],
                               y.data_ptr(), buf.data_ptr() if ws_given else None, ws_given,
                               torch.cuda.current_stream().cuda_stream)
        check(host(y), ref, m, TAU_F32, "auto, workspace %d" % ws_given)


@functools.lru_cache(maxsize=1)
def _frame_oracle():
    """The 1280x720 chain's input, layers and oracle output (computed once)."""
    x, layers = synth.chain_f32()
    ref, m = oracle.chain(x, layers, d2s=2)
    return x, layers, ref, m


@pytest.mark.parametrize("mode", ["fused", "auto"])
def test_upscale_chain_720p_full(mode):
    """The 1280x720 frame through the fused kernel, and through AUTO with its
    workspace (layer by layer, the 32 -> 32 layers on the fp32 MFMA kernel):
    every pixel of the 2560x1440 output against the oracle."""
    say("chain 720p full", mode)
    x, layers, ref, m = _frame_oracle()
    m_ = isa.IS_CHAIN_FUSED if mode == "fused" else isa.IS_CHAIN_AUTO
    d = isa.make_chain_desc(1, 720, 1280, _spec(layers), 2, m_)
    assert isa.conv_chain_kernel_name(d) == ("is_k3_chain" if mode == "fused" else "layer_by_layer")
    y = _gpu_chain(x, layers, m_)
    assert y.shape == (1, 1, 1440, 2560)
    ratio = check(y, ref, m, TAU_F32, "720p chain %s full" % mode)
    say("max err/bound %.3g" % ratio)
