"""GPU parity of the fp16-storage chain (the pages' upscaling net) and of its
first-layer kernel against the oracle.

The net of the StreamHPC CNN page ("Reducing memory traffic" table): 1 -> 64
(5x5), 64 -> 64, 64 -> 32, 32 -> 9 (3x3), ReLU after the first three layers,
data and weights stored as fp16, the 9 output channels as a 3x3 sub-pixel
upscale. Every layer's output is rounded to fp16 on both sides; the tolerance
of L layers is derived in tolerance.py (about L * 1.05e-3 * m). The 1280x720
frame is compared in full and on windows the oracle evaluates exactly
(chain_f16_window).
"""
import functools

import numpy as np
import pytest

import image_stencil_amd as isa
import oracle
import synth
from gpu_util import dev, host, say
from tolerance import TAU_F16, check, tau_f16_chain

pytestmark = pytest.mark.gpu


def _run_layer(x, w, b, relu, expect):
    import torch
    N, H, W, C = x.shape
    K, _, R, S = w.shape
    plan = isa.Plan(isa.make_desc(N, C, H, W, K, R, S, "f16", relu))
    assert plan.info()["kernel"] == expect
    y = torch.full((N, H, W, K), float("nan"), dtype=torch.float16, device="cuda")
    plan.forward(dev(x), dev(w), dev(b) if b is not None else None, y)
    return host(y)


@pytest.mark.parametrize("K,R", [(64, 5), (32, 5), (16, 3), (64, 3)])
@pytest.mark.parametrize("N,H,W", [(1, 16, 64), (2, 37, 70), (1, 1, 1), (1, 33, 129)])
def test_first_layer_kernel(K, R, N, H, W):
    """One input channel, K outputs: the taps form one MFMA k step."""
    x, w, b = synth.cnn_layer_f16_nhwc(N=N, C=1, K=K, H=H, W=W, R=R, seed=K + R + H + W)
    say("head f16", K, R, N, H, W)
    y = _run_layer(x, w, b, True, "is_k6_head_f16")
    ref, m = oracle.conv2d(x, w, b, True, "NHWC")
    check(y, ref, m, TAU_F16, "head 1->%d %dx%d %dx%dx%d" % (K, R, R, N, H, W))


def _chain(x, layers, d2s, mode=isa.IS_CHAIN_AUTO):
    dl = [(dev(w), dev(b) if b is not None else None, relu) for (w, b, relu) in layers]
    return host(isa.conv_chain(dev(x), dl, depth_to_space=d2s, mode=mode))


@pytest.mark.parametrize("N,H,W", [(1, 37, 70), (2, 20, 130), (1, 1, 1), (1, 66, 200), (1, 19, 77), (2, 35, 258),
                                   (1, 70, 2), (1, 120, 64), (1, 64, 100)])
def test_pages_net_small_frames(N, H, W):
    """AUTO (the first two layers in one launch) and UNFUSED (one launch per
    layer) against the oracle, and against each other bit for bit: both compute
    the first layer with the same products and round it to fp16 the same way."""
    x, layers = synth.chain_f16_nhwc(N=N, H=H, W=W, seed=N * 1000 + H + W)
    spec = [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]
    d = isa.make_chain_desc(N, H, W, spec, 3, isa.IS_CHAIN_AUTO, "f16")
    assert isa.conv_chain_kernel_name(d) == "head_fused"
    say("pages net", N, H, W)
    y = _chain(x, layers, 3)
    yu = _chain(x, layers, 3, isa.IS_CHAIN_UNFUSED)
    ref, m = oracle.chain_f16(x, layers, d2s=3)
    assert y.shape == (N, 3 * H, 3 * W, 1)
    ratio = check(y, ref, m, tau_f16_chain(len(layers)), "pages net %dx%dx%d" % (N, H, W))
    check(yu, ref, m, tau_f16_chain(len(layers)), "pages net unfused %dx%dx%d" % (N, H, W))
    np.testing.assert_array_equal(y.view(np.uint16), yu.view(np.uint16))
    say("max err/bound %.3g" % ratio)


@pytest.mark.parametrize("r", [3, 5])
@pytest.mark.parametrize("N,H,W,relu1,relu2,bias", [(1, 64, 32, True, True, True), (2, 37, 70, False, True, True),
                                                    (1, 1, 1, True, False, False), (1, 120, 33, True, True, False),
                                                    (1, 130, 96, False, False, True), (3, 9, 100, True, True, True)])
def test_head_fused_pair(r, N, H, W, relu1, relu2, bias):
    """Two layers, 1 -> 64 (r x r) and 64 -> 64 (3x3), in one launch: ragged
    32-column and 64-row (and 60-row, H = 120) units, single pixels, batches,
    either ReLU flag and no biases; against the oracle and against the two
    launches of the unfused path."""
    spec = ((1, 64, r, relu1), (64, 64, 3, relu2))
    x, layers = synth.chain_f16_nhwc(N=N, H=H, W=W, spec=spec, seed=r * 100 + H + W)
    if not bias:
        layers = [(w, None, rl) for (w, _, rl) in layers]
    d = isa.make_chain_desc(N, H, W, [(w.shape[1], w.shape[0], w.shape[2], rl) for (w, _, rl) in layers], 1,
                            isa.IS_CHAIN_AUTO, "f16")
    assert isa.conv_chain_kernel_name(d) == "head_fused"
    say("head fused pair", r, N, H, W, relu1, relu2, bias)
    y = _chain(x, layers, 1)
    yu = _chain(x, layers, 1, isa.IS_CHAIN_UNFUSED)
    ref, m = oracle.chain_f16(x, layers, d2s=1)
    ratio = check(y, ref, m, tau_f16_chain(2), "head fused r%d %dx%dx%d" % (r, N, H, W))
    np.testing.assert_array_equal(y.view(np.uint16), yu.view(np.uint16))
    say("max err/bound %.3g" % ratio)


def test_pages_net_1280x720_windows():
    """The full frame; windows at the corners, the edges, unit boundaries and
    inside, after the 3x3 depth-to-space (3840 x 2160 output)."""
    x, layers = synth.chain_f16_nhwc()
    say("pages net 1280x720")
    y = _chain(x, layers, 3)
    assert y.shape == (1, 2160, 3840, 1)
    assert np.isfinite(y.astype(np.float32)).all()
    tau = tau_f16_chain(len(layers))
    for (i0, i1, j0, j1) in [(0, 6, 0, 8), (62, 68, 126, 134), (350, 358, 636, 646), (714, 720, 1272, 1280),
                             (0, 4, 1270, 1280), (716, 720, 0, 6)]:
        z, m = oracle.chain_f16_window(x, layers, i0, i1, j0, j1)
        zt = np.transpose(z, (0, 3, 1, 2))
        mt = np.transpose(m, (0, 3, 1, 2))
        ref = np.transpose(oracle.depth_to_space(zt, 3), (0, 2, 3, 1))
        mref = np.transpose(oracle.depth_to_space(mt, 3), (0, 2, 3, 1))
        got = y[:, 3 * i0:3 * i1, 3 * j0:3 * j1, :]
        check(got, ref, mref, tau, "pages net window %s" % ((i0, i1, j0, j1),))


@pytest.mark.parametrize("mode", ["auto", "unfused"])
def test_pages_net_1280x720_full(mode):
    """The full frame, the first two layers in one launch (AUTO) and one launch
    per layer: every pixel of the 3840x2160 output against the oracle's
    fp16-storage chain."""
    x, layers = synth.chain_f16_nhwc()
    say("pages net 1280x720 full", mode)
    y = _chain(x, layers, 3, isa.IS_CHAIN_AUTO if mode == "auto" else isa.IS_CHAIN_UNFUSED)
    ref, m = _pages_net_frame_oracle()
    ratio = check(y, ref, m, tau_f16_chain(len(layers)), "pages net 1280x720 %s full" % mode)
    say("max err/bound %.3g" % ratio)


@functools.lru_cache(maxsize=1)
def _pages_net_frame_oracle():
    x, layers = synth.chain_f16_nhwc()
    return oracle.chain_f16(x, layers, d2s=3)


def test_f16_chain_other_shapes():
    """A 4-channel last layer with depth-to-space by 2, and a chain without
    depth-to-space (32 output channels written directly)."""
    spec2 = ((1, 32, 5, True), (32, 4, 3, False))
    x, layers = synth.chain_f16_nhwc(N=1, H=21, W=50, spec=spec2, seed=31)
    y = _chain(x, layers, 2)
    ref, m = oracle.chain_f16(x, layers, d2s=2)
    check(y, ref, m, tau_f16_chain(2), "f16 chain d2s 2")
    spec1 = ((1, 32, 5, True), (32, 32, 3, True))
    x, layers = synth.chain_f16_nhwc(N=2, H=19, W=40, spec=spec1, seed=32)
    y = _chain(x, layers, 1)
    ref, m = oracle.chain_f16(x, layers, d2s=1)
    check(y, ref, m, tau_f16_chain(2), "f16 chain no d2s")


def test_f16_chain_has_no_fused_mode():
    x, layers = synth.chain_f16_nhwc(N=1, H=8, W=8, seed=33)
    spec = [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]
    with pytest.raises(isa.ImgStencilError):
        isa.conv_chain_workspace_size(isa.make_chain_desc(1, 8, 8, spec, 3, isa.IS_CHAIN_FUSED, "f16"))
