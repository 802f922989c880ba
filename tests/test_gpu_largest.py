"""GPU parity at the largest images the plans accept (their 32-bit offset
limits), for the kernels and chains not covered next to their other tests.

At these sizes the oracle runs on windows: each window of outputs is computed
from a crop of the input grown by the receptive field's radius (the sum of the
layers' radii), clipped to the image, so that every output of the window sees
either its true input or the image's zero padding. Windows sit at the first
tile, in the middle of the image (across tile seams) and at the last tile.
"""
import numpy as np
import pytest

import image_stencil_amd as isa
import oracle
import synth
from gpu_util import dev, host, say
from tolerance import TAU_F16, TAU_F32, check

pytestmark = pytest.mark.gpu


def _windows(H, W, h, w):
    """First, middle and last h x w windows of an H x W image."""
    return [(0, h, 0, w), (H // 2 - h // 2, H // 2 + h - h // 2, W // 2 - w // 2, W // 2 + w - w // 2),
            (H - h, H, W - w, W)]


def _check_windows(x, y, run_oracle, halo, scale, tau, label, nhwc=False):
    """x: host input, y: device output (scale x the input's rows and columns);
    run_oracle(crop) -> (ref, m) for that crop in the output's layout."""
    H, W = (x.shape[1], x.shape[2]) if nhwc else (x.shape[2], x.shape[3])
    for r0, r1, c0, c1 in _windows(H, W, 24, 40):
        lr, hr, lc, hc = max(0, r0 - halo), min(H, r1 + halo), max(0, c0 - halo), min(W, c1 + halo)
        if nhwc:
            ref, m = run_oracle(x[:, lr:hr, lc:hc, :])
            got = host(y[:, lr * scale:hr * scale, lc * scale:hc * scale, :].contiguous())
            sl = (slice(None), slice((r0 - lr) * scale, (r1 - lr) * scale),
                  slice((c0 - lc) * scale, (c1 - lc) * scale), slice(None))
        else:
            ref, m = run_oracle(x[:, :, lr:hr, lc:hc])
            got = host(y[:, :, lr * scale:hr * scale, lc * scale:hc * scale].contiguous())
            sl = (slice(None), slice(None), slice((r0 - lr) * scale, (r1 - lr) * scale),
                  slice((c0 - lc) * scale, (c1 - lc) * scale))
        ratio = check(got[sl], ref[sl], m[sl], tau, "%s rows %d..%d cols %d..%d" % (label, r0, r1, c0, c1))
        say("%s rows %d..%d: max err/bound %.3g" % (label, r0, r1, ratio))


def test_f32_first_layer_largest_image():
    """1 -> 32 5x5 on the fp32 matrix cores, bias and ReLU, 3840 x 4068
    (4 H W K bytes of output just under 2e9)."""
    import torch
    H, W = 3840, 4068
    x, layers = synth.chain_f32(N=1, H=H, W=W, spec=((1, 32, 5, True),), seed=31)
    w, b, relu = layers[0]
    plan = isa.Plan(isa.make_desc(1, 1, H, W, 32, 5, 5, "f32", relu))
    assert plan.info()["kernel"] == "is_k9_head_f32"
    y = torch.full((1, 32, H, W), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(dev(x), dev(w), dev(b), y)
    _check_windows(x, y, lambda c: oracle.conv2d(c, w, b, relu), 2, 1, TAU_F32, "fp32 first layer %dx%d" % (H, W))


def test_four_filter_matrix_core_layer_largest_image():
    """32 -> 4 3x3 on the 4x4x1 matrix-core form, 5000 x 6248 (4 C H W bytes
    of input just under 4e9)."""
    import torch
    H, W = 5000, 6248
    x, w, b = synth.cnn_layer_f32(N=1, C=32, K=4, H=H, W=W, seed=32)
    plan = isa.Plan(isa.make_desc(1, 32, H, W, 4, 3, 3, "f32", True))
    assert plan.info()["kernel"] == "is_k2_multi_mfma"
    y = torch.full((1, 4, H, W), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(dev(x), dev(w), dev(b), y)
    _check_windows(x, y, lambda c: oracle.conv2d(c, w, b, True), 1, 1, TAU_F32, "32->4 %dx%d" % (H, W))


def test_f16_first_layer_largest_image():
    """1 -> 64 5x5 fp16 NHWC, 5000 x 6248 (2 H W K bytes of output just under 4e9)."""
    import torch
    H, W = 5000, 6248
    x, layers = synth.chain_f16_nhwc(N=1, H=H, W=W, spec=((1, 64, 5, True),), seed=33)
    w, b, relu = layers[0]
    plan = isa.Plan(isa.make_desc(1, 1, H, W, 64, 5, 5, "f16", relu))
    assert plan.info()["kernel"] == "is_k6_head_f16"
    y = torch.full((1, H, W, 64), float("nan"), dtype=torch.float16, device="cuda")
    plan.forward(dev(x), dev(w), dev(b), y)
    _check_windows(x, y, lambda c: oracle.conv2d(c, w, b, relu, "NHWC"), 2, 1, TAU_F16,
                   "fp16 first layer %dx%d" % (H, W), nhwc=True)


def test_fused_stencil_pipeline_largest_image():
    """Three 3x3 filters fused in one launch, 20000 x 24996 (4 H W bytes just
    under 2e9)."""
    H, W = 20000, 24996
    spec = ((1, 1, 3, True), (1, 1, 3, True), (1, 1, 3, False))
    x, layers = synth.chain_f32(N=1, H=H, W=W, spec=spec, seed=34)
    d = isa.make_chain_desc(1, H, W, [(1, 1, 3, r) for (_, _, r) in layers], 1, isa.IS_CHAIN_AUTO)
    assert isa.conv_chain_kernel_name(d) == "is_k7_fused_stencil" and isa.conv_chain_groups(d) == [3]
    y = isa.conv_chain(dev(x), [(dev(w), dev(b), r) for (w, b, r) in layers], 1, isa.IS_CHAIN_AUTO)
    _check_windows(x, y, lambda c: oracle.chain(c, layers), 3, 1, TAU_F32, "pipeline %dx%d" % (H, W))


def test_fused_chain_largest_image():
    """The upscaling chain in one launch (1 -> 32 5x5, 32 -> 32 twice, 32 -> 4,
    depth-to-space x2), 15000 x 16664 (the 2x output's 16 H W bytes just under
    4e9)."""
    H, W = 15000, 16664
    x, layers = synth.chain_f32(N=1, H=H, W=W, seed=35)
    spec = [(w.shape[1], w.shape[0], w.shape[2], r) for (w, _, r) in layers]
    d = isa.make_chain_desc(1, H, W, spec, 2, isa.IS_CHAIN_FUSED)
    assert isa.conv_chain_kernel_name(d) == "is_k3_chain"
    y = isa.conv_chain(dev(x), [(dev(w), dev(b), r) for (w, b, r) in layers], 2, isa.IS_CHAIN_FUSED)
    assert tuple(y.shape) == (1, 1, 2 * H, 2 * W)
    _check_windows(x, y, lambda c: oracle.chain(c, layers, d2s=2), 5, 2, TAU_F32, "fused chain %dx%d" % (H, W))
