"""GPU parity of the fp16 NHWC layer (MFMA implicit GEMM) against the oracle.

fp16 inputs and weights, fp32 bias and accumulation, fp16 output rounded to
nearest even: |y - y_ref| <= 2e-3 * m per element, m = sum |w*x| + |b|. The
oracle consumes the same fp16 values, widened exactly. Shapes cover exact and
ragged 64-row x 32-column units (and the 4-row stages inside them), single
pixels, batches, more units than workgroups, and the full 8x256x256x64 layer
(every output).
"""
import numpy as np
import pytest

import image_stencil_amd as isa
import oracle
import synth
from gpu_util import dev, host, say
from tolerance import TAU_F16, check

pytestmark = pytest.mark.gpu


def _run(x, w, b, relu, expect=None):
    import torch
    N, H, W, C = x.shape
    K, _, R, S = w.shape
    plan = isa.Plan(isa.make_desc(N, C, H, W, K, R, S, "f16", relu))
    if expect:
        assert plan.info()["kernel"] == expect
    y = torch.full((N, H, W, K), float("nan"), dtype=torch.float16, device="cuda")
    plan.forward(dev(x), dev(w), dev(b) if b is not None else None, y)
    return host(y)


@pytest.mark.parametrize("N,H,W", [(1, 8, 32), (2, 20, 40), (1, 1, 1), (1, 9, 33), (3, 17, 70), (1, 64, 64),
                                   (1, 130, 96), (2, 65, 33), (1, 66, 31)])
@pytest.mark.parametrize("relu", [False, True])
def test_mfma_layer_shapes(N, H, W, relu):
    x, w, b = synth.cnn_layer_f16_nhwc(N=N, H=H, W=W, seed=N * 100 + H + W)
    say("mfma", N, H, W, relu)
    y = _run(x, w, b, relu, "is_k4_mfma")
    ref, m = oracle.conv2d(x, w, b, relu, "NHWC")
    ratio = check(y, ref, m, TAU_F16, "mfma %dx%dx%d" % (N, H, W))
    say("max err/bound %.3g" % ratio)


def test_mfma_no_bias():
    x, w, _ = synth.cnn_layer_f16_nhwc(N=1, H=16, W=40, seed=5)
    y = _run(x, w, None, False, "is_k4_mfma")
    ref, m = oracle.conv2d(x, w, None, False, "NHWC")
    check(y, ref, m, TAU_F16, "mfma no bias")


def test_mfma_delta_weights_exact():
    """One-hot weights copy one shifted input channel: every product is exact and
    the fp16 input survives the fp32 sum and the rounding back to fp16."""
    x, _, _ = synth.cnn_layer_f16_nhwc(N=1, H=19, W=45, seed=6)
    w = np.zeros((64, 64, 3, 3), np.float16)
    rng = np.random.default_rng(7)
    for k in range(64):
        w[k, rng.integers(0, 64), rng.integers(0, 3), rng.integers(0, 3)] = 1.0
    y = _run(x, w, None, False, "is_k4_mfma")
    ref, _ = oracle.conv2d(x, w, None, False, "NHWC")
    np.testing.assert_array_equal(y.astype(np.float64), ref)


def test_f16_other_channel_counts_use_generic_kernel():
    x, w, b = synth.cnn_layer_f16_nhwc(N=1, C=16, K=8, H=12, W=20, seed=8)
    y = _run(x, w, b, True, "is_k0_generic_nhwc_f16")
    ref, m = oracle.conv2d(x, w, b, True, "NHWC")
    check(y, ref, m, TAU_F16, "generic f16")


def test_mfma_layer_8x256x256_full():
    """8 x 256 x 256 x 64 -> 64, the launch the benchmark times: every output
    against the oracle."""
    x, w, b = synth.cnn_layer_f16_nhwc()
    say("mfma full layer")
    y = _run(x, w, b, False, "is_k4_mfma")
    ref, m = oracle.conv2d(x, w, b, False, "NHWC")
    ratio = check(y, ref, m, TAU_F16, "8x256x256x64 fp16 layer full")
    say("max err/bound %.3g" % ratio)


def test_mfma_layer_more_units_than_workgroups():
    """3 x 700 x 260: 3 * 11 * 9 = 297 units on 256 workgroups, so some
    workgroups run two units back to back; rows on unit and stage edges."""
    x, w, b = synth.cnn_layer_f16_nhwc(N=3, H=700, W=260, seed=11)
    say("mfma 3x700x260")
    y = _run(x, w, b, True, "is_k4_mfma")
    assert np.isfinite(y.astype(np.float32)).all()
    rows = [0, 1, 3, 4, 62, 63, 64, 65, 127, 128, 639, 640, 698, 699]
    cols = list(range(0, 260, 7)) + [31, 32, 255, 256, 259]
    pts = np.array([(n, k, i, j) for n in range(3) for i in rows for j in cols for k in range(0, 64, 5)], np.int64)
    ref, m = oracle.conv2d_points(x, w, b, True, pts, "NHWC")
    got = y[pts[:, 0], pts[:, 2], pts[:, 3], pts[:, 1]]
    ratio = check(got, ref, m, TAU_F16, "3x700x260 layer")
    say("sampled %d outputs, max err/bound %.3g" % (len(pts), ratio))


@pytest.mark.parametrize("C,K", [(64, 32), (32, 32), (32, 16)])
@pytest.mark.parametrize("N,H,W", [(1, 8, 32), (2, 37, 70), (1, 66, 130), (1, 1, 1), (1, 40, 257), (1, 64, 96)])
def test_mfma_other_channel_counts(C, K, N, H, W):
    """The upscaling network's other fp16 layers (64 -> 32, 32 -> 32, 32 -> 16):
    wider units (64 and 128 pixels), shorter ones for 16 outputs, ragged edges;
    60- and 30-row units where they compute fewer rows, 64 and 32 rows at H = 64."""
    x, w, b = synth.cnn_layer_f16_nhwc(N=N, C=C, K=K, H=H, W=W, seed=C + K + H + W)
    say("mfma", C, K, N, H, W)
    y = _run(x, w, b, True, "is_k4_mfma")
    ref, m = oracle.conv2d(x, w, b, True, "NHWC")
    check(y, ref, m, TAU_F16, "mfma %d->%d %dx%dx%d" % (C, K, N, H, W))


@pytest.mark.parametrize("C,K", [(64, 32), (32, 16)])
def test_mfma_other_channel_counts_1280x720_full(C, K):
    """Two 1280x720 frames (more units than workgroups, 60-row units for the
    64-channel input): every output against the oracle."""
    x, w, b = synth.cnn_layer_f16_nhwc(N=2, C=C, K=K, H=720, W=1280, seed=C * 3 + K)
    say("mfma 2x720x1280 full", C, K)
    y = _run(x, w, b, True, "is_k4_mfma")
    ref, m = oracle.conv2d(x, w, b, True, "NHWC")
    ratio = check(y, ref, m, TAU_F16, "2x720x1280 fp16 %d->%d full" % (C, K))
    say("max err/bound %.3g" % ratio)


def test_mfma_largest_image():
    """The fp16 layer at the plan's 32-bit offset limit (2 H W C bytes just
    under 4e9: one 5000 x 6248 x 64 image). Windows in the first and last units
    and across unit seams in the middle are compared with the oracle run on
    those windows plus a one-pixel border of input (a window's own border
    outputs are compared only where they are the image's)."""
    import torch
    H, W = 5000, 6248
    x, w, b = synth.cnn_layer_f16_nhwc(N=1, H=H, W=W, seed=22)
    plan = isa.Plan(isa.make_desc(1, 64, H, W, 64, 3, 3, "f16", False))
    assert plan.info()["kernel"] == "is_k4_mfma"
    say("fp16 mfma largest image", H, W)
    xd = dev(x)
    y = torch.full((1, H, W, 64), float("nan"), dtype=torch.float16, device="cuda")
    plan.forward(xd, dev(w), dev(b), y)
    for r0, r1, c0, c1 in [(0, 70, 0, 40), (2530, 2600, 3100, 3140), (H - 70, H, W - 40, W)]:
        lr, hr, lc, hc = max(0, r0 - 1), min(H, r1 + 1), max(0, c0 - 1), min(W, c1 + 1)
        ref, m = oracle.conv2d(x[:, lr:hr, lc:hc, :], w, b, False, "NHWC")
        got = host(y[:, lr:hr, lc:hc, :].contiguous())
        ar, br = (0 if lr == 0 else 1), (hr - lr if hr == H else hr - lr - 1)
        ac, bc = (0 if lc == 0 else 1), (hc - lc if hc == W else hc - lc - 1)
        sl = (slice(None), slice(ar, br), slice(ac, bc), slice(None))
        ratio = check(got[sl], ref[sl], m[sl], TAU_F16, "fp16 mfma %dx%d rows %d..%d cols %d..%d" % (
            H, W, lr + ar, lr + br, lc + ac, lc + bc))
        say("max err/bound %.3g" % ratio)
