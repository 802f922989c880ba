"""GPU parity of single-channel filtering (C = K = 1, fp32 NCHW) against the oracle.

Every call goes through the C ABI (conv2d_create / conv2d_forward) on the
current HIP stream. Every output is compared, from ragged small images (several 256-column wave
segments and 64-row strips, ragged tails, widths that are not multiples of 4)
up to the full 8192x8192 image with each of the three filters.
"""
import numpy as np
import pytest

import image_stencil_amd as isa
import oracle
import synth
from gpu_util import dev, host, say
from tolerance import TAU_F32, check

pytestmark = pytest.mark.gpu


def _run(x, w, b=None, relu=False, expect="is_k1_single"):
    import torch
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    plan = isa.Plan(isa.make_desc(N, C, H, W, K, R, S, "f32", relu))
    assert plan.info()["kernel"] == expect
    xd, wd = dev(x), dev(w)
    bd = dev(b) if b is not None else None
    y = torch.full((N, K, H, W), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(xd, wd, bd, y)
    return host(y)


def test_small_image_3x3():
    """256x256 image, 3x3 normal(0,1) filter, seed 0, no bias: every output."""
    x, w = synth.small_image_3x3(seed=0)
    say("small image 3x3 256x256")
    y = _run(x, w)
    ref, m = oracle.conv2d(x, w)
    ratio = check(y, ref, m, TAU_F32, "256x256 3x3")
    say("max err/bound", ratio)


SHAPES = [(1, 1), (7, 3), (3, 260), (255, 257), (300, 700), (129, 1024), (1000, 260), (2, 1536)]
FILTERS = [(1, 1), (3, 3), (5, 5), (7, 7), (3, 7), (7, 1), (1, 5), (5, 3)]


@pytest.mark.parametrize("H,W", SHAPES)
@pytest.mark.parametrize("R,S", FILTERS)
def test_ragged_shapes(H, W, R, S):
    x, _ = synth.single_channel(H, W, R, N=2, seed=H * 31 + W)
    w = np.random.default_rng(R * 10 + S).standard_normal((1, 1, R, S)).astype(np.float32)
    say("single", H, W, R, S)
    y = _run(x, w)
    ref, m = oracle.conv2d(x, w)
    check(y, ref, m, TAU_F32, "single %dx%d R=%d S=%d" % (H, W, R, S))


@pytest.mark.parametrize("relu", [False, True])
def test_bias_and_relu(relu):
    x, w = synth.single_channel(300, 516, 5, N=1, seed=3)
    x = x - np.float32(0.5)
    b = np.array([0.125], np.float32)
    say("bias relu", relu)
    y = _run(x, w, b, relu)
    ref, m = oracle.conv2d(x, w, b, relu)
    check(y, ref, m, TAU_F32, "bias relu=%s" % relu)


def test_delta_filters_bit_exact():
    """A one-hot filter copies the shifted image: exact on the GPU too, since every
    product is by 1.0 or 0.0 and sums with zeros are exact."""
    x, _ = synth.single_channel(261, 520, 7, N=1, seed=5)
    for (R, S) in ((7, 7), (3, 5), (1, 1)):
        for u0 in range(R):
            for v0 in range(S):
                w = np.zeros((1, 1, R, S), np.float32)
                w[0, 0, u0, v0] = 1.0
                y = _run(x, w)
                ref, _ = oracle.conv2d(x, w)
                np.testing.assert_array_equal(y.astype(np.float64), ref, err_msg="delta %d,%d" % (u0, v0))


def test_empty_image_launches_nothing():
    import torch
    plan = isa.Plan(isa.make_desc(1, 1, 0, 16, 1, 3, 3))
    x = torch.zeros(16, device="cuda")
    w = torch.zeros(9, device="cuda")
    y = torch.zeros(16, device="cuda")
    plan.forward(x, w, None, y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("R", [3, 5, 7])
def test_large_image_full(R):
    """8192x8192 with an RxR normal(0, 1/(R*R)) filter, the launch the
    benchmark times: every output against the oracle."""
    x, w = synth.large_image(R)
    say("large image full", R)
    y = _run(x, w)
    ref, m = oracle.conv2d(x, w)
    ratio = check(y, ref, m, TAU_F32, "8192^2 %dx%d full" % (R, R))
    say("max err/bound %.3g" % ratio)


def test_widest_row_at_the_offset_limit():
    """Rows as wide as the kernel's 32-bit byte offsets allow (4 (W + 256) just
    under 2^31, the plan's limit): two rows of 2^29 - 260 columns with a 3x3
    filter. The first and last 600 columns and 600 columns around a wave
    segment boundary in the middle of the row are compared with the oracle run
    on those windows (with their neighbouring columns; a window's own edge
    columns are compared only where they are the image's)."""
    W = (1 << 29) - 260
    x, w = synth.single_channel(H=2, W=W, R=3, seed=11)
    plan = isa.Plan(isa.make_desc(1, 1, 2, W, 1, 3, 3))
    assert plan.info()["kernel"] == "is_k1_single"
    say("widest row", W)
    import torch
    xd = dev(x)
    del x
    y = torch.full((1, 1, 2, W), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(xd, dev(w), None, y)
    mid = (W // 512) * 256
    for c0, c1 in [(0, 600), (mid - 300, mid + 300), (W - 600, W)]:
        lo, hi = max(0, c0 - 1), min(W, c1 + 1)
        xs = host(xd[..., lo:hi].contiguous())
        ref, m = oracle.conv2d(xs, w)
        got = host(y[..., lo:hi].contiguous())
        a = 0 if lo == 0 else 1
        b = hi - lo if hi == W else hi - lo - 1
        ratio = check(got[..., a:b], ref[..., a:b], m[..., a:b], TAU_F32, "row of %d, columns %d..%d" % (W, lo + a, lo + b))
        say("columns %d..%d max err/bound %.3g" % (lo + a, lo + b, ratio))
