"""GPU parity of multi-channel fp32 NCHW layers against the oracle.

Calls go through the C ABI. Shapes span several tiles with ragged edges (64x16
for the register-blocked kernel and its 4-filter matrix-core form, 32 columns x
13 rows for the fp32 MFMA kernel that takes the 32 -> 32 3x3 layers, 64 columns
x 16 rows for the fp32 MFMA first layer that takes one input channel to 16, 32
or 64), channel counts that fill one or several LDS slabs, every output-channel
group size, and the full 1x32x720x1280 layer (every output, so every 13-row tile
seam). The 4-filter matrix-core form must also reproduce the vector form's bits.
"""
import numpy as np
import pytest

import image_stencil_amd as isa
import oracle
import synth
from gpu_util import dev, host, say
from tolerance import TAU_F32, check

pytestmark = pytest.mark.gpu


def _run(x, w, b, relu, expect=None):
    import torch
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    plan = isa.Plan(isa.make_desc(N, C, H, W, K, R, S, "f32", relu))
    if expect:
        assert plan.info()["kernel"] == expect
    y = torch.full((N, K, H, W), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(dev(x), dev(w), dev(b) if b is not None else None, y)
    return host(y)


CASES = [
    # N, C, K, H, W, R, relu, kernel
    (1, 32, 32, 50, 200, 3, True, "is_k5_mfma_f32"),
    (2, 32, 32, 37, 132, 3, False, "is_k5_mfma_f32"),
    (3, 32, 32, 19, 68, 3, True, "is_k5_mfma_f32"),
    (1, 32, 32, 16, 32, 3, False, "is_k5_mfma_f32"),
    (1, 32, 32, 1, 4, 3, True, "is_k5_mfma_f32"),
    (1, 32, 32, 33, 260, 3, False, "is_k5_mfma_f32"),
    (1, 32, 32, 9, 30, 3, False, "is_k2_multi_mfma"),   # rows of 30: dword pixels
    (2, 8, 16, 37, 132, 3, False, "is_k2_multi_mfma"),
    (1, 4, 8, 17, 68, 3, True, "is_k2_multi_mfma"),
    (1, 4, 4, 33, 64, 3, False, "is_k2_multi_mfma"),
    (1, 1, 32, 40, 136, 5, True, "is_k9_head_f32"),
    (1, 8, 32, 21, 72, 5, False, "is_k2_multi_mfma"),
    (1, 1, 32, 19, 68, 3, True, "is_k9_head_f32"),
    (1, 12, 32, 16, 64, 1, False, "is_k8_pointwise"),
    (1, 32, 4, 45, 140, 3, False, "is_k2_multi_mfma"),
    (3, 3, 8, 9, 20, 3, True, "is_k2_multi"),
    (2, 2, 8, 21, 72, 3, False, "is_k2_multi"),
    (1, 3, 32, 21, 72, 3, False, "is_k2_multi"),      # 16 filters per workgroup
    (1, 3, 32, 37, 132, 5, True, "is_k2_multi_mfma"),
    (2, 2, 16, 19, 68, 5, False, "is_k2_multi_mfma"),
    (1, 12, 8, 19, 68, 5, False, "is_k2_multi_mfma"),
    # K not a multiple of 4: the last group's missing filters are masked
    (1, 32, 3, 37, 132, 3, True, "is_k2_multi_mfma"),
    (2, 8, 1, 21, 72, 3, False, "is_k2_multi_mfma"),
    (1, 6, 6, 33, 196, 5, True, "is_k2_multi_mfma"),
    (3, 4, 7, 17, 68, 3, False, "is_k2_multi_mfma"),
    (1, 10, 2, 16, 64, 5, True, "is_k2_multi_mfma"),
    (1, 34, 5, 19, 260, 3, False, "is_k2_multi_mfma"),
    # odd channel counts the vector form does not take: 1-channel slabs
    (2, 5, 3, 37, 132, 3, True, "is_k2_multi_mfma"),
    (1, 3, 7, 21, 72, 5, False, "is_k2_multi_mfma"),
    (1, 7, 3, 17, 68, 5, True, "is_k2_multi_mfma"),
    # 7x7 over 1-channel slabs (the vector form has no 7x7)
    (1, 8, 8, 37, 132, 7, True, "is_k2_multi_mfma"),
    (2, 3, 5, 21, 72, 7, False, "is_k2_multi_mfma"),
    (1, 2, 16, 19, 68, 7, True, "is_k2_multi_mfma"),
    (1, 1, 4, 33, 136, 7, False, "is_k2_multi_mfma"),
    (1, 32, 4, 17, 196, 7, True, "is_k2_multi_mfma"),
    # 4 filters on the fp32 matrix cores: slabs of 2 channels through a ring of 4
    # LDS buffers (the 32-channel layer's unrolled form and the general loop:
    # 1, 3, 4, 5 and 17 slabs), 3x3 and 5x5, ragged tiles, several images
    (2, 32, 4, 37, 132, 3, True, "is_k2_multi_mfma"),
    (1, 32, 4, 16, 64, 3, False, "is_k2_multi_mfma"),
    (3, 32, 4, 1, 4, 3, True, "is_k2_multi_mfma"),
    (1, 2, 4, 21, 72, 3, True, "is_k2_multi"),
    (2, 6, 4, 40, 136, 5, False, "is_k2_multi_mfma"),
    (1, 8, 4, 33, 260, 5, True, "is_k2_multi_mfma"),
    (1, 10, 4, 19, 68, 3, False, "is_k2_multi_mfma"),
    (1, 34, 4, 17, 196, 3, True, "is_k2_multi_mfma"),
    # one input channel, F filters (F = 2 .. 12; 1x1, 3x3, 5x5)
    (1, 1, 4, 40, 136, 3, True, "is_k2_multi"),
    (2, 1, 8, 37, 132, 5, False, "is_k2_multi"),
    (1, 1, 2, 19, 68, 1, False, "is_k2_multi"),
    (1, 1, 12, 33, 260, 3, True, "is_k2_multi"),
    (1, 1, 6, 16, 64, 5, False, "is_k2_multi"),
    (1, 1, 16, 21, 72, 1, True, "is_k2_multi"),
    (1, 1, 3, 21, 72, 3, False, "is_k2_multi_mfma"),
    (1, 1, 3, 21, 70, 3, False, "is_k2_multi_mfma"),
    # one input channel to 16, 32 or 64 outputs, 3x3 or 5x5: the fp32 MFMA first
    # layer (16 x 64 tiles: ragged rows and columns, several tiles, images)
    (2, 1, 16, 37, 132, 3, False, "is_k9_head_f32"),
    (1, 1, 16, 1, 4, 5, True, "is_k9_head_f32"),
    (3, 1, 32, 17, 68, 5, False, "is_k9_head_f32"),
    (1, 1, 64, 33, 260, 5, True, "is_k9_head_f32"),
    (2, 1, 64, 16, 64, 3, False, "is_k9_head_f32"),
    (1, 1, 32, 45, 196, 5, True, "is_k9_head_f32"),
    (1, 1, 32, 21, 70, 5, True, "is_k2_multi_mfma"),
    # 1x1 filters over several channels: the pointwise kernel (planes of whole
    # 16-byte vectors, ragged last workgroup), else the fallback
    (1, 8, 16, 21, 72, 1, False, "is_k8_pointwise"),
    (2, 16, 8, 33, 132, 1, True, "is_k8_pointwise"),
    (1, 4, 4, 9, 64, 1, False, "is_k8_pointwise"),
    (1, 3, 4, 17, 68, 1, True, "is_k8_pointwise"),
    (3, 64, 32, 37, 140, 1, True, "is_k8_pointwise"),
    (1, 5, 12, 1, 4, 1, False, "is_k8_pointwise"),
    (1, 2, 4, 13, 20, 1, True, "is_k8_pointwise"),
    (1, 384, 32, 9, 64, 1, False, "is_k8_pointwise"),   # staged weights exactly 48 KB
    (1, 385, 32, 5, 64, 1, False, "is_k8_pointwise"),   # 16 channels per workgroup instead
    (1, 8, 16, 9, 30, 1, False, "is_k0_generic_nchw_f32"),
    (1, 5, 6, 11, 30, 5, False, "is_k2_multi_mfma"),
    (1, 8, 8, 10, 13, 3, True, "is_k2_multi_mfma"),
    # widths that are not whole 16-byte vectors, several tiles and images
    (2, 32, 4, 37, 130, 3, True, "is_k2_multi_mfma"),
    (1, 6, 9, 19, 197, 7, False, "is_k2_multi_mfma"),
    (3, 3, 16, 17, 67, 5, True, "is_k2_multi_mfma"),
    (1, 2, 8, 33, 1, 3, False, "is_k2_multi_mfma"),
    (1, 4, 4, 9, 30, 1, True, "is_k0_generic_nchw_f32"),
]


@pytest.mark.parametrize("N,C,K,H,W,R,relu,kernel", CASES)
def test_multichannel_shapes(N, C, K, H, W, R, relu, kernel):
    x, w, b = synth.cnn_layer_f32(N=N, C=C, K=K, H=H, W=W, R=R, seed=C * 7 + K)
    say("multi", N, C, K, H, W, R, relu)
    y = _run(x, w, b, relu, kernel)
    ref, m = oracle.conv2d(x, w, b, relu)
    ratio = check(y, ref, m, TAU_F32, "multi N%d C%d K%d %dx%d R%d" % (N, C, K, H, W, R))
    say("max err/bound %.3g" % ratio)


def test_no_bias():
    x, w, _ = synth.cnn_layer_f32(N=1, C=8, K=8, H=20, W=64, seed=2)
    y = _run(x, w, None, False, "is_k2_multi_mfma")
    ref, m = oracle.conv2d(x, w, None, False)
    check(y, ref, m, TAU_F32, "no bias")


def test_delta_weights_bit_exact():
    """One-hot weights per output channel copy a shifted input channel exactly."""
    x, _, _ = synth.cnn_layer_f32(N=1, C=8, K=8, H=33, W=136, seed=3)
    w = np.zeros((8, 8, 3, 3), np.float32)
    rng = np.random.default_rng(4)
    for k in range(8):
        w[k, rng.integers(0, 8), rng.integers(0, 3), rng.integers(0, 3)] = 1.0
    y = _run(x, w, None, False, "is_k2_multi_mfma")
    ref, _ = oracle.conv2d(x, w)
    np.testing.assert_array_equal(y.astype(np.float64), ref)


def test_mfma_f32_no_bias_and_delta_weights():
    """The fp32 MFMA kernel without bias, and with one-hot weights (each output
    channel copies one shifted input channel): products by 0 and 1 and their
    sums are exact, so the result must be too."""
    x, w, _ = synth.cnn_layer_f32(N=1, C=32, K=32, H=35, W=72, seed=6)
    y = _run(x, w, None, False, "is_k5_mfma_f32")
    ref, m = oracle.conv2d(x, w, None, False)
    check(y, ref, m, TAU_F32, "mfma f32 no bias")
    wd = np.zeros((32, 32, 3, 3), np.float32)
    rng = np.random.default_rng(7)
    for k in range(32):
        wd[k, rng.integers(0, 32), rng.integers(0, 3), rng.integers(0, 3)] = 1.0
    y = _run(x, wd, None, False, "is_k5_mfma_f32")
    ref, _ = oracle.conv2d(x, wd)
    np.testing.assert_array_equal(y.astype(np.float64), ref)


def test_head_f32_no_bias_and_delta_weights():
    """The fp32 first-layer kernel without bias, and with one-hot 5x5 filters
    (each output channel copies the image shifted by its tap): products by 0
    and 1 and their sums are exact, so the result must be too; the taps past
    the 25th, which the kernel pads with zeros, must not leak in."""
    x, w, _ = synth.cnn_layer_f32(N=1, C=1, K=32, H=35, W=72, R=5, seed=8)
    y = _run(x, w, None, False, "is_k9_head_f32")
    ref, m = oracle.conv2d(x, w, None, False)
    check(y, ref, m, TAU_F32, "head f32 no bias")
    wd = np.zeros((32, 1, 5, 5), np.float32)
    for k in range(32):
        wd[k, 0, (k % 25) // 5, (k % 25) % 5] = 1.0
    y = _run(x, wd, None, False, "is_k9_head_f32")
    ref, _ = oracle.conv2d(x, wd)
    np.testing.assert_array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("N,C,K,H,W,R,relu", [(1, 32, 4, 720, 1280, 3, False), (2, 32, 4, 45, 140, 3, True),
                                                (1, 6, 4, 40, 136, 5, True), (1, 34, 4, 17, 196, 3, False),
                                                (1, 8, 8, 33, 132, 3, True), (2, 16, 16, 21, 72, 3, False),
                                                (1, 64, 32, 19, 68, 3, True), (1, 12, 8, 17, 68, 5, False),
                                                (1, 6, 6, 21, 72, 3, True), (2, 10, 2, 19, 68, 5, False),
                                                (1, 2, 8, 33, 132, 3, False), (1, 5, 8, 19, 68, 3, True)])
def test_mfma_four_filters_bits_of_vector_path(N, C, K, H, W, R, relu):
    """The matrix-core form (4 filters per workgroup) rounds every accumulation
    once, in the vector form's order (channel, filter row, filter column), so
    it gives the same bits as every vector variant (any channels per
    workgroup); the 1280x720 case is the chain's last layer. The matrix-core
    result is also checked against the oracle."""
    import torch
    x, w, b = synth.cnn_layer_f32(N=N, C=C, K=K, H=H, W=W, R=R, seed=C + H + K)
    d = isa.make_desc(N, C, H, W, K, R, R, "f32", relu)
    names = [(v["kernel"], v["param"]) for v in isa.conv2d_list_variants(d)]
    mf = names.index(("is_k2_multi_mfma", 0))
    vec = [i for i, (k, _) in enumerate(names) if k == "is_k2_multi"]
    say("mfma vs vector", N, C, K, H, W, R, relu, [names[i] for i in vec])
    ys = []
    for i in [mf] + vec:
        y = torch.full((N, K, H, W), float("nan"), dtype=torch.float32, device="cuda")
        isa.Plan(d, variant=i).forward(dev(x), dev(w), dev(b), y)
        ys.append(host(y))
    for j in range(1, len(ys)):
        np.testing.assert_array_equal(ys[0], ys[j], err_msg=str(names[vec[j - 1]]))
    ref, m = oracle.conv2d(x, w, b, relu)
    ratio = check(ys[0], ref, m, TAU_F32, "mfma %d filters N%d C%d %dx%d R%d%s"
                  % (K, N, C, H, W, R, " (chain's last layer) full" if (H, W) == (720, 1280) else ""))
    say("max err/bound %.3g" % ratio)


def test_cnn_layer_720p_full():
    """1x32x720x1280 -> 32, 3x3, bias, ReLU, the launch the benchmark times:
    every output channel of every pixel against the oracle."""
    x, w, b = synth.cnn_layer_f32()
    say("cnn layer 720p full")
    y = _run(x, w, b, True, "is_k5_mfma_f32")
    ref, m = oracle.conv2d(x, w, b, True)
    ratio = check(y, ref, m, TAU_F32, "720p fp32 layer full")
    say("max err/bound %.3g" % ratio)


def test_mfma_f32_largest_image():
    """The fp32 MFMA layer at the plan's 32-bit offset limit (4 C H W bytes just
    under 2e9: 32 x 3840 x 4064 fp32, bias, ReLU). Windows in the first and
    last tiles and across tile seams in the middle are compared with the
    oracle run on those windows plus a one-pixel border of input (a window's own
    border outputs are compared only where they are the image's)."""
    import torch
    H, W = 3840, 4064
    x, w, b = synth.cnn_layer_f32(N=1, H=H, W=W, seed=21)
    plan = isa.Plan(isa.make_desc(1, 32, H, W, 32, 3, 3, "f32", True))
    assert plan.info()["kernel"] == "is_k5_mfma_f32"
    say("fp32 mfma largest image", H, W)
    y = torch.full((1, 32, H, W), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(dev(x), dev(w), dev(b), y)
    for r0, r1, c0, c1 in [(0, 30, 0, 70), (1940, 1972, 2010, 2080), (H - 30, H, W - 70, W)]:
        lr, hr, lc, hc = max(0, r0 - 1), min(H, r1 + 1), max(0, c0 - 1), min(W, c1 + 1)
        ref, m = oracle.conv2d(x[:, :, lr:hr, lc:hc], w, b, True)
        got = host(y[:, :, lr:hr, lc:hc].contiguous())
        ar, br = (0 if lr == 0 else 1), (hr - lr if hr == H else hr - lr - 1)
        ac, bc = (0 if lc == 0 else 1), (hc - lc if hc == W else hc - lc - 1)
        sl = (slice(None), slice(None), slice(ar, br), slice(ac, bc))
        ratio = check(got[sl], ref[sl], m[sl], TAU_F32, "fp32 mfma %dx%d rows %d..%d cols %d..%d" % (
            H, W, lr + ar, lr + br, lc + ac, lc + bc))
        say("max err/bound %.3g" % ratio)
