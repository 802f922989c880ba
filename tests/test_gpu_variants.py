"""GPU parity of every tuning variant, and the runtime tuner.

Each variant of a descriptor (conv2d_list_variants: the default kernel and
tile, the other strip heights, channel groups, swizzles and kernel families
that take the shape) must give the oracle's result on ragged shapes; the tuner
must time them all, keep the fastest and leave its result in y.
"""
import numpy as np
import pytest

import image_stencil_amd as isa
import oracle
import synth
from gpu_util import dev, host, say
from tolerance import TAU_F16, TAU_F32, check

pytestmark = pytest.mark.gpu


def _case(name):
    """(desc, x, w, b, relu, layout, weights passed to the kernel, oracle result)"""
    if name == "single_3x3":
        x, w = synth.single_channel(300, 700, 3, seed=1)
        d = isa.make_desc(1, 1, 300, 700, 1, 3, 3)
        return d, x, w, None, False, "NCHW", w, oracle.conv2d(x, w)
    if name == "separable_5x5":
        x, _ = synth.single_channel(257, 516, 5, seed=2)
        rng = np.random.default_rng(3)
        col, row = (rng.standard_normal(5) / 5).astype(np.float32), (rng.standard_normal(5) / 5).astype(np.float32)
        d = isa.make_desc(1, 1, 257, 516, 1, 5, 5, separable=True)
        return d, x, None, None, False, "NCHW", np.concatenate([col, row]), oracle.conv2d_separable(x, col, row)
    if name == "fp32_32to32":
        x, w, b = synth.cnn_layer_f32(N=1, C=32, K=32, H=50, W=200, seed=4)
        d = isa.make_desc(1, 32, 50, 200, 32, 3, 3, "f32", True)
        return d, x, w, b, True, "NCHW", w, oracle.conv2d(x, w, b, True)
    if name == "fp32_32to4":
        # the matrix-core and vector forms of the 4-filter layer (ragged tiles, 2 images)
        x, w, b = synth.cnn_layer_f32(N=2, C=32, K=4, H=45, W=140, seed=9)
        d = isa.make_desc(2, 32, 45, 140, 4, 3, 3, "f32", True)
        return d, x, w, b, True, "NCHW", w, oracle.conv2d(x, w, b, True)
    if name == "one_channel_8_filters":
        x, w, b = synth.cnn_layer_f32(N=2, C=1, K=8, H=40, W=136, R=5, seed=5)
        d = isa.make_desc(2, 1, 40, 136, 8, 5, 5, "f32", False)
        return d, x, w, b, False, "NCHW", w, oracle.conv2d(x, w, b, False)
    if name.startswith("fanout_"):
        # one channel, F filters: every strip height of the single-channel
        # kernel's F-filter form next to the multi-channel kernel's groups
        N, H, W, K, R, relu = {"fanout_2x5x5": (2, 70, 300, 2, 5, True), "fanout_4x3x3_odd": (1, 45, 301, 4, 3, False),
                               "fanout_8x3x3": (1, 67, 520, 8, 3, True), "fanout_4x1x1": (2, 33, 260, 4, 1, False)}[name]
        x, w, b = synth.cnn_layer_f32(N=N, C=1, K=K, H=H, W=W, R=R, seed=K + R + H)
        d = isa.make_desc(N, 1, H, W, K, R, R, "f32", relu)
        return d, x, w, b, relu, "NCHW", w, oracle.conv2d(x, w, b, relu)
    if name == "pointwise_8to16":
        x, w, b = synth.cnn_layer_f32(N=2, C=8, K=16, H=33, W=132, R=1, seed=7)
        d = isa.make_desc(2, 8, 33, 132, 16, 1, 1, "f32", True)
        return d, x, w, b, True, "NCHW", w, oracle.conv2d(x, w, b, True)
    if name == "fp16_64to64":
        x, w, b = synth.cnn_layer_f16_nhwc(N=2, C=64, K=64, H=37, W=70, seed=6)
        d = isa.make_desc(2, 64, 37, 70, 64, 3, 3, "f16", False)
        return d, x, w, b, False, "NHWC", w, oracle.conv2d(x, w, b, False, "NHWC")
    raise KeyError(name)


def _run(plan, x, wk, b, d):
    import torch
    if d.layout == isa.IS_NHWC:
        y = torch.full((d.n, d.h, d.w, d.k), float("nan"), dtype=torch.float16, device="cuda")
    else:
        y = torch.full((d.n, d.k, d.h, d.w), float("nan"), dtype=torch.float32, device="cuda")
    xd, wd = dev(x), dev(wk)
    bd = dev(b) if b is not None else None
    plan.forward(xd, wd, bd, y)
    return host(y), (xd, wd, bd, y)


CASES = ["single_3x3", "separable_5x5", "fp32_32to32", "fp32_32to4", "one_channel_8_filters", "pointwise_8to16",
         "fp16_64to64", "fanout_2x5x5", "fanout_4x3x3_odd", "fanout_8x3x3", "fanout_4x1x1"]


@pytest.mark.parametrize("name", CASES)
def test_every_variant_matches_oracle(name):
    d, x, w, b, relu, layout, wk, (ref, m) = _case(name)
    tau = TAU_F16 if layout == "NHWC" else TAU_F32
    variants = isa.conv2d_list_variants(d)
    assert len(variants) >= 2, variants
    if name.startswith("fanout_"):
        assert sum(v["kernel"] == "is_k1_single_fanout" for v in variants) == 6, variants
    for i, v in enumerate(variants):
        say("variant", name, i, v["kernel"], v["param"])
        plan = isa.Plan(d, variant=i)
        assert plan.info()["kernel"] == v["kernel"]
        y, _ = _run(plan, x, wk, b, d)
        check(y, ref, m, tau, "%s variant %s/%d" % (name, v["kernel"], v["param"]))


@pytest.mark.parametrize("name", ["single_3x3", "fp32_32to32", "fp16_64to64"])
def test_autotune_keeps_the_fastest(name):
    d, x, w, b, relu, layout, wk, (ref, m) = _case(name)
    tau = TAU_F16 if layout == "NHWC" else TAU_F32
    plan = isa.Plan(d)
    _, (xd, wd, bd, y) = _run(plan, x, wk, b, d)
    y.fill_(float("nan"))
    say("autotune", name)
    measured = plan.autotune(xd, wd, bd, y, reps=5)
    assert len(measured) == len(isa.conv2d_list_variants(d))
    assert all(v["ms"] > 0 for v in measured), measured
    assert measured[0]["is_default"] and not any(v["is_default"] for v in measured[1:])
    best = min(measured, key=lambda v: v["ms"])
    info = plan.info()
    assert info["kernel"] == best["kernel"]
    say("chose %s/%d" % (best["kernel"], best["param"]), ["%s/%d %.4f" % (v["kernel"], v["param"], v["ms"])
                                                         for v in measured])
    # y holds the chosen variant's result; a forward with the tuned plan too.
    check(host(y), ref, m, tau, "%s after autotune" % name)
    y.fill_(float("nan"))
    plan.forward(xd, wd, bd, y)
    check(host(y), ref, m, tau, "%s tuned forward" % name)


def test_autotune_on_the_8192_image():
    """The headline shape: the tuner's pick is at least as fast as the default
    strip height in its own measurement, and the result is right on sampled rows."""
    import torch
    x, w = synth.large_image(5)
    d = isa.make_desc(1, 1, 8192, 8192, 1, 5, 5)
    plan = isa.Plan(d)
    xd, wd = dev(x), dev(w)
    y = torch.empty((1, 1, 8192, 8192), device="cuda")
    measured = plan.autotune(xd, wd, None, y, reps=5)
    best = min(v["ms"] for v in measured)
    assert best <= measured[0]["ms"]
    say("8192^2 5x5 variants", ["%d: %.4f" % (v["param"], v["ms"]) for v in measured])
    rows = [0, 1, 2, 63, 64, 65, 127, 128, 4095, 4096, 8190, 8191]
    pts = np.array([(0, 0, i, j) for i in rows for j in range(8192)], np.int64)
    ref, m = oracle.conv2d_points(x, w, None, False, pts)
    got = host(y)[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]]
    check(got, ref, m, TAU_F32, "8192^2 after autotune")


def test_fanout_default_on_a_4096_image():
    """One channel, 2 filters 5x5 with bias and ReLU on 4096x4096: the default
    plan is the single-channel kernel's F-filter form; both output planes are
    checked on whole rows at strip boundaries and at the image edges."""
    import torch
    x, w, b = synth.cnn_layer_f32(N=1, C=1, K=2, H=4096, W=4096, R=5, seed=11)
    d = isa.make_desc(1, 1, 4096, 4096, 2, 5, 5, "f32", True)
    plan = isa.Plan(d)
    assert plan.info()["kernel"] == "is_k1_single_fanout"
    y = torch.full((1, 2, 4096, 4096), float("nan"), device="cuda")
    say("fanout 4096^2 default")
    plan.forward(dev(x), dev(w), dev(b), y)
    rows = [0, 1, 63, 64, 65, 2047, 2048, 4094, 4095]
    pts = np.array([(0, k, i, j) for k in range(2) for i in rows for j in range(4096)], np.int64)
    ref, m = oracle.conv2d_points(x, w, b, True, pts)
    got = host(y)[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]]
    check(got, ref, m, TAU_F32, "fanout 4096^2")
