"""GPU parity of stencil pipelines (chains of single-channel filters) against
the oracle's chain, fused and unfused.

Fused groups evaluate 2 or 3 filters in one pass over warp-overlapped tiles;
their intermediate images never reach HBM, and each filter still sees zero
padding outside the image. The oracle composes the filters one by one
(oracle.chain), with the error scale propagated through the layers; the
intermediate results stay fp32 on the GPU, so the fp32 bound applies.
"""
import numpy as np
import pytest

import image_stencil_amd as isa
import oracle
from gpu_util import dev, host, say
from tolerance import TAU_F32, check

pytestmark = pytest.mark.gpu


def _pipeline(N, H, W, spec, seed):
    """spec: [(r, relu, with_bias)] -> x, layers [(w, b, relu)]"""
    rng = np.random.default_rng(seed)
    x = rng.random((N, 1, H, W), dtype=np.float32)
    layers = []
    for (r, relu, with_bias) in spec:
        w = (rng.standard_normal((1, 1, r, r)) / r).astype(np.float32)
        b = rng.standard_normal(1).astype(np.float32) * 0.1 if with_bias else None
        layers.append((w, b, relu))
    return x, layers


def _run(x, layers, mode, expect=None):
    N, _, H, W = x.shape
    spec = [(1, 1, w.shape[2], relu) for (w, b, relu) in layers]
    d = isa.make_chain_desc(N, H, W, spec, 1, mode)
    if expect is not None:
        assert isa.conv_chain_groups(d) == expect, isa.conv_chain_groups(d)
    dl = [(dev(w), dev(b) if b is not None else None, relu) for (w, b, relu) in layers]
    return host(isa.conv_chain(dev(x), dl, 1, mode))


SHAPES = [
    # N, H, W, [(r, relu, bias)], groups under AUTO
    (1, 300, 700, [(3, False, False), (3, False, False)], [2]),
    (2, 129, 500, [(3, True, True), (5, False, True)], [2]),
    (1, 257, 1000, [(5, True, True), (3, True, True), (5, False, False)], [3]),
    (1, 70, 244, [(3, False, True), (3, True, False), (3, False, True)], [3]),
    (1, 1, 4, [(3, False, True), (5, False, True)], [2]),
    (1, 5, 8, [(5, True, True), (5, True, True), (5, False, True)], [3]),
    (1, 64, 248, [(5, False, False), (5, False, False)], [2]),
    (1, 131, 260, [(3, True, True)] * 7, None),
    # one 7x7 filter in a fused group
    (1, 150, 300, [(7, True, True), (3, False, True)], None),
    (1, 77, 516, [(3, False, True), (3, True, False), (7, False, True)], None),
    (2, 40, 128, [(5, True, True), (7, False, False)], None),
]


@pytest.mark.parametrize("N,H,W,spec,groups", SHAPES)
def test_pipeline_matches_oracle(N, H, W, spec, groups):
    x, layers = _pipeline(N, H, W, spec, seed=H + W)
    ref, m = oracle.chain(x, layers)
    for mode in (isa.IS_CHAIN_AUTO, isa.IS_CHAIN_UNFUSED):
        say("pipeline", N, H, W, [r for (r, _, _) in spec], mode)
        y = _run(x, layers, mode, groups if mode == isa.IS_CHAIN_AUTO else [1] * len(spec))
        ratio = check(y, ref, m, TAU_F32, "pipeline %dx%dx%d mode %d" % (N, H, W, mode))
        say("max err/bound %.3g" % ratio)


@pytest.mark.parametrize("rs", [(7, 3), (3, 7), (7, 5), (5, 7), (7, 3, 3), (3, 7, 3), (3, 3, 7)])
def test_fused_groups_with_a_7x7_filter(rs):
    """Every fused group that holds a 7x7 filter, forced with IS_CHAIN_FUSED."""
    spec = [(r, i % 2 == 0, True) for i, r in enumerate(rs)]
    x, layers = _pipeline(1, 70, 264, spec, seed=sum(rs))
    ref, m = oracle.chain(x, layers)
    say("fused group", rs)
    y = _run(x, layers, isa.IS_CHAIN_FUSED, [len(rs)])
    check(y, ref, m, TAU_F32, "fused group %s" % (rs,))


def test_fused_delta_filters_bit_exact():
    """Unit-impulse filters: the pipeline is a pure shift with zero fill, which
    the fused kernel must reproduce exactly (products by 0 and 1, sums with 0)."""
    rng = np.random.default_rng(3)
    x = rng.random((1, 1, 90, 520), dtype=np.float32)
    layers = []
    for (r, i, j) in ((3, 0, 2), (5, 4, 1), (3, 1, 1)):
        w = np.zeros((1, 1, r, r), np.float32)
        w[0, 0, i, j] = 1.0
        layers.append((w, None, False))
    y = _run(x, layers, isa.IS_CHAIN_FUSED, [3])
    ref, _ = oracle.chain(x, layers)
    np.testing.assert_array_equal(y.astype(np.float64), ref)


def test_auto_without_workspace_runs_one_fused_group():
    import torch
    x, layers = _pipeline(1, 100, 400, [(3, True, True)] * 3, seed=4)
    d = isa.make_chain_desc(1, 100, 400, [(1, 1, 3, True)] * 3, 1, isa.IS_CHAIN_AUTO)
    y = torch.full((1, 1, 100, 400), float("nan"), device="cuda")
    dl = [(dev(w), dev(b)) for (w, b, _) in layers]
    isa.conv_chain_forward(d, dev(x).data_ptr(), [w.data_ptr() for (w, _) in dl], [b.data_ptr() for (_, b) in dl],
                           y.data_ptr(), None, 0, torch.cuda.current_stream().cuda_stream)
    ref, m = oracle.chain(x, layers)
    check(host(y), ref, m, TAU_F32, "auto without workspace")


@pytest.mark.parametrize("spec,groups", [([(3, True, True), (3, False, True)], [2]),
                                         ([(3, True, False)] * 3, [3])])
def test_pipeline_8192_full(spec, groups):
    """Two and three 3x3 filters on 8192^2 (the three with ReLU and no bias are
    the group the bench times, one fused launch): every output against the
    oracle's chain."""
    x, layers = _pipeline(1, 8192, 8192, spec, seed=5)
    say("pipeline 8192^2 full", len(spec))
    y = _run(x, layers, isa.IS_CHAIN_AUTO, groups)
    ref, m = oracle.chain(x, layers)
    ratio = check(y, ref, m, TAU_F32, "pipeline 8192^2 %d filters full" % len(spec))
    say("max err/bound %.3g" % ratio)
