"""GPU parity of the separable single-channel path against the oracle.

A separable filter w[i][j] = col[i] * row[j] runs as a row pass and a column
pass inside the single-channel kernel (R + S products per pixel instead of
R * S); the oracle applies the outer-product filter by definition
(oracle.conv2d_separable). The tolerance scale is the same sum |w * x| (+ |b|),
because |col[i] * row[j]| = |col[i]| * |row[j]|.
"""
import numpy as np
import pytest

import image_stencil_amd as isa
import oracle
from gpu_util import dev, host, say
from tolerance import TAU_F32, check

pytestmark = pytest.mark.gpu


def _taps(R, seed):
    rng = np.random.default_rng(seed)
    col = (rng.standard_normal(R) / R).astype(np.float32)
    row = (rng.standard_normal(R) / R).astype(np.float32)
    return col, row


def _image(N, H, W, seed):
    rng = np.random.default_rng(seed)
    return rng.random((N, 1, H, W), dtype=np.float32)


def _run(x, col, row, b=None, relu=False):
    import torch
    N, _, H, W = x.shape
    R = col.size
    plan = isa.Plan(isa.make_desc(N, 1, H, W, 1, R, R, "f32", relu, separable=True))
    assert plan.info()["kernel"] == "is_k1_single_separable"
    y = torch.full((N, 1, H, W), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(dev(x), dev(np.concatenate([col, row])), dev(b) if b is not None else None, y)
    return host(y)


@pytest.mark.parametrize("N,H,W,R", [(1, 300, 700, 3), (1, 257, 516, 5), (2, 129, 1000, 7), (1, 64, 256, 7),
                                     (1, 1, 4, 3), (1, 70, 30, 5), (1, 7, 9, 7), (1, 200, 1030, 7)])
def test_separable_shapes(N, H, W, R):
    """Several strips and segments with ragged edges; widths that are not a
    multiple of 4 take the scalar-load variant."""
    x = _image(N, H, W, seed=H + W)
    col, row = _taps(R, seed=R)
    say("separable", N, H, W, R)
    y = _run(x, col, row)
    ref, m = oracle.conv2d_separable(x, col, row)
    ratio = check(y, ref, m, TAU_F32, "separable %dx%dx%d R%d" % (N, H, W, R))
    say("max err/bound %.3g" % ratio)


@pytest.mark.parametrize("relu", [False, True])
def test_separable_bias_relu(relu):
    x = _image(1, 130, 260, seed=5) - 0.5
    col, row = _taps(5, seed=6)
    b = np.array([0.05], np.float32)
    y = _run(x, col, row, b, relu)
    ref, m = oracle.conv2d_separable(x, col, row, b, relu)
    check(y, ref, m, TAU_F32, "separable bias relu=%s" % relu)


def test_separable_delta_taps_bit_exact():
    """One-hot column and row taps shift the image by whole pixels: products by
    0 and 1 and sums with 0 are exact, so the output is."""
    x = _image(1, 67, 264, seed=8)
    for (i, j) in ((0, 6), (3, 3), (6, 0), (2, 5)):
        col = np.zeros(7, np.float32)
        row = np.zeros(7, np.float32)
        col[i] = 1.0
        row[j] = 1.0
        y = _run(x, col, row)
        ref, _ = oracle.conv2d_separable(x, col, row)
        np.testing.assert_array_equal(y.astype(np.float64), ref)


def test_separable_8192_full():
    """8192 x 8192 with a 7x7 separable filter: every output against the
    oracle's full filter (the outer product of the taps)."""
    x = _image(1, 8192, 8192, seed=9)
    col, row = _taps(7, seed=10)
    say("separable 8192^2 7x7 full")
    y = _run(x, col, row)
    ref, m = oracle.conv2d_separable(x, col, row)
    ratio = check(y, ref, m, TAU_F32, "separable 8192^2 7x7 full")
    say("max err/bound %.3g" % ratio)


def test_separable_entry_matches_full_filter_within_rounding():
    """The Python helper: conv2d_separable(x, col, row) against the plain path
    with the outer-product filter (both within the oracle tolerance)."""
    import torch
    x = _image(1, 96, 320, seed=12)
    col, row = _taps(3, seed=13)
    got = host(isa.conv2d_separable(dev(x), dev(col), dev(row)))
    ref, m = oracle.conv2d_separable(x, col, row)
    check(got, ref, m, TAU_F32, "conv2d_separable helper")
    full = host(isa.conv2d(dev(x), torch.from_numpy(np.outer(col, row)[None, None].astype(np.float32)).cuda()))
    check(full, ref, m, TAU_F32, "outer-product filter on the plain path")
