"""The oracle against its pins (CPU only).

The oracle is the plain definition of a same-size, zero-padded, centred 2D
cross-correlation with bias and optional ReLU (per-pixel loop nest of the
StreamHPC page "Optimizing convolution kernels - CNNs in Vulkan Part 2/3",
section "Where we left off"). The pins in oracle_pins.py fix it from outside.
"""
import numpy as np
import pytest

import oracle
import oracle_pins
import synth


def _conv(x, w, b, relu, layout):
    return oracle.conv2d(x, w, b, relu, layout)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(_conv)


def test_separable_entry_is_row_then_column_pass():
    """conv2d_separable(x, col, row) equals a horizontal 1D pass with `row`
    followed by a vertical 1D pass with `col` (zero padding in each), for
    non-square sizes too, so that swapping the two tap vectors fails."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 1, 13, 17))
    for R, S in ((3, 3), (5, 5), (7, 7), (3, 7), (7, 1)):
        col, row = rng.standard_normal(R), rng.standard_normal(S)
        b = rng.standard_normal(1)
        y, m = oracle.conv2d_separable(x, col, row, b, False)
        want = oracle_pins._corr1d_cols(oracle_pins._corr1d_rows(x, row), col) + b[0]
        assert np.all(np.abs(y - want) <= oracle_pins.TIGHT * m + 1e-300), (R, S)
        y_relu, _ = oracle.conv2d_separable(x, col, row, b, True)
        np.testing.assert_array_equal(y_relu, np.maximum(y, 0.0))


def test_points_match_full():
    x, w, b = synth.cnn_layer_f32(N=2, C=3, K=5, H=9, W=14, R=3, seed=11)
    y, m = oracle.conv2d(x, w, b, True)
    rng = np.random.default_rng(12)
    pts = np.stack([rng.integers(0, 2, 40), rng.integers(0, 5, 40),
                    rng.integers(0, 9, 40), rng.integers(0, 14, 40)], axis=1)
    yp, mp = oracle.conv2d_points(x, w, b, True, pts)
    np.testing.assert_array_equal(yp, y[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]])
    np.testing.assert_array_equal(mp, m[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]])
    # NHWC points.
    xh = np.ascontiguousarray(x.transpose(0, 2, 3, 1))
    yh, _ = oracle.conv2d(xh, w, b, True, "NHWC")
    yph, _ = oracle.conv2d_points(xh, w, b, True, pts, "NHWC")
    np.testing.assert_array_equal(yph, yh[pts[:, 0], pts[:, 2], pts[:, 3], pts[:, 1]])


def test_depth_to_space_is_pixel_shuffle():
    import torch
    z = np.random.default_rng(13).standard_normal((2, 4, 5, 7))
    out = oracle.depth_to_space(z, 2)
    want = torch.pixel_shuffle(torch.from_numpy(z), 2).numpy()
    np.testing.assert_array_equal(out, want)
    # and the inverse brings it back
    back = torch.pixel_unshuffle(torch.from_numpy(out), 2).numpy()
    np.testing.assert_array_equal(back, z)
    # explicit corner values: out[2i+dy, 2j+dx] = z[2dy+dx, i, j]
    assert out[1, 0, 3, 4] == z[1, 2 * 1 + 0, 1, 2]
    assert out[0, 0, 0, 1] == z[0, 1, 0, 0]


def test_chain_is_composition():
    spec = ((1, 3, 5, True), (3, 3, 3, True), (3, 4, 3, False))
    x, layers = synth.chain_f32(N=1, H=11, W=13, spec=spec, seed=14)
    out, m = oracle.chain(x, layers, d2s=2)
    z = x.astype(np.float64)
    mz = np.abs(z)
    for w, b, relu in layers:
        z, _ = oracle.conv2d(z, w, b, relu)
        mz, _ = oracle.conv2d(mz, np.abs(w), np.abs(b), False)
    import torch
    np.testing.assert_array_equal(out, torch.pixel_shuffle(torch.from_numpy(z), 2).numpy())
    np.testing.assert_array_equal(m, torch.pixel_shuffle(torch.from_numpy(mz), 2).numpy())
    assert out.shape == (1, 1, 22, 26)
    # the propagated scale bounds the values
    assert np.all(np.abs(out) <= m)


@pytest.mark.parametrize("win", [(0, 11, 0, 13), (0, 3, 0, 4), (4, 9, 5, 13), (10, 11, 12, 13), (2, 3, 0, 13)])
def test_chain_window_matches_full(win):
    x, layers = synth.chain_f32(N=1, H=11, W=13, seed=15)
    full, mfull = oracle.chain(x, layers, d2s=1)
    i0, i1, j0, j1 = win
    z, m = oracle.chain_window(x, layers, i0, i1, j0, j1)
    np.testing.assert_array_equal(z, full[:, :, i0:i1, j0:j1])
    np.testing.assert_allclose(m, mfull[:, :, i0:i1, j0:j1], rtol=0, atol=0)


def test_fp16_inputs_are_exact_in_oracle():
    """The fp16 layer's operands widen exactly to float64, so the oracle result for
    fp16 inputs is the exact-input result (pins the widening, not the rounding)."""
    x, w, b = synth.cnn_layer_f16_nhwc(N=1, C=4, K=3, H=5, W=6, seed=16)
    y, _ = oracle.conv2d(x, w, b, False, "NHWC")
    y2, _ = oracle.conv2d(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64), False, "NHWC")
    np.testing.assert_array_equal(y, y2)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.conv2d(np.zeros((1, 1, 4, 4)), np.zeros((1, 1, 2, 2)))   # even filter
    with pytest.raises(ValueError):
        oracle.conv2d(np.zeros((1, 2, 4, 4)), np.zeros((1, 1, 3, 3)))   # channel mismatch
    with pytest.raises(ValueError):
        oracle.conv2d_points(np.zeros((1, 1, 4, 4)), np.zeros((1, 1, 3, 3)), None, False, [[0, 0, 4, 0]])


def test_empty_image():
    y, m = oracle.conv2d(np.zeros((1, 1, 0, 5)), np.ones((1, 1, 3, 3)))
    assert y.shape == (1, 1, 0, 5) and m.shape == y.shape
