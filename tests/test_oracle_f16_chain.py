"""The oracle's fp16-storage chain against pins that fix it from outside (CPU only).

The chain follows the StreamHPC CNN page's "Reducing memory traffic" step: data
and weights stored as fp16, so every layer reads the previous layer's output
rounded to fp16 (nearest even). The pins: the depth-to-space by 3 of the pages'
9-channel output is torch's pixel shuffle; a two-layer 1x1 chain whose exact
answer differs with and without the rounding between layers; delta filters
that copy exactly representable inputs; the windowed evaluation; and the
bound the rounding keeps against the exact (unrounded) chain, which the GPU
tolerance of this chain rests on.
"""
import numpy as np
import pytest

import oracle
import synth
from tolerance import f16_chain_bound


def test_depth_to_space_by_3_is_pixel_shuffle():
    import torch
    z = np.random.default_rng(21).standard_normal((2, 9, 4, 5))
    out = oracle.depth_to_space(z, 3)
    np.testing.assert_array_equal(out, torch.pixel_shuffle(torch.from_numpy(z), 3).numpy())
    assert out[1, 0, 3 * 2 + 1, 3 * 3 + 2] == z[1, 3 * 1 + 2, 2, 3]


def test_rounding_between_layers():
    """x = w1 = 1 + 2^-10 (fp16): layer 1 gives 1 + 2^-9 + 2^-20, stored as
    1 + 2^-9; layer 2 (w = 1024, b = -1026) then gives exactly 0. Without the
    rounding it would give 1024 * 2^-20 = 2^-10."""
    e = np.float16(1.0 + 2.0 ** -10)
    x = np.full((1, 1, 1, 1), e, np.float16)
    w1 = np.full((1, 1, 1, 1), e, np.float16)
    w2 = np.full((1, 1, 1, 1), 1024.0, np.float16)
    b2 = np.array([-1026.0], np.float32)
    out, _ = oracle.chain_f16(x, [(w1, None, False), (w2, b2, False)])
    assert out.shape == (1, 1, 1, 1) and out[0, 0, 0, 0] == 0.0
    exact, _ = oracle.chain(np.transpose(x, (0, 3, 1, 2)), [(w1, None, False), (w2, b2, False)])
    assert exact[0, 0, 0, 0] == 2.0 ** -10


def test_delta_filters_copy_the_input():
    """Centre-tap one-hot filters route input channels; fp16 inputs survive
    exactly, so the output is the routed input, depth-to-space by 3."""
    import torch
    rng = np.random.default_rng(22)
    x = rng.integers(-8, 9, (1, 6, 7, 1)).astype(np.float16) / np.float16(4)
    w1 = np.zeros((9, 1, 5, 5), np.float16)
    w1[:, 0, 2, 2] = 1.0                       # nine copies of the input channel
    w2 = np.zeros((9, 9, 3, 3), np.float16)
    perm = rng.permutation(9)
    for k in range(9):
        w2[k, perm[k], 1, 1] = 1.0
    out, _ = oracle.chain_f16(x, [(w1, None, False), (w2, None, False)], d2s=3)
    z = np.repeat(np.transpose(x.astype(np.float64), (0, 3, 1, 2)), 9, axis=1)[:, perm]
    want = torch.pixel_shuffle(torch.from_numpy(z), 3).numpy()
    np.testing.assert_array_equal(out, np.transpose(want, (0, 2, 3, 1)))


@pytest.mark.parametrize("win", [(0, 9, 0, 12), (0, 2, 0, 3), (3, 8, 5, 12), (8, 9, 11, 12)])
def test_window_matches_full(win):
    spec = ((1, 4, 5, True), (4, 4, 3, True), (4, 9, 3, False))
    x, layers = synth.chain_f16_nhwc(N=1, H=9, W=12, spec=spec, seed=23)
    full, mfull = oracle.chain_f16(x, layers)
    i0, i1, j0, j1 = win
    z, m = oracle.chain_f16_window(x, layers, i0, i1, j0, j1)
    np.testing.assert_array_equal(z, full[:, i0:i1, j0:j1, :])
    np.testing.assert_array_equal(m, mfull[:, i0:i1, j0:j1, :])


def test_rounding_stays_within_the_chain_bound():
    """Against the exact chain (no rounding), the fp16-storage chain stays
    within ((1 + 2^-11)^L - 1) * m after L layers (each rounding is at most half
    an fp16 ulp, 2^-11 of the value, and ReLU and the convolutions carry earlier
    errors into m): about L * 2^-11, the oracle's share of the GPU tolerance
    (tolerance.f16_chain_bound). The slack 1e-12 m covers the fp64 sums."""
    spec = ((1, 8, 5, True), (8, 8, 3, True), (8, 4, 3, True), (4, 9, 3, False))
    x, layers = synth.chain_f16_nhwc(N=1, H=10, W=11, spec=spec, seed=24)
    got, m = oracle.chain_f16(x, layers)
    exact, mx = oracle.chain(np.transpose(x, (0, 3, 1, 2)), layers)
    exact = np.transpose(exact, (0, 2, 3, 1))
    np.testing.assert_array_equal(m, np.transpose(mx, (0, 2, 3, 1)))
    bound = f16_chain_bound(len(spec), gpu=False)
    assert abs(bound - ((1 + 2.0 ** -11) ** len(spec) - 1)) < 1e-15
    err = np.abs(got - exact)
    assert np.all(err <= (bound + 1e-12) * m)
    assert np.any(got != exact)   # the rounding is visible


def test_chain_bound_is_reached_by_a_tie():
    """The one-layer bound 2^-11 m is attained up to a factor 1 - 2^-9: x = 1 +
    2^-10, w = 1, b = 2^-11 lies halfway between the fp16 neighbours 1 + 2^-10
    and 1 + 2^-9; nearest-even rounds up, by exactly 2^-11."""
    x = np.full((1, 1, 1, 1), 1.0 + 2.0 ** -10, np.float16)
    w = np.ones((1, 1, 1, 1), np.float16)
    b = np.array([2.0 ** -11], np.float32)
    got, m = oracle.chain_f16(x, [(w, b, False)])
    assert got[0, 0, 0, 0] == 1.0 + 2.0 ** -9
    err = got[0, 0, 0, 0] - (1.0 + 2.0 ** -10 + 2.0 ** -11)
    assert err == 2.0 ** -11
    assert 1 - 2.0 ** -9 < err / (f16_chain_bound(1, gpu=False) * m[0, 0, 0, 0]) <= 1.0
