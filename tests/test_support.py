"""Host tests of the test infrastructure itself: the seeded input generators are
deterministic, the tolerance check accepts and rejects what it should, and the
oracle agrees with an im2col + matrix-product formulation written here."""
import hashlib

import numpy as np
import pytest

import oracle
import synth
from tolerance import TAU_F32, check, tau_f16_chain


def _digest(*arrays):
    m = hashlib.sha256()
    for a in arrays:
        m.update(np.ascontiguousarray(a).tobytes())
    return m.hexdigest()[:16]


def test_generators_are_deterministic():
    """Seed 0 draws the same tensors in every process (digests recorded when the
    recipe was fixed; a change of the recipe must update them on purpose)."""
    x, w = synth.small_image_3x3()
    assert _digest(x, w) == "44d8cdeae322a6a8"
    x, w, b = synth.cnn_layer_f32(N=1, C=32, K=32, H=16, W=32)
    assert _digest(x, w, b) == "f0a8f2733b90ea96"
    x, w, b = synth.cnn_layer_f16_nhwc(N=1, C=64, K=64, H=8, W=8)
    assert _digest(x, w, b) == "b9cb6aab89b19150"
    x, layers = synth.chain_f16_nhwc(N=1, H=8, W=8)
    assert _digest(x, *[a for (w, b, _) in layers for a in (w, b)]) == "913b83f2383e82ee"
    a1 = synth.large_image(5, H=64, W=64, seed=3)
    a2 = synth.large_image(5, H=64, W=64, seed=3)
    assert all(np.array_equal(p, q) for p, q in zip(a1, a2))


def test_tolerance_check():
    ref = np.array([1.0, -2.0, 0.5])
    m = np.array([1.0, 2.0, 1.0])
    assert check(ref + 0.5e-5 * m, ref, m, TAU_F32) <= 0.5 + 1e-9
    with pytest.raises(AssertionError):
        check(ref + 2e-5 * m, ref, m, TAU_F32)
    with pytest.raises(AssertionError):
        check(np.array([1.0, np.nan, 0.5]), ref, m, TAU_F32)
    with pytest.raises(AssertionError):
        check(np.array([1.0, np.inf, 0.5]), ref, m, TAU_F32)
    with pytest.raises(AssertionError):
        check(ref[:2], ref, m, TAU_F32)
    # m = 0 (an all-zero window without bias): only the exact value passes
    assert check(np.zeros(2), np.zeros(2), np.zeros(2), TAU_F32) == 0.0
    with pytest.raises(AssertionError):
        check(np.array([1e-30, 0.0]), np.zeros(2), np.zeros(2), TAU_F32)
    # the derived fp16-chain tolerance: per layer twice half an fp16 ulp plus
    # the fp32 sum's bound, about 1.05e-3; four layers under the old 4 * 2e-3
    assert tau_f16_chain(1) == pytest.approx(2 * 2.0 ** -11 + 577 * 2.0 ** -23, rel=1e-3)
    assert 4 * 1.04e-3 < tau_f16_chain(4) < 4 * 1.05e-3
    assert tau_f16_chain(4) < 4 * 2e-3


def _im2col_conv(x, w, b, relu):
    """NCHW convolution as a matrix product: columns of the zero-padded input
    windows (one row per (c, u, v)) times the K x (C R S) weight matrix."""
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    P, Q = (R - 1) // 2, (S - 1) // 2
    xp = np.zeros((N, C, H + 2 * P, W + 2 * Q))
    xp[:, :, P:P + H, Q:Q + W] = x
    cols = np.empty((N, C * R * S, H * W))
    for c in range(C):
        for u in range(R):
            for v in range(S):
                cols[:, (c * R + u) * S + v, :] = xp[:, c, u:u + H, v:v + W].reshape(N, H * W)
    y = np.einsum("kr,nrp->nkp", w.reshape(K, C * R * S), cols).reshape(N, K, H, W)
    if b is not None:
        y = y + b[None, :, None, None]
    return np.maximum(y, 0.0) if relu else y


@pytest.mark.parametrize("C,K,R,S,relu", [(3, 4, 3, 3, False), (2, 5, 5, 5, True), (4, 2, 1, 7, False),
                                          (1, 3, 7, 1, True)])
def test_oracle_matches_im2col(C, K, R, S, relu):
    rng = np.random.default_rng(C * 10 + K)
    x = rng.standard_normal((2, C, 9, 11))
    w = rng.standard_normal((K, C, R, S))
    b = rng.standard_normal(K)
    y, m = oracle.conv2d(x, w, b, relu)
    want = _im2col_conv(x, w, b, relu)
    assert np.all(np.abs(y - want) <= 1e-12 * m + 1e-300)
    # the same through the NHWC entry of the oracle
    yh, mh = oracle.conv2d(np.transpose(x, (0, 2, 3, 1)), w, b, relu, "NHWC")
    np.testing.assert_allclose(np.transpose(yh, (0, 3, 1, 2)), y, rtol=0, atol=1e-12)
