"""Closed-form pins of the oracle's layer chains (CPU only).

The chain is the composition of layers, z_l = act_l(conv_l(z_{l-1}) + b_l),
followed by depth-to-space; its error scale is m_0 = |x|,
m_l = conv(|w_l|, m_{l-1}) + |b_l| (the upscaling network of the StreamHPC CNN
page, introduction and "Reducing memory traffic" table, with the per-layer
ReLU switch of its "Vectorization" section).

Each layer here has one nonzero tap per (output, input) channel pair, so its
result is worked out without any convolution loop: a one-tap filter at
(u, v) of an R x R filter reads the input at (i + u - R/2, j + v - R/2), zero
outside the image, times the tap; channels add; the bias adds; ReLU clips where
the flag says. Nonzero biases of both signs, ReLU on some layers and not on
others, and negative intermediate values make a dropped or misplaced bias, a
ReLU on the wrong layer, a flipped or transposed tap, a wrong channel route or
a transposed depth-to-space change the result. The fp16-storage chain adds a
rounding to fp16 (nearest even, numpy's cast) after every layer.
"""
import numpy as np
import pytest

import oracle


def _shift(img, du, dv):
    """img read at (i + du, j + dv), zero outside."""
    H, W = img.shape
    out = np.zeros_like(img)
    i0, i1 = max(0, -du), min(H, H - du)
    j0, j1 = max(0, -dv), min(W, W - dv)
    if i0 < i1 and j0 < j1:
        out[i0:i1, j0:j1] = img[i0 + du:i1 + du, j0 + dv:j1 + dv]
    return out


# A chain 1 -> 2 (5x5) -> 2 (3x3) -> 4 (3x3), depth-to-space 2. Each layer:
# (R, {(k, c): (u, v, tap)}, bias per output channel, relu).
CHAIN = [
    (5, {(0, 0): (0, 4, 1.5), (1, 0): (2, 2, -2.0)}, [-0.25, 0.5], True),
    (3, {(0, 0): (2, 1, 0.5), (0, 1): (0, 0, -1.0), (1, 1): (1, 2, 0.75)}, [0.125, -0.375], False),
    (3, {(0, 0): (1, 1, 1.0), (1, 1): (0, 2, 2.0), (2, 0): (2, 0, -0.5), (3, 1): (1, 0, 1.25),
         (3, 0): (2, 2, 0.25)}, [0.0, -0.0625, 0.3125, -0.5], True),
]


def _weights(spec, cin, dtype=np.float64):
    """Dense K,C,R,R weights and the bias of a layer spec."""
    R, taps, bias, relu = spec
    K = len(bias)
    w = np.zeros((K, cin, R, R), dtype)
    for (k, c), (u, v, t) in taps.items():
        w[k, c, u, v] = t
    return w, np.array(bias, np.float32), relu


def _closed_form(x, chain, round_f16=False):
    """z and m of the chain by shifts of whole images (x: H x W, one channel)."""
    z = [x.astype(np.float64)]
    m = [np.abs(z[0])]
    for (R, taps, bias, relu) in chain:
        P = R // 2
        K = len(bias)
        zn, mn = [], []
        for k in range(K):
            acc = np.zeros_like(z[0])
            mag = np.zeros_like(z[0])
            for (kk, c), (u, v, t) in taps.items():
                if kk != k:
                    continue
                acc = acc + t * _shift(z[c], u - P, v - P)
                mag = mag + abs(t) * _shift(m[c], u - P, v - P)
            acc = acc + np.float64(np.float32(bias[k]))
            if relu:
                acc = np.maximum(acc, 0.0)
            if round_f16:
                acc = acc.astype(np.float16).astype(np.float64)
            zn.append(acc)
            mn.append(mag + abs(np.float64(np.float32(bias[k]))))
        z, m = zn, mn
    return np.stack(z), np.stack(m)


def _d2s2(a):
    """4 x H x W -> 2H x 2W with out[2i+dy, 2j+dx] = a[2 dy + dx, i, j], written out."""
    _, H, W = a.shape
    out = np.zeros((2 * H, 2 * W))
    for dy in range(2):
        for dx in range(2):
            out[dy::2, dx::2] = a[2 * dy + dx]
    return out


def _layers(dtype=np.float64):
    out, cin = [], 1
    for spec in CHAIN:
        w, b, relu = _weights(spec, cin, dtype)
        out.append((w, b, relu))
        cin = len(spec[2])
    return out


@pytest.mark.parametrize("H,W", [(7, 9), (12, 5), (1, 1)])
def test_chain_closed_form(H, W):
    x = np.random.default_rng(H * 10 + W).uniform(-1.0, 1.0, (1, 1, H, W)).astype(np.float32)
    got, m = oracle.chain(x, _layers(), d2s=2)
    z, mz = _closed_form(x[0, 0], CHAIN)
    np.testing.assert_array_equal(got[0, 0], _d2s2(z))
    np.testing.assert_array_equal(m[0, 0], _d2s2(mz))
    # without depth-to-space the four channels come out as they are
    got4, m4 = oracle.chain(x, _layers(), d2s=1)
    np.testing.assert_array_equal(got4[0], z)
    np.testing.assert_array_equal(m4[0], mz)


def test_chain_closed_form_sees_relu_and_bias():
    """The pinned values exercise what they pin: ReLU clips somewhere on layers 1
    and 3, layer 2 leaves negative values, and every bias reaches the output."""
    x = np.random.default_rng(3).uniform(-1.0, 1.0, (1, 1, 9, 11)).astype(np.float32)
    layers = _layers()
    no_relu = [(w, b, False) for (w, b, _) in layers]
    no_bias = [(w, None, r) for (w, _, r) in layers]
    ref, _ = oracle.chain(x, layers, d2s=1)
    assert not np.array_equal(ref, oracle.chain(x, no_relu, d2s=1)[0])
    assert not np.array_equal(ref, oracle.chain(x, no_bias, d2s=1)[0])
    mid, _ = oracle.chain(x, layers[:2], d2s=1)
    assert (mid < 0).any()                     # layer 2 has no ReLU
    first, _ = oracle.chain(x, layers[:1], d2s=1)
    assert (first == 0).any() and (first > 0).any()


@pytest.mark.parametrize("H,W", [(6, 8), (11, 3)])
def test_chain_f16_closed_form(H, W):
    """fp16 storage: fp16 input and taps, fp32 biases, every layer's output
    rounded to fp16; taps of 1/3 and 5/7 (rounded to fp16) make the rounding
    visible. NHWC in and out."""
    rng = np.random.default_rng(H + W)
    x = rng.uniform(-1.0, 1.0, (1, H, W, 1)).astype(np.float16)
    chain = [(R, {kc: (u, v, float(np.float16(t * f))) for kc, (u, v, t) in taps.items()}, bias, relu)
             for (R, taps, bias, relu), f in zip(CHAIN, (1.0 / 3.0, 5.0 / 7.0, 1.0))]
    layers, cin = [], 1
    for spec in chain:
        w, b, relu = _weights(spec, cin, np.float16)
        layers.append((w, b, relu))
        cin = len(spec[2])
    got, m = oracle.chain_f16(x, layers, d2s=2)
    z, mz = _closed_form(x[0, :, :, 0].astype(np.float64), chain, round_f16=True)
    np.testing.assert_array_equal(got[0, :, :, 0], _d2s2(z))
    np.testing.assert_array_equal(m[0, :, :, 0], _d2s2(mz))
    zx, _ = _closed_form(x[0, :, :, 0].astype(np.float64), chain, round_f16=False)
    assert not np.array_equal(z, zx)          # the rounding between layers shows
