"""Pins for the oracle: checks against facts that the mathematics fixes.

Each pin takes the convolution under test as a callable
    conv(x, w, b, relu, layout) -> (y, m)      (float64 results)
so that the same pins run against the real oracle and, in the mutant tests,
against deliberately broken builds of it (each mutant must fail some pin).

The expected values here never come from the oracle itself: they come from
shifted copies of the input (delta filters), closed-form partial sums (constant
images), the filter's reflection (impulse responses), an independent pair of 1D
passes (separable filters), or library routines (scipy.signal.correlate2d,
torch.nn.functional.conv2d in float64, numpy einsum for 1x1 filters).
"""
import numpy as np

TIGHT = 1e-12   # relative to the error scale m, for float64 reorderings


def _rng(seed):
    return np.random.default_rng(seed)


def shift_zero(x, di, dj):
    """out[..., i, j] = x[..., i+di, j+dj], zero where i+di or j+dj is outside."""
    H, W = x.shape[-2:]
    out = np.zeros_like(x)
    i0, i1 = max(0, -di), min(H, H - di)
    j0, j1 = max(0, -dj), min(W, W - dj)
    if i0 < i1 and j0 < j1:
        out[..., i0:i1, j0:j1] = x[..., i0 + di:i1 + di, j0 + dj:j1 + dj]
    return out


def pin_delta_shift(conv, sizes=(1, 3, 5, 7), H=9, W=11):
    """A one-hot filter at (u0, v0) copies the input shifted by (u0-R/2, v0-S/2),
    zero outside the image: fixes orientation (no flip), centring and padding.
    Bit-exact, since every product is by 1.0 or 0.0."""
    x = _rng(1).random((2, 1, H, W)) - 0.5
    for R in sizes:
        for S in sizes:
            p, q = (R - 1) // 2, (S - 1) // 2
            for u0 in range(R):
                for v0 in range(S):
                    w = np.zeros((1, 1, R, S))
                    w[0, 0, u0, v0] = 1.0
                    y, m = conv(x, w, None, False, "NCHW")
                    want = shift_zero(x, u0 - p, v0 - q)
                    np.testing.assert_array_equal(y, want, err_msg="delta R=%d S=%d at (%d,%d)" % (R, S, u0, v0))
                    np.testing.assert_array_equal(m, np.abs(want))


def pin_constant_image(conv, sizes=(1, 3, 5, 7), H=10, W=13, c=0.75):
    """Constant image c: each output is c times the sum of the filter taps that
    land inside the image (the whole filter in the interior), plus the bias."""
    rng = _rng(2)
    for R in sizes:
        w = rng.standard_normal((2, 1, R, R))
        b = rng.standard_normal(2)
        x = np.full((1, 1, H, W), c)
        y, _ = conv(x, w, b, False, "NCHW")
        p = (R - 1) // 2
        for k in range(2):
            for i in range(H):
                u_lo, u_hi = max(0, p - i), min(R, H - i + p)
                for j in range(W):
                    v_lo, v_hi = max(0, p - j), min(R, W - j + p)
                    want = c * w[k, 0, u_lo:u_hi, v_lo:v_hi].sum() + b[k]
                    assert abs(y[0, k, i, j] - want) <= 1e-14 * (abs(c) * np.abs(w[k]).sum() + abs(b[k])), \
                        "constant image R=%d at (%d,%d)" % (R, i, j)


def pin_linearity(conv):
    """conv(a*x1 + b*x2) = a*conv(x1) + b*conv(x2), and likewise in the weights."""
    rng = _rng(3)
    x1, x2 = rng.standard_normal((2, 3, 7, 9)), rng.standard_normal((2, 3, 7, 9))
    w1, w2 = rng.standard_normal((4, 3, 3, 5)), rng.standard_normal((4, 3, 3, 5))
    a, bb = 0.37, -1.9
    y1, m1 = conv(x1, w1, None, False, "NCHW")
    y2, m2 = conv(x2, w1, None, False, "NCHW")
    y12, _ = conv(a * x1 + bb * x2, w1, None, False, "NCHW")
    scale = abs(a) * m1 + abs(bb) * m2
    assert np.all(np.abs(y12 - (a * y1 + bb * y2)) <= TIGHT * scale + 1e-300)
    z1, n1 = conv(x1, w1, None, False, "NCHW")
    z2, n2 = conv(x1, w2, None, False, "NCHW")
    z12, _ = conv(x1, a * w1 + bb * w2, None, False, "NCHW")
    assert np.all(np.abs(z12 - (a * z1 + bb * z2)) <= TIGHT * (abs(a) * n1 + abs(bb) * n2) + 1e-300)


def _corr1d_rows(x, v):
    """Horizontal 1D cross-correlation with zero padding, centred: independent loop."""
    q = (len(v) - 1) // 2
    out = np.zeros_like(x)
    for t in range(len(v)):
        out += v[t] * shift_zero(x, 0, t - q)
    return out


def _corr1d_cols(x, u):
    p = (len(u) - 1) // 2
    out = np.zeros_like(x)
    for t in range(len(u)):
        out += u[t] * shift_zero(x, t - p, 0)
    return out


def pin_separable(conv, sizes=((3, 3), (5, 5), (7, 7), (3, 7), (1, 5))):
    """A rank-one filter u (x) v equals a vertical 1D pass with u after a
    horizontal 1D pass with v (zero padding in each)."""
    rng = _rng(4)
    x = rng.standard_normal((1, 1, 12, 15))
    for R, S in sizes:
        u, v = rng.standard_normal(R), rng.standard_normal(S)
        w = np.outer(u, v)[None, None]
        y, m = conv(x, w, None, False, "NCHW")
        want = _corr1d_cols(_corr1d_rows(x, v), u)
        assert np.all(np.abs(y - want) <= TIGHT * m + 1e-300), "separable %dx%d" % (R, S)


def pin_impulses_8x8(conv, sizes=(1, 3, 5, 7)):
    """Brute force on 8x8: the response to a unit impulse at (a, b) is the
    filter reflected about its centre, y[a+di, b+dj] = w[p-di, p-dj], clipped to
    the image (exact). The 64 impulse responses, laid out as the columns of a
    64x64 operator built here from w alone, then reproduce conv of random inputs
    (multi-channel: a block operator over channels)."""
    H = W = 8
    rng = _rng(5)
    for R in sizes:
        p = (R - 1) // 2
        C, K = 2, 3
        w = rng.standard_normal((K, C, R, R))
        # Operator from the closed form only.
        A = np.zeros((K * H * W, C * H * W))
        for k in range(K):
            for c in range(C):
                for a in range(H):
                    for bcol in range(W):
                        col = (c * H + a) * W + bcol
                        for di in range(-p, p + 1):
                            for dj in range(-p, p + 1):
                                i, j = a + di, bcol + dj
                                if 0 <= i < H and 0 <= j < W:
                                    A[(k * H + i) * W + j, col] = w[k, c, p - di, p - dj]
        for c in range(C):
            for a in range(H):
                for bcol in range(W):
                    x = np.zeros((1, C, H, W))
                    x[0, c, a, bcol] = 1.0
                    y, _ = conv(x, w, None, False, "NCHW")
                    col = (c * H + a) * W + bcol
                    np.testing.assert_array_equal(y.reshape(-1), A[:, col],
                                                  err_msg="impulse R=%d at c=%d (%d,%d)" % (R, c, a, bcol))
        xs = rng.standard_normal((3, C, H, W))
        y, m = conv(xs, w, None, False, "NCHW")
        for n in range(3):
            want = A @ xs[n].reshape(-1)
            assert np.all(np.abs(y[n].reshape(-1) - want) <= TIGHT * m[n].reshape(-1) + 1e-300)


def pin_scipy_single_channel(conv, sizes=(1, 3, 5, 7)):
    """Single channel, odd filter: scipy.signal.correlate2d(mode='same') with a
    zero-filled boundary is the same operation; its error scale is the same
    correlation of |x| with |w|."""
    from scipy.signal import correlate2d
    rng = _rng(6)
    for R in sizes:
        for (H, W) in ((1, 1), (2, 9), (17, 6), (16, 16)):
            x = rng.standard_normal((1, 1, H, W))
            w = rng.standard_normal((1, 1, R, R))
            y, m = conv(x, w, None, False, "NCHW")
            want = correlate2d(x[0, 0], w[0, 0], mode="same", boundary="fill", fillvalue=0)
            mwant = correlate2d(np.abs(x[0, 0]), np.abs(w[0, 0]), mode="same", boundary="fill", fillvalue=0)
            assert np.all(np.abs(y[0, 0] - want) <= TIGHT * m[0, 0] + 1e-300), "scipy R=%d %dx%d" % (R, H, W)
            assert np.all(np.abs(m[0, 0] - mwant) <= TIGHT * mwant + 1e-300)


def pin_torch_multichannel(conv):
    """Multi-channel with bias and ReLU: torch.nn.functional.conv2d in float64 on
    the CPU with padding R//2, then ReLU; NHWC is the same after a transpose."""
    import torch
    rng = _rng(7)
    for (N, C, K, H, W, R, S) in ((1, 3, 4, 6, 7, 3, 3), (2, 5, 2, 9, 4, 5, 3), (1, 8, 8, 5, 5, 1, 1),
                                  (1, 4, 6, 11, 10, 7, 5)):
        x = rng.standard_normal((N, C, H, W))
        w = rng.standard_normal((K, C, R, S))
        b = rng.standard_normal(K)
        for relu in (False, True):
            y, m = conv(x, w, b, relu, "NCHW")
            t = torch.nn.functional.conv2d(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b),
                                           padding=((R - 1) // 2, (S - 1) // 2))
            if relu:
                t = torch.relu(t)
            assert np.all(np.abs(y - t.numpy()) <= TIGHT * m + 1e-300)
            yh, mh = conv(np.ascontiguousarray(x.transpose(0, 2, 3, 1)), w, b, relu, "NHWC")
            assert np.all(np.abs(yh - y.transpose(0, 2, 3, 1)) <= TIGHT * mh + 1e-300)


def pin_pointwise_1x1(conv):
    """A 1x1 filter is a per-pixel matrix product over channels plus bias."""
    rng = _rng(8)
    x = rng.standard_normal((2, 6, 5, 4))
    w = rng.standard_normal((3, 6, 1, 1))
    b = rng.standard_normal(3)
    y, m = conv(x, w, b, False, "NCHW")
    want = np.einsum("kc,nchw->nkhw", w[:, :, 0, 0], x) + b[None, :, None, None]
    assert np.all(np.abs(y - want) <= TIGHT * m + 1e-300)


def pin_channel_sum_bias_relu(conv):
    """Multi-channel = sum over channels of single-channel results; the bias is
    added once after the sum; ReLU is max(0, .) of the biased sum."""
    rng = _rng(9)
    x = rng.standard_normal((1, 4, 8, 9))
    w = rng.standard_normal((2, 4, 3, 5))
    b = rng.standard_normal(2)
    y, m = conv(x, w, None, False, "NCHW")
    parts = sum(conv(x[:, c:c + 1], w[:, c:c + 1], None, False, "NCHW")[0] for c in range(4))
    assert np.all(np.abs(y - parts) <= TIGHT * m + 1e-300)
    yb, mb = conv(x, w, b, False, "NCHW")
    assert np.all(np.abs(yb - (y + b[None, :, None, None])) <= TIGHT * mb + 1e-300)
    np.testing.assert_array_equal(mb, m + np.abs(b)[None, :, None, None])
    yr, _ = conv(x, w, b, True, "NCHW")
    np.testing.assert_array_equal(yr, np.maximum(yb, 0.0))


ALL_PINS = (pin_delta_shift, pin_constant_image, pin_linearity, pin_separable, pin_impulses_8x8,
            pin_scipy_single_channel, pin_torch_multichannel, pin_pointwise_1x1, pin_channel_sum_bias_relu)
