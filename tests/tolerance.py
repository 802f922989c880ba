"""Per-element tolerance check against the oracle.

A result y passes when |y - y_ref| <= tau * m for every element, where m is the
oracle's error scale sum |w*x| + |b| (propagated layer by layer for chains).
tau = 1e-5 for fp32 and 2e-3 for fp16 inputs with fp32 accumulation. NaN or
infinity in y fails.

fp16-storage chains round every layer's output to fp16. Each rounding moves a
value by at most half an fp16 ulp, 2^-11 of it, and ReLU and the next layers
carry earlier differences into m, so after L layers the oracle's chain and the
exact one differ by at most L * 2^-10 * m (pinned in the oracle's tests); the
GPU's fp32 sums may round to the other neighbour at the same L layers, so the
two stay within 2 * L * 2^-10 * m < L * TAU_F16 * m: tau = L * 2e-3.
"""
import numpy as np

TAU_F32 = 1e-5
TAU_F16 = 2e-3


def tau_f16_chain(layers):
    return layers * TAU_F16


def check(y, ref, m, tau, label=""):
    """Raise AssertionError naming the worst element; return max err / bound."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    assert y.shape == ref.shape == m.shape, (label, y.shape, ref.shape, m.shape)
    err = np.abs(y - ref)
    bound = tau * m
    bad = ~(err <= bound)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    if bad.any():
        idx = np.unravel_index(int(np.argmax(np.where(bad, ratio, -1))), y.shape)
        raise AssertionError("%s: %d of %d elements out of tolerance; worst at %s: got %r want %r "
                             "(|err| %.3g > %.3g = tau*m)" % (label, int(bad.sum()), y.size, idx, y[idx],
                                                              ref[idx], err[idx], bound[idx]))
    return worst
