"""Per-element tolerance check against the oracle.

A result y passes when |y - y_ref| <= tau * m for every element, where m is the
oracle's error scale sum |w*x| + |b| (propagated layer by layer for chains).
tau = 1e-5 for fp32 and 2e-3 for fp16 inputs with fp32 accumulation. NaN or
infinity in y fails.

fp16-storage chains round every layer's output to fp16. The bound of such a
chain is derived layer by layer (f16_chain_bound): with e_l the distance of a
chain's layer-l values from the exact chain's (no rounding), |exact| <= m and
conv(|w_l|, m_{l-1}) <= m_l,
  * the oracle rounds the fp64 value once per layer, by at most 2^-11 of it, so
    e_l <= (1 + 2^-11) conv(|w_l|, e_{l-1}) + 2^-11 m_l;
  * the GPU first sums n = C R S + 1 terms in fp32 (error at most
    gamma_n = n u / (1 - n u) of the sum of their magnitudes, u = 2^-23 so that a
    directed rounding in the matrix core's adder is covered too), then rounds to
    fp16: e_l <= (1 + gamma_n)(1 + 2^-11) conv(|w_l|, e_{l-1})
    + (2^-11 + gamma_n (1 + 2^-11)) m_l;
and the two distances add. The rounding bound 2^-11 |v| holds in fp16's normal
range (|v| >= 2^-14) and for 0, which is where these chains' values lie.
"""
import numpy as np

TAU_F32 = 1e-5
TAU_F16 = 2e-3

# Terms of the longest fp16 chain sum: a 64-channel 3x3 layer plus its bias.
F16_CHAIN_TERMS = 64 * 9 + 1


def f16_chain_bound(layers, terms=F16_CHAIN_TERMS, gpu=True):
    """Relative bound (in units of m) on |chain - exact chain| after `layers`
    fp16-storage layers: the oracle's alone (gpu=False) or the oracle's plus the
    GPU's (gpu=True), by the recurrences above."""
    half = 2.0 ** -11
    u = 2.0 ** -23
    gamma = terms * u / (1.0 - terms * u)
    a_oracle = a_gpu = 0.0
    for _ in range(layers):
        a_oracle = a_oracle * (1.0 + half) + half
        a_gpu = a_gpu * (1.0 + gamma) * (1.0 + half) + half + gamma * (1.0 + half)
    return a_oracle + a_gpu if gpu else a_oracle


def tau_f16_chain(layers):
    """Tolerance of an fp16-storage chain of `layers` layers against the oracle
    (about layers * 1.04e-3)."""
    return f16_chain_bound(layers)


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
    record(label, worst, y.size)
    return worst


# max err / bound of every passing check of the session, printed in pytest's
# terminal summary (tests/conftest.py) so that the ratios are visible without -s.
RATIOS = []


def record(label, ratio, count):
    if label:
        RATIOS.append((label, float(ratio), int(count)))
