"""GPU parity on a fixed list of seeded random layer shapes, across every kernel
family the plan can choose (single channel, separable, one channel with F
filters, multi-channel register-blocked, pointwise, fp32 MFMA, fp16 MFMA, fp16
first layer, fallback), each compared with the oracle element by element.

The shapes are drawn once from a fixed seed: small enough for the oracle,
ragged in every dimension, and biased towards the sizes that select the
specialised kernels (W % 4 == 0, channel counts of 32 and 64, K multiples of
the channel blocks).
"""
import numpy as np
import pytest

import image_stencil_amd as isa
import oracle
from gpu_util import dev, host, say
from tolerance import TAU_F16, TAU_F32, check

pytestmark = pytest.mark.gpu


def _draw_cases(n=80, seed=1234):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kind = rng.choice(["single", "separable", "fanout", "multi", "pointwise", "mfma32", "f16", "f16head"])
        N = int(rng.integers(1, 3))
        H = int(rng.integers(1, 70))
        W = int(rng.integers(1, 40)) * 4 if rng.random() < 0.8 else int(rng.integers(1, 160))
        relu = bool(rng.random() < 0.5)
        bias = bool(rng.random() < 0.7)
        if kind == "single":
            C, K, R = 1, 1, int(rng.choice([1, 3, 5, 7]))
            S = int(rng.choice([1, 3, 5, 7]))
        elif kind == "separable":
            C, K, R = 1, 1, int(rng.choice([3, 5, 7]))
            S = R
        elif kind == "fanout":
            C, K, R = 1, int(rng.choice([2, 4, 6, 8, 12, 16, 32])), int(rng.choice([1, 3, 5]))
            S = R
        elif kind == "multi":
            C, K, R = int(rng.integers(2, 40)), int(rng.choice([4, 8, 16, 32, 3, 5])), int(rng.choice([3, 5]))
            S = R
        elif kind == "pointwise":
            C, K, R = int(rng.integers(2, 70)), int(rng.choice([4, 8, 16, 32, 12, 7])), 1
            S = 1
        elif kind == "mfma32":
            C, K, R, S = 32, 32, 3, 3
        elif kind == "f16":
            C, K = [(64, 64), (64, 32), (32, 32), (32, 16), (8, 8), (3, 5)][int(rng.integers(0, 6))]
            R = S = 3
        else:
            C, K, R = 1, int(rng.choice([16, 32, 64])), int(rng.choice([3, 5]))
            S = R
        cases.append((i, kind, N, C, K, H, W, R, S, relu, bias))
    return cases


def _draw_multi_cases(n=24, seed=4321):
    """Multi-channel fp32 layers of any channel and filter count with 3x3, 5x5
    or 7x7 filters (the register-blocked kernel in either form, its masked last
    filter group, 1-channel slabs, the fallback for widths that are not whole
    16-byte vectors)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        N = int(rng.integers(1, 3))
        H = int(rng.integers(1, 60))
        W = int(rng.integers(1, 40)) * 4 if rng.random() < 0.85 else int(rng.integers(1, 120))
        C, K, R = int(rng.integers(1, 40)), int(rng.integers(1, 13)), int(rng.choice([3, 5, 7]))
        cases.append((100 + i, "multi_any", N, C, K, H, W, R, R, bool(rng.random() < 0.5), bool(rng.random() < 0.7)))
    return cases


CASES = _draw_cases() + _draw_multi_cases()


@pytest.mark.parametrize("i,kind,N,C,K,H,W,R,S,relu,bias", CASES, ids=[str(c[0]) for c in CASES])
def test_random_shape(i, kind, N, C, K, H, W, R, S, relu, bias):
    import torch
    rng = np.random.default_rng(1000 + i)
    f16 = kind in ("f16", "f16head")
    sep = kind == "separable"
    say("random", i, kind, N, C, K, H, W, R, S, relu, bias)
    if f16:
        x = (rng.random((N, H, W, C), dtype=np.float32) * 2 - 1).astype(np.float16)
        w = (rng.standard_normal((K, C, R, S)) * np.sqrt(2.0 / (C * R * S))).astype(np.float16)
    else:
        x = rng.random((N, C, H, W), dtype=np.float32) * 2 - 1
        w = (rng.standard_normal((K, C, R, S)) * np.sqrt(2.0 / (C * R * S))).astype(np.float32)
    b = (rng.standard_normal(K) * 0.1).astype(np.float32) if bias else None
    d = isa.make_desc(N, C, H, W, K, R, S, "f16" if f16 else "f32", relu, separable=sep)
    plan = isa.Plan(d)
    if sep:
        col = (rng.standard_normal(R) / R).astype(np.float32)
        row = (rng.standard_normal(S) / S).astype(np.float32)
        wk = np.concatenate([col, row])
        ref, m = oracle.conv2d_separable(x, col, row, b, relu)
    else:
        wk = w
        ref, m = oracle.conv2d(x, w, b, relu, "NHWC" if f16 else "NCHW")
    if f16:
        y = torch.full((N, H, W, K), float("nan"), dtype=torch.float16, device="cuda")
    else:
        y = torch.full((N, K, H, W), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(dev(x), dev(wk), dev(b) if b is not None else None, y)
    got = host(y)
    check(got, ref, m, TAU_F16 if f16 else TAU_F32,
          "random %d %s (%s)" % (i, kind, plan.info()["kernel"]))


def _draw_pipelines(n=24, seed=4321):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        L = int(rng.integers(1, 7))
        rs = [int(rng.choice([1, 3, 3, 5, 5, 7])) for _ in range(L)]
        N = int(rng.integers(1, 3))
        H = int(rng.integers(1, 90))
        W = int(rng.integers(1, 80)) * 4 if rng.random() < 0.8 else int(rng.integers(1, 300))
        out.append((i, N, H, W, tuple(rs)))
    return out


PIPES = _draw_pipelines()


@pytest.mark.parametrize("i,N,H,W,rs", PIPES, ids=[str(p[0]) for p in PIPES])
def test_random_pipeline(i, N, H, W, rs):
    """Chains of single-channel filters under the model's grouping."""
    rng = np.random.default_rng(2000 + i)
    x = rng.random((N, 1, H, W), dtype=np.float32)
    layers = []
    for r in rs:
        w = (rng.standard_normal((1, 1, r, r)) / r).astype(np.float32)
        b = (rng.standard_normal(1) * 0.1).astype(np.float32) if rng.random() < 0.6 else None
        layers.append((w, b, bool(rng.random() < 0.5)))
    d = isa.make_chain_desc(N, H, W, [(1, 1, r, relu) for r, (_, _, relu) in zip(rs, layers)], 1, isa.IS_CHAIN_AUTO)
    groups = isa.conv_chain_groups(d)
    say("pipeline", i, N, H, W, rs, groups)
    dl = [(dev(w), dev(b) if b is not None else None, relu) for (w, b, relu) in layers]
    y = host(isa.conv_chain(dev(x), dl, 1, isa.IS_CHAIN_AUTO))
    ref, m = oracle.chain(x, layers)
    check(y, ref, m, TAU_F32, "pipeline %d %s groups %s" % (i, rs, groups))
