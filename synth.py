"""Seeded synthetic inputs for the convolution workloads.

This module only draws random numbers: it holds none of the convolution's
arithmetic, so both the oracle side and the HIP side of every test and of the
benchmark take their inputs from here.

Recipe (one fresh numpy.random.default_rng(seed) per case, PCG64):
  * draw order: input x first, then for each layer its weights w, then its bias b;
  * uniform[0,1) is rng.random(dtype=float32); uniform[-1,1) is 2*u-1 in float32
    (exact: every value is a multiple of 2**-23);
  * normal(0, s) is rng.standard_normal(dtype=float32) * float32(s): the second
    parameter is the standard deviation;
  * fp16 tensors are the round-to-nearest-even cast of the fp32 draw;
  * weights are K,C,R,S; inputs are N,C,H,W except the fp16 layer, which is N,H,W,C.

Workloads (full sizes; every function also takes smaller sizes for tests):
  single-channel 3x3 on a 256x256 image:  x U[0,1), w N(0,1), no bias
  single-channel 8192x8192, R in {3,5,7}: x U[0,1), w N(0, 1/(R*R)), no bias
  fp32 CNN layer 32->32, 3x3, 720x1280:   x U[-1,1), w N(0, sqrt(2/(C*9))), b N(0,0.01), ReLU
  fp32 upscaling chain at 720x1280:       x U[0,1); 1->32 (5x5), 32->32, 32->32, 32->4 (3x3);
                                          He-normal w N(0, sqrt(2/(C*R*S))), b N(0,0.01);
                                          ReLU on layers 1-3; depth-to-space x2 -> 1440x2560
  fp16 NHWC layer 8x64->64, 3x3, 256x256: x U[-1,1) fp16, w N(0, sqrt(2/(64*9))) fp16,
                                          b fp32 N(0,0.01), no ReLU, fp16 output
"""
import numpy as np

F32 = np.float32


def _uniform01(rng, shape):
    return rng.random(shape, dtype=F32)


def _uniform_pm1(rng, shape):
    return rng.random(shape, dtype=F32) * F32(2.0) - F32(1.0)


def _normal(rng, shape, std):
    return rng.standard_normal(shape, dtype=F32) * F32(std)


def single_channel(H=256, W=256, R=3, N=1, seed=0, std=None):
    """Single-channel filtering: x (N,1,H,W) U[0,1); one RxR filter w (1,1,R,R).

    The filter's standard deviation defaults to 1/(R*R); the 256x256 3x3 case
    passes std=1.0 because its filter is drawn from normal(0,1).
    """
    rng = np.random.default_rng(seed)
    x = _uniform01(rng, (N, 1, H, W))
    s = (1.0 / (R * R)) if std is None else std
    w = _normal(rng, (1, 1, R, R), s)
    return x, w


def small_image_3x3(seed=0):
    """256x256 image, one 3x3 filter of normal(0,1) values, no bias."""
    return single_channel(256, 256, 3, 1, seed, std=1.0)


def large_image(R, H=8192, W=8192, seed=0):
    """8192x8192 image, one RxR filter of normal(0, 1/(R*R)) values, no bias."""
    return single_channel(H, W, R, 1, seed)


def cnn_layer_f32(N=1, C=32, K=32, H=720, W=1280, R=3, seed=0):
    """fp32 NCHW layer: x U[-1,1), He-normal weights, bias normal(0,0.01)."""
    rng = np.random.default_rng(seed)
    x = _uniform_pm1(rng, (N, C, H, W))
    w = _normal(rng, (K, C, R, R), np.sqrt(2.0 / (C * R * R)))
    b = _normal(rng, (K,), 0.01)
    return x, w, b


UPSCALE_CHAIN = ((1, 32, 5, True), (32, 32, 3, True), (32, 32, 3, True), (32, 4, 3, False))


def chain_f32(N=1, H=720, W=1280, spec=UPSCALE_CHAIN, seed=0):
    """Chain input x (N,1,H,W) U[0,1) and layers [(w, b, relu), ...]."""
    rng = np.random.default_rng(seed)
    x = _uniform01(rng, (N, spec[0][0], H, W))
    layers = []
    for (c, k, r, relu) in spec:
        w = _normal(rng, (k, c, r, r), np.sqrt(2.0 / (c * r * r)))
        b = _normal(rng, (k,), 0.01)
        layers.append((w, b, relu))
    return x, layers


def cnn_layer_f16_nhwc(N=8, C=64, K=64, H=256, W=256, R=3, seed=0):
    """fp16 NHWC layer: x (N,H,W,C) fp16 U[-1,1), w (K,C,R,R) fp16 He-normal, b fp32."""
    rng = np.random.default_rng(seed)
    x = _uniform_pm1(rng, (N, H, W, C)).astype(np.float16)
    w = _normal(rng, (K, C, R, R), np.sqrt(2.0 / (C * R * R))).astype(np.float16)
    b = _normal(rng, (K,), 0.01)
    return x, w, b


# The pages' upscaling network (StreamHPC CNN page, "Reducing memory traffic"
# table): 1 -> 64 (5x5), 64 -> 64, 64 -> 32, 32 -> 9 (3x3); ReLU after the
# first three layers.
PAGES_NET = ((1, 64, 5, True), (64, 64, 3, True), (64, 32, 3, True), (32, 9, 3, False))


def chain_f16_nhwc(N=1, H=720, W=1280, spec=PAGES_NET, seed=0):
    """fp16-storage chain: x (N,H,W,C0) fp16 U[0,1) and layers [(w, b, relu)]
    with w (K,C,R,R) fp16 He-normal and b fp32 normal(0, 0.01)."""
    rng = np.random.default_rng(seed)
    x = _uniform01(rng, (N, H, W, spec[0][0])).astype(np.float16)
    layers = []
    for (c, k, r, relu) in spec:
        w = _normal(rng, (k, c, r, r), np.sqrt(2.0 / (c * r * r))).astype(np.float16)
        b = _normal(rng, (k,), 0.01)
        layers.append((w, b, relu))
    return x, layers
