"""conv_chain_forward_noalloc (the library's own workspace) against
conv_chain_forward (the caller's workspace), through the C ABI.

Both run the same kernels on the same inputs, so the results must agree bit
for bit; each is also checked against the oracle. Two calls in a row per
chain, the second on a smaller input, so that the second call reuses the
workspace the first one left behind. A chain larger than the workspace is
refused before any GPU call.
"""
import numpy as np
import pytest

import image_stencil_amd as isa
from image_stencil_amd import _abi
import oracle
import synth
from gpu_util import dev, host, say
from tolerance import TAU_F32, check, tau_f16_chain

pytestmark = pytest.mark.gpu


def _spec(layers):
    return [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]


def _both(d, x, layers, out_shape, dtype):
    """(y from conv_chain_forward with its workspace, y from the no-alloc entry)."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    xd = dev(x)
    wl = [(dev(w), dev(b) if b is not None else None) for (w, b, _) in layers]
    wp = [w.data_ptr() for (w, _) in wl]
    bp = [b.data_ptr() if b is not None else None for (_, b) in wl]
    tdt = torch.float16 if dtype == "f16" else torch.float32
    ws_bytes = isa.conv_chain_workspace_size(d)
    assert 0 < ws_bytes <= _abi.IS_NOALLOC_MAX_WORKSPACE
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y_ws = torch.full(out_shape, float("nan"), dtype=tdt, device="cuda")
    isa.conv_chain_forward(d, xd.data_ptr(), wp, bp, y_ws.data_ptr(), ws.data_ptr(), ws_bytes, stream)
    y_na = torch.full(out_shape, float("nan"), dtype=tdt, device="cuda")
    isa.conv_chain_forward_noalloc(d, xd.data_ptr(), wp, bp, y_na.data_ptr(), stream)
    return host(y_ws), host(y_na)


@pytest.mark.parametrize("sizes", [[(1, 70, 200), (1, 23, 60)]])
def test_noalloc_fp32_chain_matches_workspace_entry(sizes):
    """The fp32 upscaling chain (layer by layer, depth-to-space x2)."""
    for (N, H, W) in sizes:
        x, layers = synth.chain_f32(N=N, H=H, W=W, seed=H + W)
        d = isa.make_chain_desc(N, H, W, _spec(layers), 2, isa.IS_CHAIN_AUTO)
        assert isa.conv_chain_kernel_name(d) == "layer_by_layer"
        say("noalloc fp32 chain", N, H, W)
        y_ws, y_na = _both(d, x, layers, (N, 1, 2 * H, 2 * W), "f32")
        np.testing.assert_array_equal(y_na, y_ws)
        ref, m = oracle.chain(x, layers, d2s=2)
        check(y_na, ref, m, TAU_F32, "noalloc fp32 chain %dx%dx%d" % (N, H, W))


def test_noalloc_fp16_net_matches_workspace_entry():
    """The pages' net in fp16 storage (depth-to-space x3)."""
    for (N, H, W) in [(1, 66, 130), (1, 19, 40)]:
        x, layers = synth.chain_f16_nhwc(N=N, H=H, W=W, seed=N + H + W)
        d = isa.make_chain_desc(N, H, W, _spec(layers), 3, isa.IS_CHAIN_AUTO, "f16")
        say("noalloc fp16 net", N, H, W)
        y_ws, y_na = _both(d, x, layers, (N, 3 * H, 3 * W, 1), "f16")
        np.testing.assert_array_equal(y_na.view(np.uint16), y_ws.view(np.uint16))
        ref, m = oracle.chain_f16(x, layers, d2s=3)
        check(y_na, ref, m, tau_f16_chain(len(layers)), "noalloc fp16 net %dx%dx%d" % (N, H, W))


def test_noalloc_stencil_pipeline_matches_workspace_entry():
    """Four single-channel filters, one launch each (three intermediate images
    in the workspace, ping-pong)."""
    for (H, W) in [(300, 520), (40, 64)]:
        rng = np.random.default_rng(H)
        x = rng.random((1, 1, H, W), dtype=np.float32)
        layers = [((rng.standard_normal((1, 1, r, r)) / r).astype(np.float32),
                   (0.01 * rng.standard_normal(1)).astype(np.float32), relu)
                  for r, relu in ((3, True), (5, False), (3, True), (7, False))]
        d = isa.make_chain_desc(1, H, W, _spec(layers), 1, isa.IS_CHAIN_UNFUSED)
        say("noalloc stencil pipeline", H, W)
        y_ws, y_na = _both(d, x, layers, (1, 1, H, W), "f32")
        np.testing.assert_array_equal(y_na, y_ws)
        ref, m = oracle.chain(x, layers)
        check(y_na, ref, m, TAU_F32, "noalloc stencil pipeline %dx%d" % (H, W))


def test_noalloc_refuses_chains_beyond_its_workspace():
    """2 x 32 fp32 channels of 1440 x 1280 need 2 x 225 MiB: refused with
    IS_ERR_WORKSPACE before anything is launched (no pointer is touched)."""
    spec = [(1, 32, 5, True), (32, 32, 3, True), (32, 4, 3, False)]
    d = isa.make_chain_desc(1, 1440, 1280, spec, 2, isa.IS_CHAIN_AUTO)
    assert isa.conv_chain_workspace_size(d) > _abi.IS_NOALLOC_MAX_WORKSPACE
    with pytest.raises(isa.ImgStencilError) as e:
        isa.conv_chain_forward_noalloc(d, 0x1000, [0x2000] * 3, [None] * 3, 0x100000, None)
    assert e.value.status == _abi.IS_ERR_WORKSPACE
    ok = isa.make_chain_desc(1, 720, 1280, spec, 2, isa.IS_CHAIN_AUTO)
    assert isa.conv_chain_workspace_size(ok) <= _abi.IS_NOALLOC_MAX_WORKSPACE
