"""The forward path inside HIP graphs, and one plan used on two streams at once.

The library only enqueues kernel launches on the caller's stream (no device
allocation, no synchronisation, no memset), so a forward captured in a graph
replays the same work. Each graph test replays several times, with eager
launches and synchronisations between the replays, and checks every replay
against the eager result bit for bit (same kernels, same inputs, same order of
operations). The stream test runs one plan on two default-priority streams
concurrently and compares each with its eager result.
"""
import numpy as np
import pytest

import image_stencil_amd as isa
import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _check_replays(launch, out, replays=3):
    """Run `launch` eagerly, capture it, replay it `replays` times with a fill
    of `out` and a synchronisation before each, and compare."""
    import torch
    launch()
    torch.cuda.synchronize()
    want = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    for i in range(replays):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), "replay %d differs from the eager result" % i


def _plan_case(x, w, b, relu, dtype):
    import torch
    if dtype == "f32":
        N, C, H, W = x.shape
        out = torch.empty((N, w.shape[0], H, W), dtype=torch.float32, device="cuda")
    else:
        N, H, W, C = x.shape
        out = torch.empty((N, H, W, w.shape[0]), dtype=torch.float16, device="cuda")
    plan = isa.Plan(isa.make_desc(N, C, H, W, w.shape[0], w.shape[2], w.shape[3], dtype, relu))
    xd, wd = dev(x), dev(w)
    bd = dev(b) if b is not None else None
    return plan, xd, wd, bd, out


@pytest.mark.parametrize("case", ["single", "fp32_layer", "fp16_layer"])
def test_forward_in_a_graph(case):
    if case == "single":
        x, w = synth.single_channel(1024, 1024, 5, seed=3)
        args = _plan_case(x, w, None, False, "f32")
        kernel = "is_k1_single"
    elif case == "fp32_layer":
        x, w, b = synth.cnn_layer_f32(H=100, W=200, seed=4)
        args = _plan_case(x, w, b, True, "f32")
        kernel = "is_k5_mfma_f32"
    else:
        x, w, b = synth.cnn_layer_f16_nhwc(N=2, H=130, W=96, seed=5)
        args = _plan_case(x, w, b, False, "f16")
        kernel = "is_k4_mfma"
    plan, xd, wd, bd, out = args
    assert plan.info()["kernel"] == kernel
    say("graph", case)
    _check_replays(lambda: plan.forward(xd, wd, bd, out), out)


def test_chain_in_a_graph():
    """The layer-by-layer upscaling chain with a caller-owned workspace."""
    import torch
    x, layers = synth.chain_f32(N=1, H=72, W=128, seed=6)
    spec = [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]
    d = isa.make_chain_desc(1, 72, 128, spec, 2, isa.IS_CHAIN_AUTO)
    assert isa.conv_chain_kernel_name(d) == "layer_by_layer"
    ws_bytes = isa.conv_chain_workspace_size(d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    xd = dev(x)
    wl = [(dev(w), dev(b)) for (w, b, _) in layers]
    y = torch.empty((1, 1, 144, 256), dtype=torch.float32, device="cuda")

    def launch():
        isa.conv_chain_forward(d, xd.data_ptr(), [w.data_ptr() for (w, _) in wl],
                               [b.data_ptr() for (_, b) in wl], y.data_ptr(), ws.data_ptr(), ws_bytes,
                               torch.cuda.current_stream().cuda_stream)

    say("graph chain")
    _check_replays(launch, y)


def _chain_graph_case(x, layers, d, out_shape, out_dtype):
    import torch
    ws_bytes = isa.conv_chain_workspace_size(d)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    xd = dev(x)
    wl = [(dev(w), dev(b) if b is not None else None) for (w, b, _) in layers]
    y = torch.empty(out_shape, dtype=out_dtype, device="cuda")

    def launch():
        isa.conv_chain_forward(d, xd.data_ptr(), [w.data_ptr() for (w, _) in wl],
                               [b.data_ptr() if b is not None else None for (_, b) in wl], y.data_ptr(),
                               ws.data_ptr() if ws_bytes else None, ws_bytes,
                               torch.cuda.current_stream().cuda_stream)

    return launch, y


def test_fp16_net_in_a_graph():
    """The pages' net in fp16 storage (first-layer kernel, three MFMA layers,
    depth-to-space in the last one's stores)."""
    import torch
    x, layers = synth.chain_f16_nhwc(N=1, H=48, W=96, seed=10)
    spec = [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]
    d = isa.make_chain_desc(1, 48, 96, spec, 3, isa.IS_CHAIN_AUTO, "f16")
    launch, y = _chain_graph_case(x, layers, d, (1, 144, 288, 1), torch.float16)
    say("graph fp16 net")
    _check_replays(launch, y)


def test_stencil_pipeline_in_a_graph():
    """A stencil pipeline in two launch groups (fused 3+3 layers)."""
    import torch
    rng = np.random.default_rng(11)
    x = rng.random((1, 1, 200, 512), dtype=np.float32)
    layers = [((rng.standard_normal((1, 1, 3, 3)) / 3).astype(np.float32), np.zeros(1, np.float32), True)
              for _ in range(6)]
    d = isa.make_chain_desc(1, 200, 512, [(1, 1, 3, True)] * 6, 1, isa.IS_CHAIN_AUTO)
    assert len(isa.conv_chain_groups(d)) >= 2
    launch, y = _chain_graph_case(x, layers, d, (1, 1, 200, 512), torch.float32)
    say("graph stencil pipeline", isa.conv_chain_groups(d))
    _check_replays(launch, y)


def test_one_plan_on_two_streams():
    import torch
    xs = [synth.cnn_layer_f32(H=160, W=320, seed=s)[0] for s in (7, 8)]
    _, w, b = synth.cnn_layer_f32(H=160, W=320, seed=9)
    plan = isa.Plan(isa.make_desc(1, 32, 160, 320, 32, 3, 3, "f32", True))
    assert plan.info()["kernel"] == "is_k5_mfma_f32"
    wd, bd = dev(w), dev(b)
    xd = [dev(x) for x in xs]
    want = []
    for i in range(2):
        y = torch.empty((1, 32, 160, 320), device="cuda")
        plan.forward(xd[i], wd, bd, y)
        want.append(y)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [torch.full((1, 32, 160, 320), float("nan"), device="cuda") for _ in range(2)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    say("two streams")
    for rep in range(4):
        for i in range(2):
            plan.forward(xd[i], wd, bd, got[i], stream=streams[i].cuda_stream)
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.equal(got[i], want[i]), "stream %d" % i
