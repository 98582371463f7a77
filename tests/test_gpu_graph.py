"""HIP-graph capture of a whole decode step (the benchmark's launch mode):
every replay, with eager work and synchronizations in between, must equal
the eagerly launched step bit for bit."""
import numpy as np
import pytest

from gpu_helpers import cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,variant", [("c1", 1), ("c1", 0), ("c2", 1), ("c5", 1), ("c1", 3),
                                          ("c2", 3), ("c5", 3)])
def test_graph_replay_equals_eager(name, variant):
    import torch
    from decode_step_attention_layer_amd import synth
    from decode_step_attention_layer_amd.workload import DeviceStack

    dev = cuda()
    stack = DeviceStack(synth.CONFIGS[name], dev, layers=4 if name == "c2" else None)
    desc = stack.desc(variant)
    ws = stack.workspace(desc)
    eager = stack.step(desc, ws).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stack.step(desc, ws)
    last = stack.bufs[(stack.nlayers - 1) % 2]
    for i in range(5):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(last, eager), f"replay {i} differs"
        # eager work between replays
        again = stack.step(desc, ws)
        torch.cuda.synchronize()
        assert torch.equal(again, eager)


@pytest.mark.parametrize("name", ["c1", "c2", "c5"])
def test_graph_replay_persistent_step(name):
    """The whole-step persistent kernel (and its counter-clearing kernel)
    captured once and replayed: every replay equals the eager step."""
    import torch
    from decode_step_attention_layer_amd import ck, synth
    from decode_step_attention_layer_amd.workload import DeviceStack

    dev = cuda()
    stack = DeviceStack(synth.CONFIGS[name], dev, layers=4 if name == "c2" else None)
    desc = stack.desc(ck.CK_VARIANT_PERSISTENT)
    ws = stack.step_workspace(desc)
    eager = stack.decode_step(desc, ws).clone()
    torch.cuda.synchronize()
    assert stack.step_status(desc, ws) == 0
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stack.decode_step(desc, ws, out=out)
    for i in range(5):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert stack.step_status(desc, ws) == 0
        assert torch.equal(out, eager), f"replay {i} differs"
        again = stack.decode_step(desc, ws)
        torch.cuda.synchronize()
        assert torch.equal(again, eager)


@pytest.mark.parametrize("name", ["c1", "c3", "c5"])
@pytest.mark.parametrize("variant", [0, 1, 3], ids=["chain", "fused", "two_launch"])
def test_layer_in_two_parts_equals_the_layer(name, variant):
    """ck_decode_layer_part 1 (steps 1-6) then 2 (steps 7-8) on one workspace
    equals ck_decode_layer bit for bit: output, cache bytes and the
    intermediates the workspace keeps (the layer itself is checked against
    the oracle in test_gpu_layer.py)."""
    import torch
    from decode_step_attention_layer_amd import ck, synth
    from decode_step_attention_layer_amd.workload import DeviceStack

    dev = cuda()
    a = DeviceStack(synth.CONFIGS[name], dev, layers=1)
    b = a.clone()
    desc = a.desc(variant)
    wa, wb = a.workspace(desc), b.workspace(desc)
    ya = torch.empty((a.cfg.m, a.cfg.D), dtype=torch.float32, device=dev)
    yb = torch.empty_like(ya)
    La, Lb = a.layers[0], b.layers[0]
    ck.ck_decode_layer(desc, La.weights, La.cache, a.x0, a.x0, a.pos, ya, wa, wa.numel())
    for part in (1, 2):
        ck.ck_decode_layer_part(desc, Lb.weights, Lb.cache, b.x0, b.x0, b.pos, yb, wb,
                                wb.numel(), part)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)
    for n in ("k", "v"):
        assert torch.equal(La.tensors[n].view(torch.int32), Lb.tensors[n].view(torch.int32))
    from test_gpu_layer import ws_reader
    ra = ws_reader(ck, desc, a.max_ctx, wa, a.cfg)()
    rb = ws_reader(ck, desc, b.max_ctx, wb, b.cfg)()
    for n in ra:
        assert np.array_equal(ra[n].view(np.uint8), rb[n].view(np.uint8)), n
