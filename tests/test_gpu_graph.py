"""HIP-graph capture of a whole decode step (the benchmark's launch mode):
every replay, with eager work and synchronizations in between, must equal
the eagerly launched step bit for bit."""
import numpy as np
import pytest

from gpu_helpers import cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,variant", [("c1", 1), ("c1", 0), ("c2", 1), ("c5", 1)])
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
