"""Device-resident positions (ck_decode_layer_devpos / ck_decode_step_devpos):
the graph-capturable decode loop.

  * With the same fixed attention chunk, a layer or step reading its positions
    from device memory equals the host-position call bit for bit (outputs and
    every cache byte), in the chain, fused and persistent variants; the
    host-position calls are the ones verified against the oracle elsewhere.
  * A decode loop captured once (the step, then an in-graph increment of the
    device positions) and replayed for four successive tokens equals the
    eager host-position steps at those positions, output by output and cache
    byte by cache byte.
"""
import numpy as np
import pytest

from decode_step_attention_layer_amd import synth
from gpu_helpers import cuda, host

pytestmark = pytest.mark.gpu

CHUNK = 64
STEPS = 4


def _stack(name, layers, extra_tokens):
    import torch
    from decode_step_attention_layer_amd.workload import DeviceStack

    cfg = synth.CONFIGS[name]
    stack = DeviceStack(cfg, cuda(), keep_host=True, spare_pages=16 if cfg.page_size else 0,
                        layers=layers)
    if cfg.page_size:
        # map a spare page wherever the next tokens start a new page
        for L in stack.layers:
            table = L.host["table"]
            free = sorted(set(range(L.host["k"].shape[0])) - set(table[table >= 0].tolist()))
            for s, p in enumerate(stack.pos):
                for t in range(p, p + extra_tokens):
                    if table[s, t // cfg.page_size] < 0:
                        table[s, t // cfg.page_size] = free.pop(0)
            L.tensors["table"].copy_(torch.from_numpy(table))
    return stack


def _caches(stack):
    return [(host(L.tensors["k"]).copy(), host(L.tensors["v"]).copy()) for L in stack.layers]


@pytest.mark.parametrize("variant", [0, 1, 2], ids=["chain", "fused", "persistent"])
@pytest.mark.parametrize("name,layers", [("c1", None), ("c2", 3), ("c5", None)])
def test_devpos_step_equals_host_positions(name, layers, variant):
    import torch
    from decode_step_attention_layer_amd import ck

    a = _stack(name, layers, 1)
    b = a.clone()
    desc = a.desc(variant, attn_chunk=CHUNK)
    max_ctx = a.max_ctx + 7                      # a bound above the positions
    ws_a = a.step_workspace(desc)
    ws_b = torch.empty(ck.ck_decode_step_workspace_size(desc, b.nlayers, max_ctx),
                       dtype=torch.uint8, device=b.device)
    out_a = a.decode_step(desc, ws_a)
    pos_dev = torch.tensor(b.pos, dtype=torch.int32, device=b.device)
    out_b = torch.empty_like(out_a)
    wts, cs = b.step_arrays()
    ck.ck_decode_step_devpos(desc, wts, cs, b.x0, pos_dev, max_ctx, out_b, ws_b, ws_b.numel())
    torch.cuda.synchronize()
    if variant == 2:
        assert a.step_status(desc, ws_a) == 0 and b.step_status(desc, ws_b) == 0
    assert torch.equal(out_a, out_b), f"{name} variant {variant}: device positions differ"
    for (ka, va), (kb, vb) in zip(_caches(a), _caches(b)):
        assert np.array_equal(ka.view(np.uint32), kb.view(np.uint32))
        assert np.array_equal(va.view(np.uint32), vb.view(np.uint32))

    # the single-layer entry point too
    if variant != 2:
        L_a, L_b = a.layers[0], b.layers[0]
        wsl_a, wsl_b = a.workspace(desc), torch.empty(
            ck.ck_decode_layer_workspace_size(desc, max_ctx), dtype=torch.uint8, device=b.device)
        ya, yb = torch.empty_like(out_a), torch.empty_like(out_a)
        ck.ck_decode_layer(desc, L_a.weights, L_a.cache, a.x0, a.x0, a.pos, ya, wsl_a,
                           wsl_a.numel())
        ck.ck_decode_layer_devpos(desc, L_b.weights, L_b.cache, b.x0, b.x0, pos_dev, max_ctx, yb,
                                  wsl_b, wsl_b.numel())
        torch.cuda.synchronize()
        assert torch.equal(ya, yb)


@pytest.mark.parametrize("variant", [1, 2], ids=["fused", "persistent"])
@pytest.mark.parametrize("name,layers", [("c1", None), ("c2", 2), ("c5", None)])
def test_graph_decode_loop_with_device_positions(name, layers, variant):
    import torch
    from decode_step_attention_layer_amd import ck

    a = _stack(name, layers, STEPS)              # eager, host positions
    b = a.clone()                                # captured, device positions
    desc = a.desc(variant, attn_chunk=CHUNK)
    max_ctx = max(a.pos) + STEPS + 1
    ws_a = torch.empty(ck.ck_decode_step_workspace_size(desc, a.nlayers, max_ctx),
                       dtype=torch.uint8, device=a.device)
    ws_b = torch.empty_like(ws_a)
    pos0 = list(a.pos)
    pos_dev = torch.tensor(pos0, dtype=torch.int32, device=b.device)
    out_b = torch.empty((a.cfg.m, a.cfg.D), dtype=torch.float32, device=b.device)
    wts, cs = b.step_arrays()

    # one eager call first (it appends at the first position, as the first
    # replay will again, with the same values)
    ck.ck_decode_step_devpos(desc, wts, cs, b.x0, pos_dev, max_ctx, out_b, ws_b, ws_b.numel())
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        ck.ck_decode_step_devpos(desc, wts, cs, b.x0, pos_dev, max_ctx, out_b, ws_b, ws_b.numel())
        pos_dev.add_(1)
    # capture ran nothing: positions and caches are untouched
    assert host(pos_dev).tolist() == pos0

    for step in range(STEPS):
        a.pos = [p + step for p in pos0]
        ref = a.decode_step(desc, ws_a, out=torch.empty_like(out_b)).clone()
        g.replay()
        torch.cuda.synchronize()
        if variant == 2:
            assert a.step_status(desc, ws_a) == 0 and b.step_status(desc, ws_b) == 0
        assert torch.equal(out_b, ref), f"{name} step {step}: replay differs from the eager step"
        assert host(pos_dev).tolist() == [p + step + 1 for p in pos0]
    for (ka, va), (kb, vb) in zip(_caches(a), _caches(b)):
        assert np.array_equal(ka.view(np.uint32), kb.view(np.uint32))
        assert np.array_equal(va.view(np.uint32), vb.view(np.uint32))
