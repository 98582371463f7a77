"""Device-resident positions (ck_decode_layer_devpos / ck_decode_step_devpos):
the graph-capturable decode loop (the spark_model page attn_v41/decode.rs,
decode_prep / decode_body: the replayed step equals the eager one).

  * With the same fixed attention chunk (64 tokens), a layer or step reading
    its positions from device memory equals the host-position call bit for
    bit (outputs and every cache byte), in the chain, fused and persistent
    variants, and that host-position step at chunk 64 matches the oracle
    chain (within max(2e-3, 3 x the oracle's own +-1-ulp noise floor)).
  * A decode loop captured once (the step, then an in-graph increment of the
    device positions) and replayed for four successive tokens equals the
    eager host-position steps at those positions, output by output and cache
    byte by cache byte; and at every replayed step the output matches the
    oracle's own decode loop (its own caches, appended at every step) at that
    step's positions, the caches changed only at the appended slots, whose
    contents match the oracle loop's; for the persistent variant the last
    layer's xq and aq bytes equal the oracle quantizer's on the GPU's fp32 and
    its attention is within 1e-4 of the oracle's on the GPU's q and cache.
"""
import numpy as np
import pytest

import oracle
import parity
from decode_step_attention_layer_amd import synth
from gpu_helpers import assert_close_rms, cuda, host

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


def _mk_cache(stack):
    cfg = stack.cfg

    def mk(l, k, v):
        L = stack.layers[l]
        if cfg.page_size:
            return oracle.Cache(k, v, cfg.KV, cfg.hd, page_size=cfg.page_size,
                                page_table=L.host["table"],
                                max_pages_per_seq=cfg.max_pages_per_seq, num_pages=k.shape[0])
        return oracle.Cache(k, v, cfg.KV, cfg.hd, capacity=cfg.capacity)
    return mk


def _oracle_loop(stack):
    cos, sin = synth.rope_for(stack.cfg)
    return parity.OracleLoop(stack.cfg, [L.host for L in stack.layers], cos, sin, _mk_cache(stack))


def _slot_mask(stack, l, pos):
    """The flat cache elements of layer l that a step at `pos` appends."""
    cfg = stack.cfg
    L = stack.layers[l]
    mask = np.zeros(L.host["k"].size, bool)
    for s in range(cfg.m):
        for g in range(cfg.KV):
            t = pos[s]
            if cfg.page_size:
                page = int(L.host["table"][s, t // cfg.page_size])
                row = ((page * cfg.KV + g) * cfg.page_size + t % cfg.page_size) * cfg.hd
            else:
                row = ((s * cfg.KV + g) * cfg.capacity + t) * cfg.hd
            mask[row:row + cfg.hd] = True
    return mask


def _caches(stack):
    return [(host(L.tensors["k"]).copy(), host(L.tensors["v"]).copy()) for L in stack.layers]


@pytest.mark.parametrize("variant", [0, 1, 2, 3], ids=["chain", "fused", "persistent", "two_launch"])
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
    # the host-position step at this chunk size, against the oracle chain
    ref, floor = _oracle_loop(a).step(a.x0_host, a.pos)
    assert_close_rms(host(out_a), ref, max(2e-3, 3.0 * floor),
                     f"{name} variant {variant} chunk {CHUNK} vs oracle")
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


@pytest.mark.parametrize("variant", [1, 2, 3], ids=["fused", "persistent", "two_launch"])
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

    orc = _oracle_loop(a)
    if variant == 2:
        from test_gpu_layer import ws_reader
        read = ws_reader(ck, desc, max_ctx, ws_b, a.cfg)
    for step in range(STEPS):
        print(f"{name} variant {variant} replay {step}", flush=True)
        a.pos = [p + step for p in pos0]
        ref = a.decode_step(desc, ws_a, out=torch.empty_like(out_b)).clone()
        before = _caches(b)
        g.replay()
        torch.cuda.synchronize()
        if variant == 2:
            assert a.step_status(desc, ws_a) == 0 and b.step_status(desc, ws_b) == 0
        assert torch.equal(out_b, ref), f"{name} step {step}: replay differs from the eager step"
        assert host(pos_dev).tolist() == [p + step + 1 for p in pos0]
        # the replay against the oracle's own loop at this step's positions
        tag = f"{name} variant {variant} replay {step} at {a.pos}"
        x_orc, floor = orc.step(a.x0_host, a.pos)
        bound = max(2e-3, 3.0 * floor)
        assert_close_rms(host(out_b), x_orc, bound, tag + " out")
        after = _caches(b)
        for l, ((kb, vb), (ka, va), oc) in enumerate(zip(before, after, orc.caches)):
            mask = _slot_mask(b, l, a.pos).reshape(kb.shape)
            for x0_, x1_, o_ in ((kb, ka, oc.k), (vb, va, oc.v)):
                assert np.array_equal(x0_[~mask].view(np.uint32), x1_[~mask].view(np.uint32)), \
                    tag + f" layer {l}: a slot other than the appended one changed"
                assert_close_rms(x1_[mask], o_[mask], bound, tag + f" layer {l} appended slot")
        if variant == 2:
            # the last layer's intermediates, on the GPU's own values
            st = read()
            Ll = b.layers[-1]
            kl, vl = after[-1]
            gc = _mk_cache(b)(len(b.layers) - 1, kl.copy(), vl.copy())
            for s_ in range(a.cfg.m):
                assert np.array_equal(st["xq"][s_], oracle.quantize_q8_0(st["xn"][s_])), tag
                a0 = oracle.attention(st["q"][s_], gc, s_, a.pos[s_] + 1, a.cfg.H)
                assert_close_rms(st["attn"][s_], a0, 1e-4, tag + " attention")
                assert np.array_equal(st["aq"][s_], oracle.quantize_q8_0(st["attn"][s_])), tag
    for (ka, va), (kb, vb) in zip(_caches(a), _caches(b)):
        assert np.array_equal(ka.view(np.uint32), kb.view(np.uint32))
        assert np.array_equal(va.view(np.uint32), vb.view(np.uint32))
