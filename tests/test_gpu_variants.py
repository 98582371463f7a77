"""The reduced-precision caches combined with the sliding window, the ring
buffer and the sparse selection, on the GPU, against the oracle: one fused
decode layer of the 7B-shaped, long-context and batched paged workloads.

Per case, as in the other layer tests: out within 2e-3 x RMS of the oracle
layer on the same input and cache bytes; the attention on the GPU's own q and
cache within 1e-4 x RMS; the appended slot holding exactly the oracle's codes
of the GPU's own k and v; every other cache byte unchanged. The query groups
of 7 and 4 cover both row layouts of the fp8 attention (16 and 8 lanes a row).
"""
import numpy as np
import pytest

import oracle
from decode_step_attention_layer_amd import synth
from gpu_helpers import assert_close_rms, cuda, host

pytestmark = pytest.mark.gpu

BF16, FP8 = synth.KV_BF16, synth.KV_FP8
CASES = [
    # workload, cache type, window, ring, topk
    ("c3", BF16, 1000, False, 0),
    ("c3", FP8, 1024, True, 0),
    ("c3", FP8, 0, False, 600),
    ("c4", FP8, 4096, True, 0),
    ("c4", BF16, 0, False, 2048),
    ("c4", FP8, 3000, False, 0),
    ("c5", FP8, 0, False, 2048),
    ("c5", BF16, 1500, False, 0),
]


def _id(c):
    name, dt, w, ring, k = c
    return f"{name}-{'bf16' if dt == BF16 else 'fp8'}-" + (f"top{k}" if k else
                                                            f"w{w}" + ("ring" if ring else ""))


def _slot_offsets(cfg, stack, L, s, g, t):
    """Element offset of (sequence, KV head, token) in the layer's cache."""
    hd, KV = cfg.hd, cfg.KV
    if cfg.page_size:
        page = int(L.host["table"][s, t // cfg.page_size])
        return ((page * KV + g) * cfg.page_size + t % cfg.page_size) * hd
    slot = t % stack.capacity if stack.ring else t
    return ((s * KV + g) * stack.capacity + slot) * hd


@pytest.mark.parametrize("name,dtype,window,ring,topk", CASES, ids=[_id(c) for c in CASES])
def test_reduced_cache_with_window_ring_or_selection(name, dtype, window, ring, topk):
    import torch
    from decode_step_attention_layer_amd import ck
    from decode_step_attention_layer_amd.workload import DeviceStack

    dev = cuda()
    cfg = synth.CONFIGS[name]
    print(f"{_id((name, dtype, window, ring, topk))}", flush=True)
    stack = DeviceStack(cfg, dev, keep_host=True, layers=1, kv_dtype=dtype, window=window,
                        ring=ring, topk=topk, spare_pages=2 if cfg.page_size else 0)
    L = stack.layers[0]
    m, D, H, KV, hd = cfg.m, cfg.D, cfg.H, cfg.KV, cfg.hd
    desc = stack.desc(ck.CK_VARIANT_FUSED)
    ws = stack.workspace(desc)
    n_ws = max(stack.max_ctx, topk)
    off = {n: ck.ck_decode_layer_ws_offset(desc, n_ws, n) for n in ("q", "k", "v", "attn")}
    kb, vb = host(L.tensors["k"]).copy(), host(L.tensors["v"]).copy()
    out = host(stack.step(desc, ws)).copy()
    torch.cuda.synchronize()

    kvd = dict(dtype=dtype, k_scale=stack.k_scale, v_scale=stack.v_scale, window=window,
               ring=ring)
    geo = (dict(page_size=cfg.page_size, page_table=L.host["table"],
                max_pages_per_seq=cfg.max_pages_per_seq, num_pages=kb.shape[0])
           if cfg.page_size else dict(capacity=stack.capacity))
    cos, sin = synth.rope_for(cfg)
    dims = dict(D=D, H=H, KV=KV, hd=hd, m=m, eps=cfg.eps)
    wts = dict(L.host, rope_cos=cos, rope_sin=sin)
    sel = L.host.get("sel")
    sink = L.host.get("sink")
    x = stack.x0_host
    ref = oracle.decode_layer(dims, wts, oracle.Cache(kb.copy(), vb.copy(), KV, hd, **kvd, **geo),
                              x, x, stack.pos, sel=sel, sink=sink)
    for s in range(m):
        assert_close_rms(out[s] - x[s], ref[s] - x[s], 2e-3, f"seq {s} out")

    gk, gv = host(L.tensors["k"]), host(L.tensors["v"])
    gc = oracle.Cache(gk.copy(), gv.copy(), KV, hd, **kvd, **geo)
    rd = lambda n, c: ws[off[n]: off[n] + 4 * c].cpu().numpy().view(np.float32)
    gq = rd("q", m * H * hd).reshape(m, H * hd)
    at = rd("attn", m * H * hd).reshape(m, H * hd)
    kk = rd("k", m * KV * hd).reshape(m, KV * hd)
    vv = rd("v", m * KV * hd).reshape(m, KV * hd)
    changed = np.zeros(gk.size, bool)
    for s in range(m):
        p = stack.pos[s]
        if topk:
            a0 = oracle.attention_sparse(gq[s], gc, s, p + 1, H, sel[s], sink)
        else:
            a0 = oracle.attention(gq[s], gc, s, p + 1, H)
        assert_close_rms(at[s], a0, 1e-4, f"seq {s} attention")
        ek = oracle.encode_cache(kk[s], dtype, stack.k_scale).reshape(KV, hd)
        ev = oracle.encode_cache(vv[s], dtype, stack.v_scale).reshape(KV, hd)
        for g in range(KV):
            o = _slot_offsets(cfg, stack, L, s, g, p)
            assert np.array_equal(gk.reshape(-1)[o:o + hd], ek[g]), f"seq {s} head {g} k codes"
            assert np.array_equal(gv.reshape(-1)[o:o + hd], ev[g]), f"seq {s} head {g} v codes"
            changed[o:o + hd] = True
    assert np.array_equal(gk.reshape(-1)[~changed], kb.reshape(-1)[~changed])
    assert np.array_equal(gv.reshape(-1)[~changed], vb.reshape(-1)[~changed])
