"""Sparse attention over -1-padded selections with a sink, on the GPU, against
the oracle.

  * ck_attn_sparse on contiguous, paged and ring caches, one to four
    sequences, selections with duplicates and -1 padding, with and without a
    sink: within 1e-4 x RMS of the oracle per sequence; also with selections
    split into 65-128 chunks (the three- and four-wavefront merges) and more
    (the workgroup merge), with and without a sink;
  * with a fixed split, padding a selection with -1 (even whole chunks of it)
    changes nothing, bit for bit, and the selection of every token in order
    without a sink is the dense attention (bit for bit where both run the
    vector kernel, within fp32 rounding against the matrix-core kernel);
  * an entry past its sequence makes that sequence's outputs NaN and leaves
    the others' alone; an all -1 selection gives zeros, with or without a sink;
  * ck_decode_layer_sparse (chain and fused) over a decode loop: out within
    2e-3 x RMS of the oracle layer, the attention on the GPU's own q and cache
    within 1e-4;
  * a captured sparse decode step with device positions and a device
    selection rewritten between replays equals the eager host-position steps,
    output and cache byte for byte.
"""
import numpy as np
import pytest

import oracle
from decode_step_attention_layer_amd import synth
from gpu_helpers import assert_close_rms, cuda, host

pytestmark = pytest.mark.gpu


def _t(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _build(layout, m, KV, hd, pos, R, seed):
    """Host K/V (+ table), the oracle cache and the ck.kv_cache geometry. Every
    token a sequence holds is N(0,1); the rest is NaN."""
    g = np.random.default_rng(seed)
    nan = np.float32("nan")
    if layout == "ring":
        k = g.standard_normal((m, KV, R, hd), dtype=np.float32)
        v = g.standard_normal((m, KV, R, hd), dtype=np.float32)
        oc = oracle.Cache(k, v, KV, hd, capacity=R, ring=True, window=R)
        return k, v, None, oc, dict(capacity=R, window=R, ring=True)
    if layout == "contig":
        cap = max(pos) + 9
        k = g.standard_normal((m, KV, cap, hd), dtype=np.float32)
        v = g.standard_normal((m, KV, cap, hd), dtype=np.float32)
        for s, p in enumerate(pos):
            k[s, :, p + 1:] = nan
            v[s, :, p + 1:] = nan
        oc = oracle.Cache(k, v, KV, hd, capacity=cap)
        return k, v, None, oc, dict(capacity=cap)
    ps = 16
    maxp = -(-(max(pos) + 1) // ps)
    counts = [p // ps + 1 for p in pos]
    P = sum(counts) + 2
    perm = g.permutation(P).astype(np.int32)
    table = np.full((m, maxp), -1, np.int32)
    k = np.full((P, KV, ps, hd), nan, np.float32)
    v = np.full((P, KV, ps, hd), nan, np.float32)
    nxt = 0
    for s, p in enumerate(pos):
        for lp in range(counts[s]):
            table[s, lp] = perm[nxt]
            nxt += 1
        for t in range(p + 1):
            k[table[s, t // ps], :, t % ps] = g.standard_normal((KV, hd), dtype=np.float32)
            v[table[s, t // ps], :, t % ps] = g.standard_normal((KV, hd), dtype=np.float32)
    oc = oracle.Cache(k, v, KV, hd, page_size=ps, page_table=table, max_pages_per_seq=maxp,
                      num_pages=P)
    return k, v, table, oc, dict(page_size=ps, max_pages_per_seq=maxp, num_pages=P)


def _dev(ck, dev, KV, hd, k, v, table, geo):
    kd, vd = _t(k, dev), _t(v, dev)
    td = _t(table, dev) if table is not None else None
    return ck.kv_cache(kd, vd, KV, hd, page_table=td, **geo), (kd, vd, td)


def _selection(g, pos, topk, held_from=0):
    """Per sequence: the last 16 tokens, random earlier ones (some twice),
    then -1 up to topk."""
    rows = []
    for p in pos:
        lo = 0 if held_from == 0 else max(0, p + 1 - held_from)
        win = list(range(max(lo, p - 15), p + 1))
        n = min(topk - len(win) - 3, max(0, p - 16 - lo))
        rest = list(g.choice(np.arange(lo, max(lo + 1, p - 15)), size=max(0, n), replace=False))
        if rest:
            rest += rest[:2]                       # duplicates
        sel = (win + rest)[:topk]
        rows.append(sel + [-1] * (topk - len(sel)))
    return np.array(rows, np.int32)


def _sparse(ck, dev, c, q, pos, sel, sink, m, H, KV, hd, chunk=0):
    import torch

    topk = sel.shape[1]
    out = torch.empty(m * H * hd, dtype=torch.float32, device=dev)
    nws = ck.ck_attn_workspace_size(m, H, KV, hd, topk, chunk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    sd = _t(sel, dev)
    skd = _t(sink, dev) if sink is not None else None
    ck.ck_attn_sparse(_t(q, dev), c, pos, sd, topk, skd, out, m, H, 1.0 / np.sqrt(hd), chunk, ws,
                      nws)
    torch.cuda.synchronize()
    return host(out).reshape(m, H * hd)


CASES = [
    # layout, m, H, KV, hd, positions, topk, ring slots, sink
    ("contig", 1, 4, 2, 64, [40], 24, 0, True),
    ("contig", 1, 28, 4, 128, [4096], 2048, 0, True),
    ("contig", 2, 32, 8, 128, [900, 100], 300, 0, False),
    ("paged", 3, 8, 1, 64, [89, 20, 64], 40, 0, True),
    ("paged", 4, 32, 8, 128, [700, 1500, 255, 256], 512, 0, True),
    ("ring", 1, 14, 2, 64, [5000], 100, 128, True),
    ("ring", 2, 16, 2, 128, [9000, 300], 700, 1024, False),
]


@pytest.mark.parametrize("layout,m,H,KV,hd,pos,topk,R,with_sink", CASES, ids=str)
def test_sparse_attention(layout, m, H, KV, hd, pos, topk, R, with_sink):
    from decode_step_attention_layer_amd import ck

    dev = cuda()
    print(f"sparse {layout} m={m} H={H} KV={KV} hd={hd} pos={pos} topk={topk}", flush=True)
    k, v, table, oc, geo = _build(layout, m, KV, hd, pos, R, topk + H)
    c, keep = _dev(ck, dev, KV, hd, k, v, table, geo)
    g = np.random.default_rng(topk)
    sel = _selection(g, pos, topk, held_from=R if layout == "ring" else 0)
    q = synth.seeded_vector(topk + 1, m * H * hd)
    sink = (g.standard_normal(H) * 2).astype(np.float32) if with_sink else None
    got = _sparse(ck, dev, c, q, pos, sel, sink, m, H, KV, hd)
    for s in range(m):
        ref = oracle.attention_sparse(q[s * H * hd:(s + 1) * H * hd], oc, s, pos[s] + 1, H, sel[s],
                                      sink)
        assert_close_rms(got[s], ref, 1e-4, f"{layout} sparse s={s}")


MANY_CHUNK_CASES = [
    # layout, m, H, KV, hd, positions, topk, chunk, sink: more than 128
    # chunks per sequence (the workgroup merge), past its first 16 preloaded
    # slots per thread (16 x 8 chunks for 128-wide heads, 16 x 16 for
    # 64-wide); 65-128 chunks (three and four merge wavefronts)
    ("contig", 1, 28, 4, 128, [9000], 8000, 48, True),
    ("contig", 1, 8, 2, 64, [20000], 18000, 64, True),
    ("paged", 2, 32, 8, 128, [5000, 3000], 4500, 64, False),
    ("contig", 1, 28, 4, 128, [9000], 4000, 48, True),     # 84 chunks
    ("contig", 1, 8, 2, 64, [20000], 8000, 64, True),      # 125 chunks
]


@pytest.mark.parametrize("layout,m,H,KV,hd,pos,topk,chunk,with_sink", MANY_CHUNK_CASES, ids=str)
def test_sparse_attention_many_chunks(layout, m, H, KV, hd, pos, topk, chunk, with_sink):
    """Selections split into many chunks: the three- and four-wavefront
    merges and the workgroup merge, with and without a sink, against the
    oracle within 1e-4."""
    from decode_step_attention_layer_amd import ck

    dev = cuda()
    print(f"sparse many chunks {layout} m={m} H={H} hd={hd} topk={topk} chunk={chunk}", flush=True)
    k, v, table, oc, geo = _build(layout, m, KV, hd, pos, 0, topk + chunk)
    c, keep = _dev(ck, dev, KV, hd, k, v, table, geo)
    g = np.random.default_rng(topk + 7)
    sel = _selection(g, pos, topk)
    q = synth.seeded_vector(topk + 3, m * H * hd)
    sink = (g.standard_normal(H) * 2).astype(np.float32) if with_sink else None
    got = _sparse(ck, dev, c, q, pos, sel, sink, m, H, KV, hd, chunk=chunk)
    for s in range(m):
        ref = oracle.attention_sparse(q[s * H * hd:(s + 1) * H * hd], oc, s, pos[s] + 1, H, sel[s],
                                      sink)
        assert_close_rms(got[s], ref, 1e-4, f"{layout} sparse many chunks s={s}")


def test_padding_is_inert_and_full_selection_is_dense():
    import torch
    from decode_step_attention_layer_amd import ck

    dev = cuda()
    m, H, KV, hd, pos = 2, 28, 4, 128, [1500, 700]
    k, v, table, oc, geo = _build("contig", m, KV, hd, pos, 0, 3)
    c, keep = _dev(ck, dev, KV, hd, k, v, table, geo)
    g = np.random.default_rng(4)
    q = synth.seeded_vector(8, m * H * hd)
    sink = g.standard_normal(H).astype(np.float32)
    sel = _selection(g, pos, 100)
    padded = np.concatenate([sel, np.full((m, 300), -1, np.int32)], axis=1)
    a = _sparse(ck, dev, c, q, pos, sel, sink, m, H, KV, hd, chunk=64)
    b = _sparse(ck, dev, c, q, pos, padded, sink, m, H, KV, hd, chunk=64)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # every token in order, no sink: the dense attention with the same split.
    # Groups of 4 heads run the same vector kernel both ways (bit-identical);
    # the dense attention of 7-head groups runs on the matrix cores, whose
    # sums take another order (equal within fp32 rounding)
    full = np.full((m, 1501), -1, np.int32)
    for s, p in enumerate(pos):
        full[s, :p + 1] = np.arange(p + 1)
    for Hs in (16, H):
        qs = q[:m * Hs * hd] if Hs == H else synth.seeded_vector(9, m * Hs * hd)
        sp = _sparse(ck, dev, c, qs, pos, full, None, m, Hs, KV, hd, chunk=192)
        out = torch.empty(m * Hs * hd, dtype=torch.float32, device=dev)
        nws = ck.ck_attn_workspace_size(m, Hs, KV, hd, 1501, 192)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        ck.ck_attn_decode_gqa(_t(qs, dev), c, pos, out, m, Hs, 1.0 / np.sqrt(hd), 192, ws, nws)
        torch.cuda.synchronize()
        dense = host(out).reshape(m, -1)
        if Hs // KV <= 4:
            assert np.array_equal(sp.view(np.uint32), dense.view(np.uint32))
        else:
            for s in range(m):
                assert_close_rms(sp[s], dense[s], 1e-5, f"full selection vs dense s={s}")


def test_bad_entries_and_empty_selections():
    from decode_step_attention_layer_amd import ck

    dev = cuda()
    m, H, KV, hd, pos = 3, 8, 2, 64, [50, 60, 70]
    k, v, table, oc, geo = _build("contig", m, KV, hd, pos, 0, 5)
    c, keep = _dev(ck, dev, KV, hd, k, v, table, geo)
    q = synth.seeded_vector(9, m * H * hd)
    sink = np.linspace(-1, 1, H).astype(np.float32)
    sel = np.array([[3, 50, -1, 7], [61, 2, -1, -1], [-1, -1, -1, -1]], np.int32)   # 61 > pos 60
    got = _sparse(ck, dev, c, q, pos, sel, sink, m, H, KV, hd)
    assert np.all(np.isnan(got[1]))
    ref0 = oracle.attention_sparse(q[:H * hd], oc, 0, 51, H, sel[0], sink)
    assert_close_rms(got[0], ref0, 1e-4, "sequence 0 beside a bad one")
    assert np.all(got[2] == 0.0)
    empty = _sparse(ck, dev, c, q, pos, np.full((m, 5), -1, np.int32), None, m, H, KV, hd)
    assert np.all(empty == 0.0)


LAYER_CASES = [("c1", 12, 0, 4), ("c1", 12, 1, 4), ("c2", 96, 1, 2), ("c3", 600, 1, 2)]


@pytest.mark.parametrize("name,topk,variant,steps", LAYER_CASES, ids=str)
def test_sparse_decode_layer(name, topk, variant, steps):
    import torch
    from decode_step_attention_layer_amd import ck
    from decode_step_attention_layer_amd.workload import DeviceStack

    dev = cuda()
    cfg = synth.CONFIGS[name]
    stack = DeviceStack(cfg, dev, keep_host=True, layers=1)
    L = stack.layers[0]
    m, D, H, KV, hd = cfg.m, cfg.D, cfg.H, cfg.KV, cfg.hd
    desc = stack.desc(variant)
    max_ctx = max(cfg.pos + steps + 1, topk)
    ws = torch.empty(ck.ck_decode_layer_workspace_size(desc, max_ctx), dtype=torch.uint8,
                     device=dev)
    off = {n: ck.ck_decode_layer_ws_offset(desc, max_ctx, n) for n in ("q", "attn")}
    dims = dict(D=D, H=H, KV=KV, hd=hd, m=m, eps=cfg.eps)
    cos, sin = synth.rope_for(cfg)
    wts = dict(L.host, rope_cos=cos, rope_sin=sin)
    out = torch.empty((m, D), dtype=torch.float32, device=dev)
    g = np.random.default_rng(41)
    sink = (g.standard_normal(H)).astype(np.float32)
    skd = _t(sink, dev)
    for i in range(steps):
        p = cfg.pos + i
        print(f"{name} sparse layer variant={variant} pos={p}", flush=True)
        sel = _selection(g, [p], topk)
        x = g.standard_normal((m, D), dtype=np.float32)
        bk, bv = host(L.tensors["k"]).copy(), host(L.tensors["v"]).copy()
        xd = _t(x, dev)
        ck.ck_decode_layer_sparse(desc, L.weights, L.cache, xd, xd, _t(sel, dev), topk, skd, out,
                                  ws, ws.numel(), pos=[p])
        torch.cuda.synchronize()
        oc = oracle.Cache(bk, bv, KV, hd, capacity=cfg.capacity)
        ref = oracle.decode_layer(dims, wts, oc, x, x, [p], sel=sel, sink=sink)
        tag = f"{name} sparse pos={p}"
        assert_close_rms(host(out) - x, ref - x, 2e-3, tag + " out")
        gq = ws[off["q"]: off["q"] + 4 * H * hd].cpu().numpy().view(np.float32)
        at = ws[off["attn"]: off["attn"] + 4 * H * hd].cpu().numpy().view(np.float32)
        gc = oracle.Cache(host(L.tensors["k"]).copy(), host(L.tensors["v"]).copy(), KV, hd,
                          capacity=cfg.capacity)
        assert_close_rms(at, oracle.attention_sparse(gq, gc, 0, p + 1, H, sel[0], sink), 1e-4,
                         tag + " attention")


def test_graph_sparse_decode_loop():
    """The captured step reads its position and selection from device memory,
    rewritten between replays; it equals the eager host-position steps, and at
    every replayed step the output matches the oracle's sparse layer on a cache
    of its own (appended at every step) within 2e-3, and only the appended slot
    changed, holding what the oracle appended there."""
    import torch
    from decode_step_attention_layer_amd import ck
    from decode_step_attention_layer_amd.workload import DeviceStack

    dev = cuda()
    cfg = synth.CONFIGS["c2"]
    a = DeviceStack(cfg, dev, layers=1, keep_host=True)
    b = a.clone()
    desc = a.desc(ck.CK_VARIANT_FUSED, attn_chunk=64)
    topk, steps = 80, 4
    max_ctx = cfg.pos + steps + 1
    ws_a = torch.empty(ck.ck_decode_layer_workspace_size(desc, max_ctx), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty_like(ws_a)
    g = np.random.default_rng(5)
    sels = [_selection(g, [cfg.pos + i], topk) for i in range(steps)]
    sink_h = g.standard_normal(cfg.H).astype(np.float32)
    sink = _t(sink_h, dev)
    sel_dev = _t(sels[0], dev)
    pos_dev = torch.tensor([cfg.pos], dtype=torch.int32, device=dev)
    La, Lb = a.layers[0], b.layers[0]
    out_b = torch.empty((1, cfg.D), dtype=torch.float32, device=dev)

    def step_b():
        ck.ck_decode_layer_sparse(desc, Lb.weights, Lb.cache, b.x0, b.x0, sel_dev, topk, sink,
                                  out_b, ws_b, ws_b.numel(), pos_dev=pos_dev, max_ctx=max_ctx)

    step_b()                                     # eager first call (same as the first replay)
    gr = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(gr):
        step_b()
    cos, sin = synth.rope_for(cfg)
    wts = dict(La.host, rope_cos=cos, rope_sin=sin)
    dims = dict(D=cfg.D, H=cfg.H, KV=cfg.KV, hd=cfg.hd, m=cfg.m, eps=cfg.eps)
    oc = oracle.Cache(La.host["k"].copy(), La.host["v"].copy(), cfg.KV, cfg.hd,
                      capacity=cfg.capacity)
    for i in range(steps):
        print(f"sparse graph replay {i}", flush=True)
        kb, vb = host(Lb.tensors["k"]).copy(), host(Lb.tensors["v"]).copy()
        p = cfg.pos + i
        ref = torch.empty_like(out_b)
        ck.ck_decode_layer_sparse(desc, La.weights, La.cache, a.x0, a.x0, _t(sels[i], dev), topk,
                                  sink, ref, ws_a, ws_a.numel(), pos=[p])
        sel_dev.copy_(_t(sels[i], dev))
        pos_dev.fill_(p)
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_b, ref), f"replay {i} differs from the eager step"
        tag = f"sparse graph replay {i} at {p}"
        x_orc = oracle.decode_layer(dims, wts, oc, a.x0_host, a.x0_host, [p], sel=sels[i],
                                    sink=sink_h)
        assert_close_rms(host(out_b), x_orc, 2e-3, tag + " out")
        for n_, x0_, o_ in (("k", kb, oc.k), ("v", vb, oc.v)):
            x1_ = host(Lb.tensors[n_])
            mask = np.zeros(x1_.shape, bool)
            mask[0, :, p] = True
            assert np.array_equal(x0_[~mask].view(np.uint32), x1_[~mask].view(np.uint32)), \
                tag + f" {n_}: a slot other than the appended one changed"
            assert_close_rms(x1_[mask], o_[mask], 2e-3, tag + f" {n_} appended slot")
    for n in ("k", "v"):
        assert np.array_equal(host(La.tensors[n]).view(np.uint32),
                              host(Lb.tensors[n]).view(np.uint32))
