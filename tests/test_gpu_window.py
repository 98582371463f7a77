"""Sliding-window attention and ring-buffer caches on the GPU, against the oracle.

  * ck_attn_decode_gqa with a window, on contiguous, paged and ring caches,
    several sequences of unequal lengths, chunk sizes that do and do not divide
    the window: within 1e-4 x RMS of the oracle per sequence. Every token
    outside the window holds NaN (paged: pages wholly before the window are
    unmapped), so a read outside the window cannot go unnoticed.
  * One sequence over a bf16 or fp8 cache (the bf16 matrix-core kernel), for
    query groups of 1 to 8 heads, both head sizes, contiguous, paged, windowed
    and ring caches and a chunk that is not a whole number of steps: within
    1e-4 x RMS of the oracle on the same cache codes.
  * A window that covers the sequence gives the unwindowed result bit for bit;
    the two-pass entry points with the window give what the one-pass call does.
  * ck_kv_append on a ring writes slot pos % capacity and nothing else, bit for
    bit as the oracle's append.
  * The decode layer (chain and fused) over a loop of tokens that wraps the
    ring: per step, out within 2e-3 x RMS of the oracle layer, the attention
    on the GPU's own q and cache within 1e-4, the appended slot holding exactly
    the layer's k and v, every other slot unchanged.
  * A captured decode loop with device positions on a ring equals the eager
    host-position steps, output and cache byte for byte, across the wrap.
"""
import numpy as np
import pytest

import oracle
import parity
from decode_step_attention_layer_amd import synth
from gpu_helpers import assert_close_rms, cuda, host

pytestmark = pytest.mark.gpu

NAN = np.float32("nan")


def _t(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _build(layout, m, KV, hd, pos, W, R, seed):
    """Host K/V (+ page table), the oracle cache and the ck.kv_cache geometry."""
    g = np.random.default_rng(seed)
    if layout == "ring":
        k = g.standard_normal((m, KV, R, hd), dtype=np.float32)
        v = g.standard_normal((m, KV, R, hd), dtype=np.float32)
        for s, p in enumerate(pos):
            if p + 1 < R:                       # slots never written yet
                k[s, :, p + 1:] = NAN
                v[s, :, p + 1:] = NAN
        oc = oracle.Cache(k, v, KV, hd, capacity=R, ring=True, window=W)
        return k, v, None, oc, dict(capacity=R, window=W, ring=True)
    if layout == "contig":
        cap = max(pos) + 9
        k = g.standard_normal((m, KV, cap, hd), dtype=np.float32)
        v = g.standard_normal((m, KV, cap, hd), dtype=np.float32)
        for s, p in enumerate(pos):
            t0 = max(0, p + 1 - W) if W else 0
            k[s, :, p + 1:] = NAN
            v[s, :, p + 1:] = NAN
            k[s, :, :t0] = NAN                  # outside the window
            v[s, :, :t0] = NAN
        oc = oracle.Cache(k, v, KV, hd, capacity=cap, window=W)
        return k, v, None, oc, dict(capacity=cap, window=W)
    # paged: only the pages that hold window tokens are mapped
    ps = 16
    maxp = -(-(max(pos) + 1) // ps)
    firsts = [(max(0, p + 1 - W) if W else 0) // ps for p in pos]
    counts = [p // ps - f + 1 for p, f in zip(pos, firsts)]
    P = sum(counts) + 2
    perm = g.permutation(P).astype(np.int32)
    table = np.full((m, maxp), -1, np.int32)
    k = np.full((P, KV, ps, hd), NAN, np.float32)
    v = np.full((P, KV, ps, hd), NAN, np.float32)
    nxt = 0
    for s, p in enumerate(pos):
        t0 = max(0, p + 1 - W) if W else 0
        for lp in range(firsts[s], firsts[s] + counts[s]):
            table[s, lp] = perm[nxt]
            nxt += 1
        for t in range(t0, p + 1):
            pg, sl = table[s, t // ps], t % ps
            k[pg, :, sl] = g.standard_normal((KV, hd), dtype=np.float32)
            v[pg, :, sl] = g.standard_normal((KV, hd), dtype=np.float32)
    oc = oracle.Cache(k, v, KV, hd, page_size=ps, page_table=table, max_pages_per_seq=maxp,
                      num_pages=P, window=W)
    return k, v, table, oc, dict(page_size=ps, max_pages_per_seq=maxp, num_pages=P, window=W)


def _dev(ck, dev, KV, hd, k, v, table, geo):
    kd, vd = _t(k, dev), _t(v, dev)
    td = _t(table, dev) if table is not None else None
    c = ck.kv_cache(kd, vd, KV, hd, page_table=td, **geo)
    return c, (kd, vd, td)


def _attend(ck, dev, c, q, pos, m, H, KV, hd, W, chunk):
    import torch

    out = torch.empty(m * H * hd, dtype=torch.float32, device=dev)
    att = max(min(p + 1, W) if W else p + 1 for p in pos)
    nws = ck.ck_attn_workspace_size(m, H, KV, hd, att, chunk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    ck.ck_attn_decode_gqa(_t(q, dev), c, pos, out, m, H, 1.0 / np.sqrt(hd), chunk, ws, nws)
    torch.cuda.synchronize()
    return host(out).reshape(m, H * hd)


ATTN_CASES = [
    # layout, m, H, KV, hd, positions, window, ring slots, chunk
    ("contig", 1, 4, 2, 64, [16], 5, 0, 0),
    ("contig", 1, 28, 4, 128, [4096], 1024, 0, 0),
    ("contig", 1, 28, 4, 128, [4096], 1000, 0, 64),
    ("contig", 2, 16, 2, 128, [300, 40], 100, 0, 64),
    ("contig", 1, 32, 8, 128, [32768], 4096, 0, 0),
    ("paged", 3, 8, 1, 64, [89, 20, 64], 33, 0, 64),
    ("paged", 4, 32, 8, 128, [700, 1500, 255, 256], 256, 0, 0),
    ("ring", 1, 32, 8, 128, [32768], 4096, 4096, 0),
    ("ring", 2, 14, 2, 64, [5000, 37], 100, 128, 0),
    ("ring", 1, 28, 4, 128, [9000], 1000, 1024, 64),
    ("ring", 1, 4, 2, 64, [10], 1, 1, 0),
    ("ring", 1, 4, 2, 64, [3], 8, 8, 0),
]


@pytest.mark.parametrize("layout,m,H,KV,hd,pos,W,R,chunk", ATTN_CASES, ids=str)
def test_window_attention(layout, m, H, KV, hd, pos, W, R, chunk):
    dev = cuda()
    from decode_step_attention_layer_amd import ck

    print(f"window attention {layout} m={m} H={H} KV={KV} hd={hd} pos={pos} W={W} R={R}",
          flush=True)
    k, v, table, oc, geo = _build(layout, m, KV, hd, pos, W, R, 7 * H + W + m)
    c, keep = _dev(ck, dev, KV, hd, k, v, table, geo)
    q = synth.seeded_vector(W + 3, m * H * hd)
    got = _attend(ck, dev, c, q, pos, m, H, KV, hd, W, chunk)
    for s in range(m):
        ref = oracle.attention(q[s * H * hd:(s + 1) * H * hd], oc, s, pos[s] + 1, H)
        assert_close_rms(got[s], ref, 1e-4, f"{layout} window attention s={s}")


REDUCED_CASES = [
    # layout, H, KV, hd, position, window, ring slots, chunk
    ("contig", 28, 4, 128, 4096, 0, 0, 0),       # query groups of 7, 128-wide heads
    ("contig", 14, 2, 64, 1024, 0, 0, 0),        # groups of 7, 64-wide heads
    ("contig", 12, 4, 128, 1999, 0, 0, 0),       # groups of 3
    ("contig", 24, 3, 128, 776, 0, 0, 40),       # groups of 8; partial steps inside the sequence
    ("paged", 8, 8, 128, 2999, 0, 0, 0),         # paged, groups of 1
    ("paged", 16, 2, 64, 699, 0, 0, 0),          # paged 64-wide heads, groups of 8
    ("contig", 28, 4, 128, 4096, 1000, 0, 0),    # a window starting off a step
    ("paged", 32, 8, 128, 1500, 256, 0, 0),
    ("ring", 28, 4, 128, 9000, 1000, 1024, 64),  # a ring wrapping inside a step
    ("ring", 32, 8, 128, 32768, 4096, 4096, 0),
    ("ring", 4, 2, 64, 10, 1, 1, 0),
]


@pytest.mark.parametrize("layout,H,KV,hd,pos,W,R,chunk", REDUCED_CASES, ids=str)
@pytest.mark.parametrize("dtype", [synth.KV_BF16, synth.KV_FP8], ids=["bf16", "fp8"])
def test_reduced_cache_attention_one_sequence(dtype, layout, H, KV, hd, pos, W, R, chunk):
    """One sequence over a bf16 or fp8 cache (the bf16 matrix-core kernel):
    query groups of 1 to 8 heads, 64- and 128-wide heads, paged, windowed and
    ring caches, an explicit chunk that is not a whole number of steps;
    within 1e-4 x RMS of the oracle on the same cache codes."""
    dev = cuda()
    from decode_step_attention_layer_amd import ck

    print(f"reduced-cache attention dtype={dtype} {layout} H={H} KV={KV} hd={hd} pos={pos} "
          f"W={W} R={R} chunk={chunk}", flush=True)
    k, v, table, _, geo = _build(layout, 1, KV, hd, [pos], W, R, 11 * H + W)
    kc = synth.cache_codes(k, dtype, 40 + H, 0, True)
    vc = synth.cache_codes(v, dtype, 40 + H, 0, False)
    ks, vs = (synth.FP8_K_SCALE, synth.FP8_V_SCALE) if dtype == synth.KV_FP8 else (1.0, 1.0)
    if layout == "paged":
        oc = oracle.Cache(kc, vc, KV, hd, page_size=16, page_table=table,
                          max_pages_per_seq=geo["max_pages_per_seq"], num_pages=geo["num_pages"],
                          window=W, dtype=dtype, k_scale=ks, v_scale=vs)
    else:
        oc = oracle.Cache(kc, vc, KV, hd, capacity=geo["capacity"], ring=geo.get("ring", False),
                          window=W, dtype=dtype, k_scale=ks, v_scale=vs)
    kd, vd = _t(kc, dev), _t(vc, dev)
    td = _t(table, dev) if table is not None else None
    c = ck.kv_cache(kd, vd, KV, hd, page_table=td, dtype=dtype, k_scale=ks, v_scale=vs, **geo)
    q = synth.seeded_vector(W + 5, H * hd)
    got = _attend(ck, dev, c, q, [pos], 1, H, KV, hd, W, chunk)
    ref = oracle.attention(q, oc, 0, pos + 1, H)
    assert_close_rms(got[0], ref, 1e-4, f"{layout} reduced-cache attention")


def test_window_covering_the_sequence_is_unwindowed():
    dev = cuda()
    from decode_step_attention_layer_amd import ck

    m, H, KV, hd, pos = 2, 28, 4, 128, [2047, 1000]
    k, v, table, oc, geo = _build("contig", m, KV, hd, pos, 0, 0, 5)
    q = synth.seeded_vector(77, m * H * hd)
    outs = []
    for W in (0, 2048, 2049, 100000):
        c, keep = _dev(ck, dev, KV, hd, k, v, table, dict(geo, window=W))
        outs.append(_attend(ck, dev, c, q, pos, m, H, KV, hd, W, 0))
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


@pytest.mark.parametrize("layout", ["paged", "ring"])
def test_window_two_pass_entry_points_match(layout):
    import torch
    from decode_step_attention_layer_amd import ck

    dev = cuda()
    m, H, KV, hd, W = 3, 32, 8, 128, 300
    pos = [900, 150, 2000]
    k, v, table, oc, geo = _build(layout, m, KV, hd, pos, W, 512 if layout == "ring" else 0, 6)
    c, keep = _dev(ck, dev, KV, hd, k, v, table, geo)
    q = _t(synth.seeded_vector(5, m * H * hd), dev)
    # an explicit split: the two automatic ones may differ
    chunk = 64
    nws = ck.ck_attn_workspace_size(m, H, KV, hd, W, chunk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    a = torch.empty(m * H * hd, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    ck.ck_attn_decode_gqa(q, c, pos, a, m, H, 1.0 / np.sqrt(hd), chunk, ws, nws)
    ck.ck_attn_partial(q, c, pos, m, H, 1.0 / np.sqrt(hd), chunk, ws, nws)
    ck.ck_attn_merge(ws, nws, pos, m, H, KV, hd, chunk, b, window=W)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_ring_append_bitexact():
    from decode_step_attention_layer_amd import ck

    dev = cuda()
    m, KV, hd, R, W = 2, 2, 64, 128, 100
    pos = [5000, 37]
    k, v, table, oc, geo = _build("ring", m, KV, hd, pos, W, R, 8)
    c, (kd, vd, _) = _dev(ck, dev, KV, hd, k, v, table, geo)
    knew = synth.seeded_vector(11, m * KV * hd)
    vnew = synth.seeded_vector(12, m * KV * hd)
    ck.ck_kv_append(c, _t(knew, dev), _t(vnew, dev), pos, m)
    import torch

    torch.cuda.synchronize()
    for s in range(m):
        oracle.kv_append(oc, s, pos[s], knew[s * KV * hd:(s + 1) * KV * hd],
                         vnew[s * KV * hd:(s + 1) * KV * hd])
    for got, ref in ((host(kd), oc.k), (host(vd), oc.v)):
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def _ws_read(ws, off, nbytes, dtype):
    return ws[off: off + nbytes].cpu().numpy().view(dtype)


LAYER_CASES = [
    # config, window, ring, steps, variant
    ("c1", 8, True, 12, 0),
    ("c1", 8, True, 12, 1),
    ("c1", 5, False, 4, 1),
    ("c2", 256, True, 3, 1),
    ("c2", 300, False, 2, 0),
    ("c3", 1000, True, 2, 1),
    ("c3", 1000, False, 2, 1),
    ("c1", 8, True, 12, 3),        # the two-launch variant
    ("c2", 256, True, 3, 3),
    ("c3", 1000, False, 2, 3),
]


@pytest.mark.parametrize("name,W,ring,steps,variant", LAYER_CASES, ids=str)
def test_layer_decode_loop_with_window(name, W, ring, steps, variant):
    import torch
    from decode_step_attention_layer_amd import ck
    from decode_step_attention_layer_amd.workload import DeviceStack

    dev = cuda()
    cfg = synth.CONFIGS[name]
    stack = DeviceStack(cfg, dev, keep_host=True, layers=1, window=W, ring=ring)
    L = stack.layers[0]
    R = stack.capacity
    m, D, H, KV, hd = cfg.m, cfg.D, cfg.H, cfg.KV, cfg.hd
    desc = stack.desc(variant)
    max_ctx = cfg.pos + steps + 1
    ws = torch.empty(ck.ck_decode_layer_workspace_size(desc, max_ctx), dtype=torch.uint8,
                     device=dev)
    off = {n: ck.ck_decode_layer_ws_offset(desc, max_ctx, n) for n in ("q", "k", "v", "attn")}
    dims = dict(D=D, H=H, KV=KV, hd=hd, m=m, eps=cfg.eps)
    cos, sin = synth.rope_for(cfg)
    wts = dict(L.host, rope_cos=cos, rope_sin=sin)
    out = torch.empty((m, D), dtype=torch.float32, device=dev)
    g = np.random.default_rng(31)

    def ocache(k, v):
        return oracle.Cache(k, v, KV, hd, capacity=R, ring=ring, window=W)

    for i in range(steps):
        pos = [cfg.pos + i]
        print(f"{name} W={W} ring={ring} variant={variant} pos={pos[0]}", flush=True)
        x = g.standard_normal((m, D), dtype=np.float32)
        before_k, before_v = host(L.tensors["k"]).copy(), host(L.tensors["v"]).copy()
        xd = _t(x, dev)
        ck.ck_decode_layer(desc, L.weights, L.cache, xd, xd, pos, out, ws, ws.numel())
        torch.cuda.synchronize()
        got = host(out)
        ref = oracle.decode_layer(dims, wts, ocache(before_k.copy(), before_v.copy()), x, x, pos)
        tag = f"{name} W={W} ring={ring} pos={pos[0]}"
        assert_close_rms(got - x, ref - x, 2e-3, tag + " out")
        # the attention on the GPU's own q and cache
        gk, gv = host(L.tensors["k"]), host(L.tensors["v"])
        gq = _ws_read(ws, off["q"], 4 * H * hd, np.float32)
        at = _ws_read(ws, off["attn"], 4 * H * hd, np.float32)
        a0 = oracle.attention(gq, ocache(gk.copy(), gv.copy()), 0, pos[0] + 1, H)
        assert_close_rms(at, a0, 1e-4, tag + " attention")
        # exactly one slot changed: the appended one, holding the layer's k and v
        slot = pos[0] % R if ring else pos[0]
        kk = _ws_read(ws, off["k"], 4 * KV * hd, np.float32).reshape(KV, hd)
        vv = _ws_read(ws, off["v"], 4 * KV * hd, np.float32).reshape(KV, hd)
        assert np.array_equal(gk[0, :, slot].view(np.uint32), kk.view(np.uint32)), tag
        assert np.array_equal(gv[0, :, slot].view(np.uint32), vv.view(np.uint32)), tag
        mask = np.ones(gk.shape, bool)
        mask[0, :, slot] = False
        assert np.array_equal(gk[mask].view(np.uint32), before_k[mask].view(np.uint32)), tag
        assert np.array_equal(gv[mask].view(np.uint32), before_v[mask].view(np.uint32)), tag


@pytest.mark.parametrize("name,W,layers", [("c1", 8, None), ("c2", 64, 2)])
def test_graph_decode_loop_on_a_ring(name, W, layers):
    """A captured step with device positions, replayed across the ring's wrap,
    equals the eager host-position steps byte for byte; at every replayed step
    the output matches the oracle's own decode loop on ring caches of its own
    at that step's positions (within max(2e-3, 3 x the oracle's +-1-ulp noise
    floor)), and only the slots pos % W changed, holding what the oracle
    loop appended there."""
    import torch
    from decode_step_attention_layer_amd import ck
    from decode_step_attention_layer_amd.workload import DeviceStack

    dev = cuda()
    steps = W + 3 if W <= 8 else 6
    a = DeviceStack(synth.CONFIGS[name], dev, layers=layers, window=W, ring=True, keep_host=True)
    b = a.clone()
    desc = a.desc(ck.CK_VARIANT_FUSED, attn_chunk=64)
    pos0 = list(a.pos)
    max_ctx = max(pos0) + steps + 1
    ws_a = torch.empty(ck.ck_decode_step_workspace_size(desc, a.nlayers, max_ctx),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty_like(ws_a)
    pos_dev = torch.tensor(pos0, dtype=torch.int32, device=dev)
    out_b = torch.empty((a.cfg.m, a.cfg.D), dtype=torch.float32, device=dev)
    wts, cs = b.step_arrays()
    ck.ck_decode_step_devpos(desc, wts, cs, b.x0, pos_dev, max_ctx, out_b, ws_b, ws_b.numel())
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        ck.ck_decode_step_devpos(desc, wts, cs, b.x0, pos_dev, max_ctx, out_b, ws_b, ws_b.numel())
        pos_dev.add_(1)
    cfg = a.cfg
    cos, sin = synth.rope_for(cfg)

    def mk(l, k, v):
        return oracle.Cache(k, v, cfg.KV, cfg.hd, capacity=W, ring=True, window=W)

    orc = parity.OracleLoop(cfg, [L.host for L in a.layers], cos, sin, mk)
    for step in range(steps):
        print(f"{name} ring W={W} replay {step}", flush=True)
        a.pos = [p + step for p in pos0]
        ref = a.decode_step(desc, ws_a, out=torch.empty_like(out_b)).clone()
        before = [(host(L.tensors["k"]).copy(), host(L.tensors["v"]).copy()) for L in b.layers]
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_b, ref), f"{name} step {step}: replay differs from the eager step"
        tag = f"{name} ring W={W} replay {step} at {a.pos}"
        x_orc, floor = orc.step(a.x0_host, a.pos)
        bound = max(2e-3, 3.0 * floor)
        assert_close_rms(host(out_b), x_orc, bound, tag + " out")
        slot = a.pos[0] % W
        for l, (L, (kb, vb), oc) in enumerate(zip(b.layers, before, orc.caches)):
            for n_, x0_, o_ in (("k", kb, oc.k), ("v", vb, oc.v)):
                x1_ = host(L.tensors[n_])
                mask = np.zeros(x1_.shape, bool)
                mask[0, :, slot] = True
                assert np.array_equal(x0_[~mask].view(np.uint32), x1_[~mask].view(np.uint32)), \
                    tag + f" layer {l} {n_}: a slot other than pos % W changed"
                assert_close_rms(x1_[mask], o_[mask], bound, tag + f" layer {l} {n_} slot")
    for La, Lb in zip(a.layers, b.layers):
        for n in ("k", "v"):
            assert np.array_equal(host(La.tensors[n]).view(np.uint32),
                                  host(Lb.tensors[n]).view(np.uint32))
