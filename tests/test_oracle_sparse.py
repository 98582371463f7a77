"""Pins of the oracle's sparse attention over a selection with a sink (the
spark_model page's sparse_attn; selections padded with -1 per its
decode_fixed_topk).

* brute force: numpy float64 softmax with the sink in the denominator over the
  selected rows (duplicates counted, -1 skipped), with planted mistakes (sink
  dropped, sink added to the numerator too, -1 read as token 0, the scale
  left out) that must fall outside the tolerance;
* closed forms: a single entry with a sink gives V * e^s / (e^s + e^sink); a
  sink of -inf is no sink; a huge sink drives the output to zero; an empty
  selection gives zero;
* the selection of every token, in any order, without a sink, is the dense
  attention; padding with -1 anywhere changes nothing, bit for bit;
* entries past the sequence, evicted from a ring, or on unmapped pages are
  errors;
* the layer with a selection of every token equals the dense layer.
"""
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle as orc_mod
from decode_step_attention_layer_amd import synth


def _cache(g, KV, cap, hd):
    k = g.standard_normal((1, KV, cap, hd)).astype(np.float32)
    v = g.standard_normal((1, KV, cap, hd)).astype(np.float32)
    return k, v


def _brute(q, k, v, sel, sink, H, KV, hd, plant=None):
    out = np.zeros((H, hd))
    present = [t for t in sel if t >= 0] if plant != "pad_as_zero" else [max(t, 0) for t in sel]
    for h in range(H):
        g = h * KV // H
        K = k[0, g, present].astype(np.float64)
        V = v[0, g, present].astype(np.float64)
        sc = K @ q[h * hd:(h + 1) * hd].astype(np.float64)
        if plant != "no_scale":
            sc = sc / np.sqrt(hd)
        logits = list(sc)
        if sink is not None and plant not in ("no_sink",):
            logits.append(float(sink[h]))
        lse = logsumexp(logits) if logits else -np.inf
        w = np.exp(sc - lse) if len(sc) else sc
        if plant == "sink_in_numerator" and sink is not None:
            w = w * (1.0 + np.exp(sink[h] - lse))
        out[h] = w @ V if len(sc) else 0.0
    return out.reshape(-1)


CASES = [
    # L, topk entries description, sink?
    (40, "random", True),
    (40, "random", False),
    (300, "window+random", True),
    (17, "dups", True),
]


def _selection(kind, L, g):
    if kind == "random":
        sel = g.choice(L, size=12, replace=False).astype(np.int32)
        return np.concatenate([sel, [-1, -1, -1]]).astype(np.int32)
    if kind == "window+random":
        win = np.arange(L - 64, L, dtype=np.int32)
        rest = g.choice(L - 64, size=50, replace=False).astype(np.int32)
        return np.concatenate([win, rest, np.full(14, -1, np.int32)])
    # duplicates and padding in the middle
    return np.array([3, 3, -1, 16, 0, 3, -1, 9], np.int32)


@pytest.mark.parametrize("L,kind,with_sink", CASES, ids=str)
def test_sparse_matches_brute_force(L, kind, with_sink):
    g = np.random.default_rng(L + len(kind))
    KV, H, hd = 2, 6, 32
    k, v = _cache(g, KV, L + 4, hd)
    q = (g.standard_normal(H * hd) * 2).astype(np.float32)
    sel = _selection(kind, L, g)
    sink = (g.standard_normal(H) * 2).astype(np.float32) if with_sink else None
    c = orc_mod.Cache(k, v, KV, hd, capacity=L + 4)
    got = orc_mod.attention_sparse(q, c, 0, L, H, sel, sink)
    want = _brute(q, k, v, sel, sink, H, KV, hd)
    tol = 1e-6 * np.sqrt(np.mean(want ** 2))
    assert np.max(np.abs(got - want)) <= tol
    plants = ["pad_as_zero", "no_scale"] + (["no_sink", "sink_in_numerator"] if with_sink else [])
    for plant in plants:
        bad = _brute(q, k, v, sel, sink, H, KV, hd, plant)
        assert np.max(np.abs(bad - want)) > 1e3 * tol, plant


def test_single_entry_with_sink_closed_form():
    g = np.random.default_rng(2)
    KV, H, hd, L = 1, 3, 16, 10
    k, v = _cache(g, KV, 16, hd)
    q = g.standard_normal(H * hd).astype(np.float32)
    sink = np.array([0.5, -1.0, 3.0], np.float32)
    c = orc_mod.Cache(k, v, KV, hd, capacity=16)
    got = orc_mod.attention_sparse(q, c, 0, L, H, [7, -1], sink)
    for h in range(H):
        s = float(q[h * hd:(h + 1) * hd].astype(np.float64) @ k[0, 0, 7].astype(np.float64)) / 4.0
        w = 1.0 / (1.0 + np.exp(float(sink[h]) - s))
        assert np.allclose(got[h * hd:(h + 1) * hd], w * v[0, 0, 7], rtol=1e-6, atol=1e-7)


def test_sink_limits_and_empty_selection():
    g = np.random.default_rng(3)
    KV, H, hd, L = 2, 4, 32, 30
    k, v = _cache(g, KV, 32, hd)
    q = g.standard_normal(H * hd).astype(np.float32)
    c = orc_mod.Cache(k, v, KV, hd, capacity=32)
    sel = np.array([1, 5, 29, -1], np.int32)
    plain = orc_mod.attention_sparse(q, c, 0, L, H, sel)
    ninf = orc_mod.attention_sparse(q, c, 0, L, H, sel, np.full(H, -np.inf, np.float32))
    assert np.array_equal(plain.view(np.uint32), ninf.view(np.uint32))
    huge = orc_mod.attention_sparse(q, c, 0, L, H, sel, np.full(H, 1e4, np.float32))
    assert np.max(np.abs(huge)) < 1e-30
    empty = orc_mod.attention_sparse(q, c, 0, L, H, [-1, -1], np.zeros(H, np.float32))
    assert np.all(empty == 0.0)
    assert np.all(orc_mod.attention_sparse(q, c, 0, L, H, [-1]) == 0.0)


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
def test_full_selection_is_dense_and_padding_is_inert(paged):
    g = np.random.default_rng(4 + paged)
    KV, H, hd, L = 2, 4, 32, 45
    if paged:
        ps, P, maxp = 8, 9, 7
        table = np.full((1, maxp), -1, np.int32)
        table[0, :6] = [4, 0, 8, 2, 5, 1]
        k = g.standard_normal((P, KV, ps, hd)).astype(np.float32)
        v = g.standard_normal((P, KV, ps, hd)).astype(np.float32)
        c = orc_mod.Cache(k, v, KV, hd, page_size=ps, page_table=table, max_pages_per_seq=maxp,
                          num_pages=P)
    else:
        k, v = _cache(g, KV, 64, hd)
        c = orc_mod.Cache(k, v, KV, hd, capacity=64)
    q = g.standard_normal(H * hd).astype(np.float32)
    dense = orc_mod.attention(q, c, 0, L, H)
    perm = g.permutation(L).astype(np.int32)
    sp = orc_mod.attention_sparse(q, c, 0, L, H, perm)
    assert np.max(np.abs(sp - dense)) <= 1e-6 * np.sqrt(np.mean(dense ** 2))
    # in token order the sums run in the same order as the dense ones
    ordered = orc_mod.attention_sparse(q, c, 0, L, H, np.arange(L, dtype=np.int32))
    assert np.array_equal(ordered.view(np.uint32), dense.view(np.uint32))
    sink = g.standard_normal(H).astype(np.float32)
    base = orc_mod.attention_sparse(q, c, 0, L, H, perm[:20], sink)
    padded = np.insert(perm[:20], [0, 5, 5, 20], -1).astype(np.int32)
    assert np.array_equal(orc_mod.attention_sparse(q, c, 0, L, H, padded, sink).view(np.uint32),
                          base.view(np.uint32))


def test_entries_not_held_are_errors():
    g = np.random.default_rng(6)
    KV, H, hd = 1, 2, 16
    k, v = _cache(g, KV, 16, hd)
    c = orc_mod.Cache(k, v, KV, hd, capacity=16)
    q = np.ones(H * hd, np.float32)
    with pytest.raises(ValueError):
        orc_mod.attention_sparse(q, c, 0, 10, H, [3, 10])          # past the sequence
    ring = orc_mod.Cache(k.copy(), v.copy(), KV, hd, capacity=16, ring=True, window=16)
    orc_mod.attention_sparse(q, ring, 0, 40, H, [24, 39])           # held: 24..39
    with pytest.raises(ValueError):
        orc_mod.attention_sparse(q, ring, 0, 40, H, [23])           # evicted
    table = np.array([[0, -1]], np.int32)
    pc = orc_mod.Cache(np.zeros((2, KV, 4, hd), np.float32), np.zeros((2, KV, 4, hd), np.float32),
                       KV, hd, page_size=4, page_table=table, max_pages_per_seq=2, num_pages=2)
    orc_mod.attention_sparse(q, pc, 0, 8, H, [0, 3])
    with pytest.raises(ValueError):
        orc_mod.attention_sparse(q, pc, 0, 8, H, [5])               # unmapped page


def test_layer_with_full_selection_equals_dense_layer(orc):
    cfg = synth.Config("ts", 91, 128, 4, 2, 32, 1e4, capacity=64, pos=20)
    w = synth.layer_weights(cfg, 0)
    cos, sin = synth.rope_for(cfg)
    kc, vc = synth.contiguous_cache(cfg, 0)
    x = synth.token_input(cfg)
    dims = dict(D=128, H=4, KV=2, hd=32, m=1, eps=cfg.eps)
    wts = dict(w, rope_cos=cos, rope_sin=sin)
    a = orc_mod.Cache(kc.copy(), vc.copy(), 2, 32, capacity=64)
    b = orc_mod.Cache(kc.copy(), vc.copy(), 2, 32, capacity=64)
    dense, tr_d = orc.decode_layer(dims, wts, a, x, x, [20], trace=True)
    sel = np.concatenate([np.arange(21), [-1, -1]]).astype(np.int32)[None]
    sparse, tr_s = orc.decode_layer(dims, wts, b, x, x, [20], trace=True, sel=sel)
    assert np.array_equal(tr_d["attn"].view(np.uint32), tr_s["attn"].view(np.uint32))
    assert np.array_equal(dense.view(np.uint32), sparse.view(np.uint32))
    # a strict subset with a sink: the layer's attention is the sparse attention
    # of its own q over the cache after the append
    c = orc_mod.Cache(kc.copy(), vc.copy(), 2, 32, capacity=64)
    sink = np.array([0.3, -0.2, 1.5, 0.0], np.float32)
    sub = np.array([[20, 3, -1, 11, 19]], np.int32)
    _, tr = orc.decode_layer(dims, wts, c, x, x, [20], trace=True, sel=sub, sink=sink)
    ref = orc_mod.attention_sparse(tr["q"][0], c, 0, 21, 4, sub[0], sink)
    assert np.array_equal(tr["attn"][0].view(np.uint32), ref.view(np.uint32))
