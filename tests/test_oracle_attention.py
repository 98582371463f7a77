"""Pins of the oracle's KV append and grouped-query decode attention.

Closed forms: one cached token returns that token's V for every query head of
its group; q = 0 returns the mean of V; a dominant score returns that token's V;
the softmax weights are non-negative and sum to 1. Library check: scipy's
softmax over float64 scores. Paging: the same logical tokens behind a shuffled
page table give the bit-identical result of the contiguous layout.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle as orc_mod


def _contig(KV, cap, hd, L, seed=0, m=1):
    g = np.random.default_rng(seed)
    k = np.full((m, KV, cap, hd), np.nan, np.float32)
    v = np.full((m, KV, cap, hd), np.nan, np.float32)
    k[:, :, :L] = g.standard_normal((m, KV, L, hd)).astype(np.float32)
    v[:, :, :L] = g.standard_normal((m, KV, L, hd)).astype(np.float32)
    return orc_mod.Cache(k, v, KV, hd, capacity=cap)


def _paged_from(cache, L, ps, seed=1, spare=3):
    """Copy the first L tokens of every sequence of a contiguous cache into a
    shuffled page pool."""
    m, KV, cap, hd = cache.k.shape
    npg = -(-L // ps)
    P = m * npg + spare
    perm = np.random.default_rng(seed).permutation(P).astype(np.int32)
    table = np.full((m, npg + 2), -1, np.int32)
    kp = np.full((P, KV, ps, hd), np.nan, np.float32)
    vp = np.full((P, KV, ps, hd), np.nan, np.float32)
    for s in range(m):
        for lp in range(npg):
            page = perm[s * npg + lp]
            table[s, lp] = page
            t0, t1 = lp * ps, min(L, (lp + 1) * ps)
            kp[page, :, : t1 - t0] = cache.k[s, :, t0:t1]
            vp[page, :, : t1 - t0] = cache.v[s, :, t0:t1]
    return orc_mod.Cache(kp, vp, KV, hd, page_size=ps, page_table=table,
                         max_pages_per_seq=npg + 2, num_pages=P)


@pytest.mark.parametrize("H,KV,hd,L", [(4, 2, 64, 17), (14, 2, 64, 300), (8, 8, 32, 5), (6, 1, 128, 40)])
def test_attention_matches_scipy_softmax(orc, H, KV, hd, L):
    c = _contig(KV, L + 3, hd, L, seed=H * 100 + L)
    q = np.random.default_rng(5).standard_normal(H * hd).astype(np.float32)
    out, probs = orc.attention(q, c, 0, L, H, want_probs=True)
    G = H // KV
    for h in range(H):
        g = h // G
        K = c.k[0, g, :L].astype(np.float64)
        V = c.v[0, g, :L].astype(np.float64)
        p = softmax(K @ q[h * hd:(h + 1) * hd].astype(np.float64) / np.sqrt(hd))
        assert np.allclose(probs[h], p, rtol=1e-12, atol=1e-15)
        assert np.allclose(out[h * hd:(h + 1) * hd], p @ V, rtol=2e-6, atol=2e-7)


def test_attention_probs_sum_to_one(orc):
    c = _contig(2, 40, 64, 33, seed=3)
    q = np.random.default_rng(6).standard_normal(4 * 64).astype(np.float32) * 3
    _, probs = orc.attention(q, c, 0, 33, 4, want_probs=True)
    assert np.all(probs >= 0)
    assert np.allclose(probs.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_attention_single_token_returns_v(orc):
    H, KV, hd = 6, 3, 64
    c = _contig(KV, 8, hd, 1, seed=4)
    q = np.random.default_rng(7).standard_normal(H * hd).astype(np.float32)
    out = orc.attention(q, c, 0, 1, H)
    for h in range(H):
        assert np.array_equal(out[h * hd:(h + 1) * hd], c.v[0, h // (H // KV), 0])


def test_attention_zero_query_is_mean_of_v(orc):
    H, KV, hd, L = 4, 2, 64, 50
    c = _contig(KV, 64, hd, L, seed=8)
    out = orc.attention(np.zeros(H * hd, np.float32), c, 0, L, H)
    for h in range(H):
        ref = c.v[0, h // 2, :L].astype(np.float64).mean(axis=0)
        assert np.allclose(out[h * hd:(h + 1) * hd], ref, rtol=1e-6, atol=1e-7)


def test_attention_dominant_token(orc):
    H, KV, hd, L, t = 2, 1, 64, 30, 11
    c = _contig(KV, 32, hd, L, seed=9)
    q = np.tile(c.k[0, 0, t] * 40.0, H).astype(np.float32)
    out = orc.attention(q, c, 0, L, H)
    for h in range(H):
        assert np.allclose(out[h * hd:(h + 1) * hd], c.v[0, 0, t], atol=1e-4)


@pytest.mark.parametrize("L,ps", [(37, 16), (16, 16), (1, 16), (100, 8)])
def test_paged_equals_contiguous_bitwise(orc, L, ps):
    m, H, KV, hd = 3, 8, 2, 64
    c = _contig(KV, L + 5, hd, L, seed=L, m=m)
    p = _paged_from(c, L, ps)
    q = np.random.default_rng(L).standard_normal(H * hd).astype(np.float32)
    for s in range(m):
        a = orc.attention(q, c, s, L, H)
        b = orc.attention(q, p, s, L, H)
        assert np.array_equal(a, b)


def test_paged_unmapped_page_is_an_error(orc):
    c = _contig(1, 40, 32, 32, seed=2)
    p = _paged_from(c, 32, 16)
    q = np.ones(32, np.float32)
    with pytest.raises(ValueError):
        orc.attention(q, p, 0, 33, 1)          # token 32 sits in an unmapped page


@pytest.mark.parametrize("paged", [False, True])
def test_kv_append_writes_one_slot(orc, paged):
    m, KV, hd, L = 2, 2, 64, 20
    c = _contig(KV, 32, hd, L, seed=12, m=m)
    if paged:
        c = _paged_from(c, 32, 16)
    k0, v0 = c.k.copy(), c.v.copy()
    knew = np.random.default_rng(1).standard_normal(KV * hd).astype(np.float32)
    vnew = np.random.default_rng(2).standard_normal(KV * hd).astype(np.float32)
    orc.kv_append(c, 1, L, knew, vnew)
    for before, after, new in ((k0, c.k, knew), (v0, c.v, vnew)):
        changed = ~((before == after) | (np.isnan(before) & np.isnan(after)))
        assert changed.sum() == KV * hd
        assert np.array_equal(np.sort(after[changed]), np.sort(new))
    # the appended token is the one attention sees at position L
    H = 2 * KV
    q = np.tile(np.repeat(knew.reshape(KV, hd), H // KV, axis=0).reshape(-1), 1) * 30
    out = orc.attention(q.astype(np.float32), c, 1, L + 1, H)
    for h in range(H):
        g = h // (H // KV)
        assert np.allclose(out[h * hd:(h + 1) * hd], vnew[g * hd:(g + 1) * hd], atol=1e-3)
