"""GPU parity of each C-ABI step against the oracle on identical inputs.

Bars: Q8_0 bytes and KV-cache contents bit-exact; RMSNorm, GEMV and RoPE
within 1e-5 x RMS; attention within 1e-4 x RMS (fp32 online softmax against
the oracle's double two-pass softmax). Shapes span several tiles and ragged
tails; edge cases: odd block counts, single rows, one attended token, empty
(fully masked) chunks, split-count independence, unmapped pages.
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


def _ck():
    from decode_step_attention_layer_amd import ck

    return ck


def _sync():
    import torch

    torch.cuda.synchronize()


# ------------------------------------------------------------- quantizer ---
def _tie_blocks(seed, n):
    """Blocks whose elements sit on or next to rounding boundaries: x = (k + 0.5) * d
    and its fp32 neighbours, for random scales (including fp16-subnormal d)."""
    g = np.random.default_rng(seed)
    out = np.zeros((n, 32), np.float32)
    for b in range(n):
        amax = np.float32(np.exp(g.uniform(np.log(1e-6), np.log(1e3))))
        d = np.float32(amax / np.float32(127))
        ks = g.integers(-126, 126, 31)
        x = ((ks + 0.5) * np.float64(d)).astype(np.float32)
        nudge = g.integers(-1, 2, 31)
        x = np.where(nudge < 0, np.nextafter(x, np.float32(-np.inf)),
                     np.where(nudge > 0, np.nextafter(x, np.float32(np.inf)), x))
        x = np.clip(x, -amax, amax).astype(np.float32)
        out[b, 0] = amax if g.random() < 0.5 else -amax
        out[b, 1:] = x
        g.shuffle(out[b])
    return out


def _reciprocal_blocks():
    """Blocks where x * fp32(1/d) and x / d round differently (found by search
    over integer multiples of 127)."""
    rows = []
    for amax_i in range(127 * 2, 127 * 3000, 127):
        amax = np.float32(amax_i)
        d = np.float32(amax / np.float32(127))
        idv = np.float32(np.float32(1) / d)
        for n in range(1, 126):
            x = np.float32((n + 0.5) * float(d))
            if float(x) != (n + 0.5) * float(d):
                continue
            if np.floor(float(np.float32(x * idv)) + 0.5) != n + 1:
                blk = np.zeros(32, np.float32)
                blk[0], blk[1], blk[2] = amax, x, -x
                rows.append(blk)
                break
        if len(rows) >= 64:
            break
    return np.array(rows, np.float32)


def test_quantize_q8_0_bitexact():
    dev = cuda()
    ck = _ck()
    g = np.random.default_rng(0)
    rand = g.standard_normal((40000, 32)).astype(np.float32)
    rand *= np.exp(g.uniform(-12, 8, (40000, 1))).astype(np.float32)
    zero = np.zeros((3, 32), np.float32)
    x = np.concatenate([rand, _tie_blocks(1, 4000), _reciprocal_blocks(), zero]).reshape(-1)
    nb = x.size // 32
    xd = _t(x, dev)
    import torch

    y = torch.empty(nb * 34, dtype=torch.uint8, device=dev)
    ck.ck_quantize_q8_0(xd, y, 1, x.size)
    _sync()
    ref = oracle.quantize_q8_0(x)
    got = host(y)
    bad = np.nonzero((got.reshape(nb, 34) != ref.reshape(nb, 34)).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} blocks differ, first {bad[:5]}"


@pytest.mark.parametrize("m,K", [(1, 32), (3, 896), (2, 4096)])
def test_quantize_q8_0_rows(m, K):
    dev = cuda()
    ck = _ck()
    x = synth.seeded_vector(m * K, m * K)
    import torch

    y = torch.empty(m * K // 32 * 34, dtype=torch.uint8, device=dev)
    ck.ck_quantize_q8_0(_t(x, dev), y, m, K)
    _sync()
    assert np.array_equal(host(y), oracle.quantize_q8_0(x))


# ---------------------------------------------------------------- rmsnorm ---
@pytest.mark.parametrize("m,D", [(1, 256), (1, 896), (4, 3584), (1, 4096), (2, 96)])
def test_rmsnorm(m, D):
    dev = cuda()
    ck = _ck()
    x = synth.seeded_vector(D, m * D).reshape(m, D)
    gam = synth.seeded_vector(D + 1, D, 0.1) + np.float32(1)
    import torch

    y = torch.empty((m, D), dtype=torch.float32, device=dev)
    ck.ck_rmsnorm(_t(x, dev), _t(gam, dev), y, m, D, 1e-6)
    _sync()
    for s in range(m):
        assert_close_rms(host(y)[s], oracle.rmsnorm(x[s], gam, 1e-6), 1e-5, "rmsnorm")


# ------------------------------------------------------------------- GEMV ---
GEMV_SHAPES = [
    # rows, K, m
    (1, 32, 1), (7, 96, 1), (129, 256, 1), (1152, 896, 1), (513, 3584, 1),
    (4096, 4096, 1), (200, 4096, 3), (300, 4096, 8), (64, 14336, 1), (33, 160, 2),
    # batches of 4..16 tokens with K % 64 == 0 take the matrix-core kernel:
    # ragged row tiles, block pairs spread unevenly over the 8 waves
    (100, 3584, 4), (77, 896, 5), (16, 64, 16), (48, 256, 6), (1024, 4096, 8), (40, 640, 12),
]


@pytest.mark.parametrize("q5", [True, False], ids=["q5_0", "q8_0"])
@pytest.mark.parametrize("rows,K,m", GEMV_SHAPES, ids=str)
def test_gemv(q5, rows, K, m):
    dev = cuda()
    ck = _ck()
    W = synth.seeded_vector(rows + K, rows * K, 0.02).reshape(rows, K)
    wb = (synth.weights_to_q5_0 if q5 else synth.weights_to_q8_0)(W)[0]
    x = synth.seeded_vector(K + 7, m * K)
    xq = oracle.quantize_q8_0(x)
    bias = synth.seeded_vector(rows + 3, rows, 0.02)
    res = synth.seeded_vector(rows + 4, m * rows)
    import torch

    y = torch.empty(m * rows, dtype=torch.float32, device=dev)
    fn = ck.ck_gemv_q5_0_q8_0 if q5 else ck.ck_gemv_q8_0_q8_0
    ref_fn = oracle.gemv_q5_0 if q5 else oracle.gemv_q8_0
    nbx = K // 32 * 34
    for with_res in (False, True):
        fn(_t(wb, dev), _t(xq, dev), _t(bias, dev), _t(res, dev) if with_res else None, y,
           rows, K, m)
        _sync()
        got = host(y).reshape(m, rows)
        for s in range(m):
            ref = ref_fn(wb, xq[s * nbx:(s + 1) * nbx], bias,
                         res[s * rows:(s + 1) * rows] if with_res else None, rows, K)
            base = ref - (res[s * rows:(s + 1) * rows] if with_res else 0)
            # tolerance on the projection itself (the residual would hide it)
            assert_close_rms(got[s] - (res[s * rows:(s + 1) * rows] if with_res else 0),
                             base, 1e-5, f"gemv s={s} res={with_res}")


def test_gemv_zero_weights_wiring():
    dev = cuda()
    ck = _ck()
    rows, K = 77, 896
    xq = oracle.quantize_q8_0(synth.seeded_vector(5, K))
    bias = synth.seeded_vector(6, rows, 0.02)
    res = synth.seeded_vector(7, rows)
    import torch

    y = torch.empty(rows, dtype=torch.float32, device=dev)
    ck.ck_gemv_q5_0_q8_0(_t(np.zeros(rows * K // 32 * 22, np.uint8), dev), _t(xq, dev),
                         _t(bias, dev), _t(res, dev), y, rows, K, 1)
    _sync()
    assert np.array_equal(host(y), (bias + res).astype(np.float32))


# ------------------------------------------------------------------- RoPE ---
@pytest.mark.parametrize("H,KV,hd,pos", [(4, 2, 64, 16), (28, 4, 128, 4096), (32, 8, 128, 32768)])
def test_rope(H, KV, hd, pos):
    dev = cuda()
    ck = _ck()
    rows = pos + 1
    cos, sin = synth.rope_tables(rows, hd, 5e5)
    q = synth.seeded_vector(1, H * hd)
    k = synth.seeded_vector(2, KV * hd)
    qd, kd = _t(q, dev), _t(k, dev)
    ck.ck_rope(qd, kd, _t(cos, dev), _t(sin, dev), rows, [pos], 1, H, KV, hd)
    _sync()
    rq, rk = oracle.rope(q, k, cos, sin, pos, H, KV, hd)
    assert_close_rms(host(qd), rq, 1e-5, "rope q")
    assert_close_rms(host(kd), rk, 1e-5, "rope k")


# ------------------------------------------------------------- KV append ---
def _caches(paged, m, KV, hd, L, seed, min_ctx=None):
    lo = max(1, L - 40) if min_ctx is None else min_ctx
    cfg = synth.Config("kv", 90 + seed, 64 * KV, KV, KV, hd, 1e4, m=m, capacity=L + 8, pos=L,
                       page_size=16 if paged else 0, min_ctx=lo, max_ctx=L)
    if paged:
        k, v, table, lens = synth.paged_cache(cfg, 0, spare_pages=3)
        oc = oracle.Cache(k.copy(), v.copy(), KV, hd, page_size=16, page_table=table,
                          max_pages_per_seq=cfg.max_pages_per_seq, num_pages=k.shape[0])
        return cfg, k, v, table, [int(x) for x in lens], oc
    k, v = synth.contiguous_cache(cfg, 0)
    oc = oracle.Cache(k.copy(), v.copy(), KV, hd, capacity=cfg.capacity)
    return cfg, k, v, None, [cfg.pos] * m, oc


def _dev_cache(ck, dev, cfg, k, v, table):
    kd, vd = _t(k, dev), _t(v, dev)
    td = _t(table, dev) if table is not None else None
    c = ck.kv_cache(kd, vd, cfg.KV, cfg.hd, cfg.capacity, cfg.page_size, td,
                    cfg.max_pages_per_seq, k.shape[0])
    return c, kd, vd, td


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
def test_kv_append_bitexact(paged):
    dev = cuda()
    ck = _ck()
    m, KV, hd, L = 3, 2, 64, 37
    cfg, k, v, table, pos, oc = _caches(paged, m, KV, hd, L, 1)
    c, kd, vd, td = _dev_cache(ck, dev, cfg, k, v, table)
    knew = synth.seeded_vector(11, m * KV * hd)
    vnew = synth.seeded_vector(12, m * KV * hd)
    ck.ck_kv_append(c, _t(knew, dev), _t(vnew, dev), pos, m)
    _sync()
    for s in range(m):
        oracle.kv_append(oc, s, pos[s], knew[s * KV * hd:(s + 1) * KV * hd],
                         vnew[s * KV * hd:(s + 1) * KV * hd])
    for got, ref in ((host(kd), oc.k), (host(vd), oc.v)):
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# -------------------------------------------------------------- attention ---
ATTN_CASES = [
    # m, H, KV, hd, L, chunk, paged
    (1, 4, 2, 64, 17, 0, False),
    (1, 4, 2, 64, 1, 0, False),
    (1, 14, 2, 64, 1025, 0, False),
    (1, 28, 4, 128, 4097, 0, False),
    (1, 28, 4, 128, 4097, 1024, False),
    (1, 8, 8, 128, 300, 64, False),
    (1, 40, 5, 128, 129, 0, False),
    (2, 16, 2, 128, 65, 128, False),
    (1, 32, 8, 128, 32769, 0, False),
    (4, 32, 8, 128, 700, 0, True),
    (3, 8, 1, 64, 90, 64, True),
    # 65-128 chunks per sequence (three and four merge wavefronts), more
    # than 128 (the workgroup merge), and past its 16 preloaded chunk slots
    # per thread (128 chunks at hd 128, 256 at hd 64)
    (1, 28, 4, 128, 6000, 0, False),       # the automatic plan: 63 chunks of 96
    (1, 28, 4, 128, 6000, 48, False),      # 125 chunks
    (1, 28, 4, 128, 9000, 48, False),      # 188 chunks
    (1, 14, 2, 64, 4097, 64, False),       # 65 chunks
    (1, 8, 1, 64, 20000, 64, False),       # 313 chunks
    (4, 32, 8, 128, 5000, 64, True),       # paged, m = 4: up to 79 chunks
    (1, 32, 8, 128, 6500, 64, False),      # 102 chunks
]


@pytest.mark.parametrize("m,H,KV,hd,L,chunk,paged", ATTN_CASES, ids=str)
def test_attention(m, H, KV, hd, L, chunk, paged):
    dev = cuda()
    ck = _ck()
    cfg, k, v, table, pos, oc = _caches(paged, m, KV, hd, L - 1, H + L)
    # the contiguous case attends pos + 1 = L tokens; fill slot pos too
    if not paged:
        g = np.random.default_rng(L)
        k[:, :, L - 1] = g.standard_normal((m, KV, hd)).astype(np.float32)
        v[:, :, L - 1] = g.standard_normal((m, KV, hd)).astype(np.float32)
        oc = oracle.Cache(k.copy(), v.copy(), KV, hd, capacity=cfg.capacity)
    else:
        for s in range(m):
            kn = synth.seeded_vector(100 + s, KV * hd)
            vn = synth.seeded_vector(200 + s, KV * hd)
            oracle.kv_append(oc, s, pos[s], kn, vn)
        k, v = oc.k.copy(), oc.v.copy()
    c, kd, vd, td = _dev_cache(ck, dev, cfg, k, v, table)
    q = synth.seeded_vector(7 + L, m * H * hd)
    import torch

    out = torch.empty(m * H * hd, dtype=torch.float32, device=dev)
    nws = ck.ck_attn_workspace_size(m, H, KV, hd, max(pos) + 1, chunk)
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)   # counters start at zero
    ck.ck_attn_decode_gqa(_t(q, dev), c, pos, out, m, H, 1.0 / np.sqrt(hd), chunk, ws, nws)
    _sync()
    got = host(out).reshape(m, H * hd)
    for s in range(m):
        ref = oracle.attention(q[s * H * hd:(s + 1) * H * hd], oc, s, pos[s] + 1, H)
        assert_close_rms(got[s], ref, 1e-4, f"attention s={s}")


def test_attention_split_count_independent():
    dev = cuda()
    ck = _ck()
    m, H, KV, hd, L = 1, 28, 4, 128, 4097
    cfg, k, v, table, pos, oc = _caches(False, m, KV, hd, L - 1, 3)
    k[:, :, L - 1] = 0.5
    v[:, :, L - 1] = -0.5
    c, kd, vd, td = _dev_cache(ck, dev, cfg, k, v, table)
    q = _t(synth.seeded_vector(9, m * H * hd), dev)
    import torch

    outs = []
    for chunk in (64, 192, 1024, 4160):
        out = torch.empty(m * H * hd, dtype=torch.float32, device=dev)
        nws = ck.ck_attn_workspace_size(m, H, KV, hd, L, chunk)
        ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
        ck.ck_attn_decode_gqa(q, c, pos, out, m, H, 1.0 / np.sqrt(hd), chunk, ws, nws)
        _sync()
        outs.append(host(out))
    for o in outs[1:]:
        assert_close_rms(o, outs[0], 1e-5, "split count")


def test_attention_two_pass_entry_points_match():
    """ck_attn_partial + ck_attn_merge give exactly what ck_attn_decode_gqa
    gives at the same explicit split (same kernels), and the merge's Q8_0
    output is the quantizer's. Groups of 4 heads (the vector kernel) and of 8
    (the matrix-core kernel); the automatic splits of the two may differ."""
    dev = cuda()
    ck = _ck()
    m, KV, hd, L = 3, 8, 128, 900
    cfg, k, v, table, pos, oc = _caches(True, m, KV, hd, L, 6)
    pos = [p - 1 for p in pos]
    c, kd, vd, td = _dev_cache(ck, dev, cfg, k, v, table)
    import torch

    for H, chunk in ((32, 192), (64, 64)):
        q = _t(synth.seeded_vector(5, m * H * hd), dev)
        nws = ck.ck_attn_workspace_size(m, H, KV, hd, max(pos) + 1, chunk)
        ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
        a = torch.empty(m * H * hd, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        bq = torch.empty(m * H * hd // 32 * 34, dtype=torch.uint8, device=dev)
        ck.ck_attn_decode_gqa(q, c, pos, a, m, H, 1.0 / np.sqrt(hd), chunk, ws, nws)
        ck.ck_attn_partial(q, c, pos, m, H, 1.0 / np.sqrt(hd), chunk, ws, nws)
        ck.ck_attn_merge(ws, nws, pos, m, H, KV, hd, chunk, b, bq)
        _sync()
        assert torch.equal(a, b), H
        assert np.array_equal(host(bq), oracle.quantize_q8_0(host(b)))


def test_attention_workspace_reuse():
    """Counters return to zero after every call: ten calls on one workspace
    give the same result as the first."""
    dev = cuda()
    ck = _ck()
    m, H, KV, hd, L = 2, 32, 8, 128, 3000
    cfg, k, v, table, pos, oc = _caches(True, m, KV, hd, L, 8)
    pos = [p - 1 for p in pos]          # attend the filled tokens only
    c, kd, vd, td = _dev_cache(ck, dev, cfg, k, v, table)
    q = _t(synth.seeded_vector(4, m * H * hd), dev)
    import torch

    nws = ck.ck_attn_workspace_size(m, H, KV, hd, max(pos) + 1, 128)
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
    outs = []
    for _ in range(10):
        out = torch.empty(m * H * hd, dtype=torch.float32, device=dev)
        ck.ck_attn_decode_gqa(q, c, pos, out, m, H, 1.0 / np.sqrt(hd), 128, ws, nws)
        outs.append(out)
    _sync()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    ref = oracle.attention(host(q)[:H * hd], oc, 0, pos[0] + 1, H)
    assert_close_rms(host(outs[0])[:H * hd], ref, 1e-4, "attention reuse")


def test_attention_unmapped_page_gives_nan():
    dev = cuda()
    ck = _ck()
    m, H, KV, hd, L = 2, 8, 2, 64, 40
    cfg, k, v, table, pos, oc = _caches(True, m, KV, hd, L, 5, min_ctx=L)
    table = table.copy()
    table[1, 1] = 10 ** 6                    # out of range for sequence 1 only
    c, kd, vd, td = _dev_cache(ck, dev, cfg, k, v, table)
    import torch

    out = torch.empty(m * H * hd, dtype=torch.float32, device=dev)
    nws = ck.ck_attn_workspace_size(m, H, KV, hd, max(pos) + 1, 0)
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
    pos = [30] * m
    ck.ck_attn_decode_gqa(_t(synth.seeded_vector(3, m * H * hd), dev), c, pos, out, m, H, 0.125,
                          0, ws, nws)
    _sync()
    got = host(out).reshape(m, H * hd)
    assert np.all(np.isnan(got[1]))
    assert np.all(np.isfinite(got[0]))
