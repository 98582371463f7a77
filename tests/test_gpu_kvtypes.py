"""GPU parity of the bf16 and FP8 E4M3 KV caches against the oracle.

  * Store: ck_kv_append of random values and of hand-built edge values (ties
    of both formats, fp8 subnormals, values past the fp8 range, NaN) writes
    exactly the oracle's codes at the appended slot and nothing elsewhere.
  * Load: attention over a single cached token returns that token's V, so
    every fp8 code (and a sweep of bf16 codes) read through the attention
    kernel equals the oracle's decoded value (times the scale) exactly; and
    every K code (fp8 but the NaNs; bf16 finite codes with the subnormals)
    read through the scores gives the oracle's softmax weights.
  * Attention over thousands of cached tokens within 1e-4 x RMS of the
    oracle on the same cache bytes, contiguous and paged.
  * Whole layer (tiny, long-context, batched paged) with fused and chain
    variants: the appended bytes equal the oracle's codes of the GPU's own k
    and v; attention within 1e-4 of the oracle on the GPU's q and cache;
    output within 2e-3 x RMS of the oracle run on the same input; every other
    cache byte unchanged.
"""
import math

import numpy as np
import pytest

import oracle
from decode_step_attention_layer_amd import synth
from gpu_helpers import assert_close_rms, cuda, host

pytestmark = pytest.mark.gpu

DTYPES = [synth.KV_BF16, synth.KV_FP8]
IDS = ["bf16", "fp8"]
NP_T = {synth.KV_BF16: np.uint16, synth.KV_FP8: np.uint8}
SCALES = {synth.KV_BF16: (1.0, 1.0), synth.KV_FP8: (synth.FP8_K_SCALE, synth.FP8_V_SCALE)}


def _t(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _edge_values(dtype, n):
    if dtype == synth.KV_BF16:
        base = [1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 2.0**-130, 0.0, -0.0, math.inf,
                -math.inf, math.nan, 3.3895314e38, 65504.0, 1e-38]
    else:
        s = synth.FP8_K_SCALE
        # value / scale lands on ties, subnormals and past the range
        base = [v * s for v in [2**-10, 3 * 2**-10, 5 * 2**-10, 1.0625, 1.1875, 448.0, 456.0,
                                464.0, 465.0, 1e6, -1e6, 2**-7, 0.0, -0.0, math.nan,
                                math.inf, 240.0 + 8.0]]
    vals = np.array(base * (n // len(base) + 1), np.float32)[:n]
    return vals


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("edge", [False, True], ids=["random", "edge"])
def test_append_writes_the_oracle_codes(dtype, paged, edge):
    import torch

    dev = cuda()
    from decode_step_attention_layer_amd import ck

    KV, hd, m = 2, 64, 2
    ks, vs = SCALES[dtype]
    g = np.random.default_rng(3 + dtype + 2 * paged)
    if paged:
        ps, P, maxp = 16, 9, 4
        table = np.full((m, maxp), -1, np.int32)
        table[0, :3] = [4, 1, 7]
        table[1, :3] = [0, 8, 2]
        shape = (P, KV, ps, hd)
        pos = [37, 21]
    else:
        shape = (m, KV, 64, hd)
        pos = [40, 5]
    kc = g.integers(0, 2**16 if dtype == synth.KV_BF16 else 256, size=shape).astype(NP_T[dtype])
    vc = g.integers(0, 2**16 if dtype == synth.KV_BF16 else 256, size=shape).astype(NP_T[dtype])
    n = m * KV * hd
    if edge:
        kn, vn = _edge_values(dtype, n), _edge_values(dtype, n)[::-1].copy()
    else:
        kn = (g.standard_normal(n) * 2).astype(np.float32)
        vn = (g.standard_normal(n) * 2).astype(np.float32)
    dk, dv = _t(kc, dev), _t(vc, dev)
    if paged:
        dt = _t(table, dev)
        cache = ck.kv_cache(dk, dv, KV, hd, 0, ps, dt, maxp, P, dtype=dtype, k_scale=ks,
                            v_scale=vs)
    else:
        cache = ck.kv_cache(dk, dv, KV, hd, 64, dtype=dtype, k_scale=ks, v_scale=vs)
    ck.ck_kv_append(cache, _t(kn, dev), _t(vn, dev), pos, m)
    torch.cuda.synchronize()
    gk, gv = host(dk), host(dv)
    oc = oracle.Cache(kc.copy(), vc.copy(), KV, hd, dtype=dtype, k_scale=ks, v_scale=vs,
                      **(dict(page_size=ps, page_table=table, max_pages_per_seq=maxp,
                              num_pages=P) if paged else dict(capacity=64)))
    for s in range(m):
        oracle.kv_append(oc, s, pos[s], kn[s * KV * hd:(s + 1) * KV * hd],
                         vn[s * KV * hd:(s + 1) * KV * hd])
    assert np.array_equal(gk, oc.k), "K cache bytes differ from the oracle's"
    assert np.array_equal(gv, oc.v), "V cache bytes differ from the oracle's"


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
def test_single_token_attention_decodes_every_code(dtype):
    """L = 1: the output is the token's V exactly (weight 1), so the kernel's
    decode of each code is compared with the oracle's, bit for bit."""
    import torch

    dev = cuda()
    from decode_step_attention_layer_amd import ck

    hd = 128
    ks, vs = SCALES[dtype]
    if dtype == synth.KV_FP8:
        codes = np.arange(256, dtype=np.uint8)
    else:
        g = np.random.default_rng(9)
        codes = np.concatenate([
            np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0,
                      0x3F80, 0x3F81, 0x4049], np.uint16),
            g.integers(0, 2**16, size=244).astype(np.uint16)])
    KV = len(codes) // hd                      # one row of V codes per KV head
    H = KV
    shape = (1, KV, 4, hd)
    kc = np.zeros(shape, NP_T[dtype])
    vc = np.zeros(shape, NP_T[dtype])
    vc[0, :, 0, :] = codes.reshape(KV, hd)
    # the cache view holds raw pointers: the tensors must outlive every call
    kd, vd = _t(kc, dev), _t(vc, dev)
    cache = ck.kv_cache(kd, vd, KV, hd, 4, dtype=dtype, k_scale=ks, v_scale=vs)
    q = torch.ones(H * hd, dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    nws = ck.ck_attn_workspace_size(1, H, KV, hd, 1, 0)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    ck.ck_attn_decode_gqa(q, cache, [0], out, 1, H, 1.0 / math.sqrt(hd), 0, ws, nws)
    torch.cuda.synchronize()
    got = host(out)
    want = oracle.decode_cache(codes, dtype, vs)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    # equal as numbers (the attention's sums start at +0, so a -0 code reads
    # back as +0); every other value, subnormals and infinities included, exactly
    bad = got[~nan] != want[~nan]
    assert not bad.any(), (codes[~nan][bad], got[~nan][bad], want[~nan][bad])


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
def test_scores_decode_every_k_code(dtype):
    """The score path reads every K code as the oracle does: one KV head per
    code (every fp8 code but the NaNs; a sweep of finite bf16 codes with the
    subnormals and the extremes), two cached tokens per head: token 0's K
    holds the code at dim 0, token 1's K is zero, and V picks out the two
    softmax weights. q is scaled per head so that a correctly read code
    scores exactly 1 against token 1's 0 (within |q| <= 1e30: the smallest
    bf16 subnormals cannot reach it): a code read as another value (a
    subnormal flushed to zero, a wrong exponent) moves the weights far
    beyond the 1e-4 x RMS the output is held to against the oracle."""
    import torch

    dev = cuda()
    from decode_step_attention_layer_amd import ck

    hd = 64
    ks, vs = SCALES[dtype]
    g = np.random.default_rng(5)
    if dtype == synth.KV_FP8:
        codes = g.permutation(np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8))
    else:
        fixed = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x00FF, 0x7F7F, 0xFF7F, 0x3F80,
                 0xBF80, 0x0100, 0x4B00, 0x3400]
        rnd = g.integers(0, 2**16, size=400).astype(np.uint16)
        rnd = rnd[(rnd & 0x7F80) != 0x7F80][:240]          # finite only
        codes = np.concatenate([np.array(fixed, np.uint16), rnd])
    KV = H = len(codes)
    kc = np.zeros((1, KV, 2, hd), NP_T[dtype])
    kc[0, :, 0, 0] = codes
    one = oracle.encode_cache(np.array([1.0], np.float32), dtype, vs)[0]
    vc = np.zeros((1, KV, 2, hd), NP_T[dtype])
    vc[0, :, 0, 0] = one
    vc[0, :, 1, 1] = one
    kval = oracle.decode_cache(codes, dtype, ks).astype(np.float64)
    scale = 1.0 / math.sqrt(hd)
    q = np.zeros(H * hd, np.float32)
    nz = kval != 0
    # |q| within [1e-30, 1e30]: bf16 codes too small (or too large) for a
    # score of 1 with such a q are read at the nearest bound instead
    target = 1.0 / (kval[nz] * scale)
    q[np.arange(H)[nz] * hd] = (np.sign(target) *
                                np.clip(np.abs(target), 1e-30, 1e30)).astype(np.float32)
    kd, vd = _t(kc, dev), _t(vc, dev)   # the view holds raw pointers: keep them alive
    cache = ck.kv_cache(kd, vd, KV, hd, 2, dtype=dtype, k_scale=ks, v_scale=vs)
    out = torch.empty(H * hd, dtype=torch.float32, device=dev)
    nws = ck.ck_attn_workspace_size(1, H, KV, hd, 2, 0)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    ck.ck_attn_decode_gqa(_t(q, dev), cache, [1], out, 1, H, scale, 0, ws, nws)
    torch.cuda.synchronize()
    got = host(out)
    oc = oracle.Cache(kc, vc, KV, hd, capacity=2, dtype=dtype, k_scale=ks, v_scale=vs)
    ref = oracle.attention(q, oc, 0, 2, H)
    # every head's weight pair, one by one (a correctly read code gives
    # weights e/(e+1), 1/(e+1)), then the whole output
    w = got.reshape(H, hd)[:, :2]
    wr = ref.reshape(H, hd)[:, :2]
    bad = np.abs(w - wr).max(axis=1) > 1e-4 * np.abs(wr).max(axis=1)
    assert not bad.any(), ([hex(int(c)) for c in codes[bad]], w[bad], wr[bad])
    assert_close_rms(got, ref, 1e-4, "per-code scores")


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("name", ["c4", "c5"])
def test_attention_over_reduced_cache(dtype, name):
    import torch

    dev = cuda()
    from decode_step_attention_layer_amd import ck
    from decode_step_attention_layer_amd.workload import DeviceStack

    cfg = synth.CONFIGS[name]
    stack = DeviceStack(cfg, dev, keep_host=True, kv_dtype=dtype)
    L = stack.layers[0]
    m, H, KV, hd = cfg.m, cfg.H, cfg.KV, cfg.hd
    q = synth.seeded_vector(77, m * H * hd).astype(np.float32)
    out = torch.empty(m * H * hd, dtype=torch.float32, device=dev)
    nws = ck.ck_attn_workspace_size(m, H, KV, hd, stack.max_ctx, 0)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    # attend the prior tokens only (the slot at pos is still poisoned)
    prior = [p - 1 for p in stack.pos]
    ck.ck_attn_decode_gqa(_t(q, dev), L.cache, prior, out, m, H, 1.0 / math.sqrt(hd), 0, ws,
                          nws)
    torch.cuda.synchronize()
    got = host(out).reshape(m, H * hd)
    ks, vs = stack.k_scale, stack.v_scale
    geo = (dict(page_size=cfg.page_size, page_table=L.host["table"],
                max_pages_per_seq=cfg.max_pages_per_seq, num_pages=L.host["k"].shape[0])
           if cfg.page_size else dict(capacity=cfg.capacity))
    oc = oracle.Cache(L.host["k"], L.host["v"], KV, hd, dtype=dtype, k_scale=ks, v_scale=vs, **geo)
    for s in range(m):
        ref = oracle.attention(q[s * H * hd:(s + 1) * H * hd], oc, s, stack.pos[s], H)
        assert_close_rms(got[s], ref, 1e-4, f"{name} seq {s} attention")


def _layer_check(name, dtype, variant):
    import torch

    dev = cuda()
    from decode_step_attention_layer_amd import ck
    from decode_step_attention_layer_amd.workload import DeviceStack

    cfg = synth.CONFIGS[name]
    stack = DeviceStack(cfg, dev, keep_host=True, spare_pages=2 if cfg.page_size else 0,
                        layers=1, kv_dtype=dtype)
    L = stack.layers[0]
    m, D, H, KV, hd = cfg.m, cfg.D, cfg.H, cfg.KV, cfg.hd
    desc = stack.desc(variant)
    ws = stack.workspace(desc)
    off = {n: ck.ck_decode_layer_ws_offset(desc, stack.max_ctx, n) for n in ("q", "k", "v", "attn")}
    out = stack.bufs[0]
    ck.ck_decode_layer(desc, L.weights, L.cache, stack.x0, stack.x0, stack.pos, out, ws,
                       ws.numel())
    torch.cuda.synchronize()

    def rd(n, count):
        return ws[off[n]: off[n] + 4 * count].cpu().numpy().view(np.float32)

    gq = rd("q", m * H * hd).reshape(m, H * hd)
    gk = rd("k", m * KV * hd).reshape(m, KV * hd)
    gv = rd("v", m * KV * hd).reshape(m, KV * hd)
    at = rd("attn", m * H * hd).reshape(m, H * hd)
    ks, vs = stack.k_scale, stack.v_scale
    geo = (dict(page_size=cfg.page_size, page_table=L.host["table"],
                max_pages_per_seq=cfg.max_pages_per_seq, num_pages=L.host["k"].shape[0])
           if cfg.page_size else dict(capacity=cfg.capacity))
    # the cache after the GPU's append == the original cache + the oracle's codes
    # of the GPU's own k and v
    exp = oracle.Cache(L.host["k"].copy(), L.host["v"].copy(), KV, hd, dtype=dtype, k_scale=ks,
                       v_scale=vs, **geo)
    for s in range(m):
        oracle.kv_append(exp, s, stack.pos[s], gk[s], gv[s])
    ck_, cv_ = host(L.tensors["k"]), host(L.tensors["v"])
    assert np.array_equal(ck_, exp.k) and np.array_equal(cv_, exp.v), "cache bytes"
    # attention on the GPU's q and cache
    gcache = oracle.Cache(ck_, cv_, KV, hd, dtype=dtype, k_scale=ks, v_scale=vs, **geo)
    for s in range(m):
        a0 = oracle.attention(gq[s], gcache, s, stack.pos[s] + 1, H)
        assert_close_rms(at[s], a0, 1e-4, f"{name} seq {s} attention")
    # the whole layer on the same input
    cos, sin = synth.rope_for(cfg)
    oc = oracle.Cache(L.host["k"].copy(), L.host["v"].copy(), KV, hd, dtype=dtype, k_scale=ks,
                      v_scale=vs, **geo)
    ref = oracle.decode_layer(dict(D=D, H=H, KV=KV, hd=hd, m=m, eps=cfg.eps),
                              dict(L.host, rope_cos=cos, rope_sin=sin), oc, stack.x0_host,
                              stack.x0_host, stack.pos)
    assert_close_rms(host(out), ref, 2e-3, f"{name} layer output")


@pytest.mark.parametrize("variant", [0, 1, 3], ids=["chain", "fused", "two_launch"])
@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("name", ["c1", "c4", "c5"])
def test_layer_with_reduced_cache(name, dtype, variant):
    _layer_check(name, dtype, variant)
