"""Pins of the oracle's whole decode layer against float64 brute force.

The brute force below is written independently of the oracle: dequantized
weights come from the generator's codes and scales, RMSNorm and the
projections are numpy float64 matrix products, RoPE is complex multiplication,
attention is scipy's softmax over the appended cache. Two references:

* exact-steps: the two activation quantizations are applied (with the
  separately pinned Q8_0 quantizer), so the oracle must agree to fp32 rounding;
* unquantized: no activation quantization at all, so the oracle must agree
  within the error that 8-bit activations introduce.

Planted mistakes (wrong sign, dropped bias, wrong head map, no RoPE, wrong
scale, a transposed operand) are made in the brute force and must fall outside
the exact-steps tolerance, so the tolerance is known to discriminate.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle as orc_mod
from decode_step_attention_layer_amd import synth


def _dq5(codes, s16):
    rows, nb, _ = codes.shape
    return (s16.astype(np.float64)[..., None] * (codes.astype(np.float64) - 16)).reshape(rows, nb * 32)


def _dq8(codes, s16):
    rows, nb, _ = codes.shape
    return (s16.astype(np.float64)[..., None] * codes.astype(np.float64)).reshape(rows, nb * 32)


def _dq_act(blocks):
    b = blocks.reshape(-1, 34)
    d = b[:, :2].copy().view("<f2")[:, 0].astype(np.float64)
    return (d[:, None] * b[:, 2:].view(np.int8).astype(np.float64)).reshape(-1)


def _small_cfg(D, H, KV, hd, pos, cap, theta=1e4, index=50):
    return synth.Config("t", index, D, H, KV, hd, theta, capacity=cap, pos=pos)


def brute(cfg, w, x, kc, vc, pos, quantize=None, plant=None):
    """float64 layer; kc/vc: [KV][cap][hd] prior cache (tokens < pos valid)."""
    D, H, KV, hd = cfg.D, cfg.H, cfg.KV, cfg.hd
    half = hd // 2
    x64 = x.astype(np.float64)
    xn = x64 / np.sqrt(np.mean(x64 * x64) + cfg.eps) * w["gamma"].astype(np.float64)
    xin = _dq_act(quantize(xn.astype(np.float32))) if quantize else xn
    Wq, Wk = _dq5(w["wq_codes"], w["wq_scales"]), _dq5(w["wk_codes"], w["wk_scales"])
    Wv, Wo = _dq8(w["wv_codes"], w["wv_scales"]), _dq5(w["wo_codes"], w["wo_scales"])
    if plant == "transpose_wo":
        Wo = Wo.reshape(H * hd, D).T if D == H * hd else Wo
        Wo = Wo[::-1]
    q = Wq @ xin + w["bq"]
    k = Wk @ xin + w["bk"]
    v = Wv @ xin + (0 if plant == "drop_bv" else w["bv"])
    if plant != "no_rope":
        ang = pos * cfg.theta ** (-2.0 * np.arange(half) / hd)
        rot = np.exp(1j * ang)

        def rope(a, n):
            a = a.reshape(n, hd)
            z = (a[:, :half] + 1j * a[:, half:]) * rot
            return np.concatenate([z.real, z.imag], axis=1).reshape(-1)
        q, k = rope(q, H), rope(k, KV)
    # the oracle stores q, k, v in fp32 before attention
    q, k, v = (t.astype(np.float32).astype(np.float64) for t in (q, k, v))
    scale = 1.0 / np.sqrt(hd) * (2.0 if plant == "scale" else 1.0)
    a = np.zeros(H * hd)
    G = H // KV
    for h in range(H):
        g = (h % KV) if plant == "head_map" else h // G
        Kc = np.concatenate([kc[g, :pos].astype(np.float64), k[g * hd:(g + 1) * hd][None]], 0)
        Vc = np.concatenate([vc[g, :pos].astype(np.float64), v[g * hd:(g + 1) * hd][None]], 0)
        p = softmax(Kc @ q[h * hd:(h + 1) * hd] * scale)
        a[h * hd:(h + 1) * hd] = p @ Vc
    ain = _dq_act(quantize(a.astype(np.float32))) if quantize else a
    branch = Wo @ ain + w["bo"]
    if plant == "sign":
        branch = -branch
    return branch, dict(xn=xn, q=q, k=k, v=v, attn=a)


SHAPES = [
    # D, H, KV, hd, pos, cap
    (64, 2, 1, 32, 3, 8),
    (64, 2, 2, 32, 0, 4),
    (224, 7, 1, 32, 9, 16),
    (256, 4, 2, 64, 16, 64),      # the tiny workload's shape
]


def _run(orc, shape, seed_layer=0):
    D, H, KV, hd, pos, cap = shape
    cfg = _small_cfg(D, H, KV, hd, pos, cap, index=60 + D + H)
    w = synth.layer_weights(cfg, seed_layer, keep_codes=True)
    x = synth.token_input(cfg)
    kc, vc = synth.contiguous_cache(cfg, seed_layer)
    cos, sin = synth.rope_for(cfg)
    cache = orc_mod.Cache(kc.copy(), vc.copy(), KV, hd, capacity=cap)
    dims = dict(D=D, H=H, KV=KV, hd=hd, m=1, eps=cfg.eps)
    wts = dict(w, rope_cos=cos, rope_sin=sin)
    out, tr = orc.decode_layer(dims, wts, cache, x, x, [pos], trace=True)
    return cfg, w, x, kc[0], vc[0], out[0], tr, cache


@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_layer_matches_exact_steps_brute_force(orc, shape):
    cfg, w, x, kc, vc, out, tr, _ = _run(orc, shape)
    branch, mid = brute(cfg, w, x[0], kc, vc, cfg.pos, quantize=orc.quantize_q8_0)
    got = out.astype(np.float64) - x[0].astype(np.float64)
    rms = np.sqrt(np.mean(branch ** 2))
    assert np.max(np.abs(got - branch)) <= 2e-5 * rms
    assert np.max(np.abs(tr["attn"][0] - mid["attn"])) <= 1e-5 * np.sqrt(np.mean(mid["attn"] ** 2))


@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_layer_within_activation_quantization_error(orc, shape):
    cfg, w, x, kc, vc, out, tr, _ = _run(orc, shape)
    branch, _ = brute(cfg, w, x[0], kc, vc, cfg.pos, quantize=None)
    got = out.astype(np.float64) - x[0].astype(np.float64)
    rms = np.sqrt(np.mean(branch ** 2))
    # two 8-bit activation quantizations: about 1% of the branch RMS
    assert np.max(np.abs(got - branch)) <= 0.05 * rms


@pytest.mark.parametrize("plant", ["sign", "drop_bv", "no_rope", "scale", "head_map", "transpose_wo"])
def test_planted_mistakes_exceed_tolerance(orc, plant):
    shape = (256, 4, 2, 64, 16, 64)
    cfg, w, x, kc, vc, out, tr, _ = _run(orc, shape)
    bad, _ = brute(cfg, w, x[0], kc, vc, cfg.pos, quantize=orc.quantize_q8_0, plant=plant)
    good, _ = brute(cfg, w, x[0], kc, vc, cfg.pos, quantize=orc.quantize_q8_0)
    rms = np.sqrt(np.mean(good ** 2))
    assert np.max(np.abs(bad - good)) > 2e-3 * rms, plant


def test_layer_appends_exactly_one_token(orc):
    cfg, w, x, kc, vc, out, tr, cache = _run(orc, SHAPES[3])
    pos = cfg.pos
    assert np.array_equal(cache.k[0, :, pos].reshape(-1), tr["k"][0])
    assert np.array_equal(cache.v[0, :, pos].reshape(-1), tr["v"][0])
    same_k = np.array_equal(cache.k[0, :, :pos], kc[:, :pos])
    assert same_k and np.array_equal(cache.v[0, :, :pos], vc[:, :pos])
    assert np.all(np.isnan(cache.k[0, :, pos + 1:])) and np.all(np.isnan(cache.v[0, :, pos + 1:]))


def test_layer_trace_is_consistent_with_steps(orc):
    # the layer is the composition of the separately pinned steps
    cfg, w, x, kc, vc, out, tr, cache = _run(orc, SHAPES[2])
    xn = orc.rmsnorm(x[0], w["gamma"], cfg.eps)
    assert np.array_equal(xn, tr["xn"][0])
    assert np.array_equal(orc.quantize_q8_0(xn), tr["xq"][0])
    HD = cfg.H * cfg.hd
    assert np.array_equal(orc.gemv_q5_0(w["wq"], tr["xq"][0], w["bq"], None, HD, cfg.D), tr["q_pre"][0])
    assert np.array_equal(orc.quantize_q8_0(tr["attn"][0]), tr["aq"][0])
    o = orc.gemv_q5_0(w["wo"], tr["aq"][0], w["bo"], x[0], cfg.D, HD)
    assert np.array_equal(o, out)


def test_batched_sequences_are_independent(orc):
    # m tokens in one call equal m single-token calls (paged cache)
    cfg = synth.Config("tp", 70, 128, 4, 2, 32, 5e5, m=3, page_size=16, min_ctx=5, max_ctx=40)
    w = synth.layer_weights(cfg, 0)
    kp, vp, table, lens = synth.paged_cache(cfg, 0, spare_pages=2)
    cos, sin = synth.rope_for(cfg)
    x = synth.token_input(cfg)
    dims = dict(D=128, H=4, KV=2, hd=32, m=3, eps=cfg.eps)
    wts = dict(w, rope_cos=cos, rope_sin=sin)
    mk = lambda: orc_mod.Cache(kp.copy(), vp.copy(), 2, 32, page_size=16, page_table=table,
                              max_pages_per_seq=cfg.max_pages_per_seq, num_pages=kp.shape[0])
    ca = mk()
    out = orc.decode_layer(dims, wts, ca, x, x, lens)
    for s in range(3):
        cb = mk()
        tb = cb.page_table.copy()
        cb.page_table = np.ascontiguousarray(tb[s:s + 1])
        o1 = orc.decode_layer(dict(dims, m=1), wts, cb, x[s:s + 1], x[s:s + 1], lens[s:s + 1])
        assert np.array_equal(o1[0], out[s])
