"""Parity checks shared by the GPU tests: the layer checked stage by stage on
the GPU's own intermediates, the branch (out - residual) against the oracle
with a bound derived from the data, Q8_0 rounding-boundary flips, and an
oracle decode loop that keeps its own caches.

Why a data-derived branch bound. The GPU and the oracle round differently
(fp32 with reassociated sums against double), so the fp32 value entering a
Q8_0 quantizer can differ in its last bits; where it sits on a rounding
boundary one code flips by one. A flip is legitimate, and its effect on the
output is not small against the 2e-3 x RMS(branch) budget: one flipped code of
the attention output moves every output row e by |Wo[e, j]| times the block's
scale. So the branch is checked against the oracle run from the GPU's own
xq codes (the "conditioned" oracle, whose only difference from the GPU is
last-bit rounding upstream of aq) within

    2e-3 x RMS(branch) + sum_j |Wo[e, j]| * |deq(aq_gpu)_j - deq(aq_oracle)_j|,

the second term being exactly the largest movement the counted aq flips can
cause (it is zero where no code differs), after every differing aq code has
been shown to be a +-1 flip at a rounding boundary. The plain oracle on the
same input differs from the conditioned one only by the xq flips (themselves
checked to be boundary flips), whose effect the oracle evaluates: the
difference of the two oracle runs. Nothing from the GPU widens a bound except
its quantized codes, and those only after the flip check.
"""
from __future__ import annotations

import numpy as np

import oracle
from gpu_helpers import assert_close_rms, rms

TOL = 2e-3


# ---------------------------------------------------------------- Q8_0 -----
def q8_parts(b):
    """(scales as float64, codes as int64 [nblocks][32]) of Q8_0 bytes."""
    b = np.ascontiguousarray(b, np.uint8).reshape(-1, 34)
    d = b[:, :2].copy().view("<f2")[:, 0].astype(np.float64)
    return d, b[:, 2:].view(np.int8).astype(np.int64)


def q8_values(b):
    """Dequantized values (float64) of Q8_0 bytes: scale times code."""
    d, q = q8_parts(b)
    return (d[:, None] * q).reshape(-1)


def check_flips(gpu_bytes, orc_bytes, gpu_vals, orc_vals, tag):
    """Q8_0 blocks from two pipelines whose fp32 inputs differ in the last
    bits: scales may differ by one binary16 step, codes by one, and only where
    both pipelines' scaled values sit within 1% of a quantum of the rounding
    boundary. Returns the number of differing codes."""
    dg, qg = q8_parts(gpu_bytes)
    do, qo = q8_parts(orc_bytes)
    step = np.spacing(np.maximum(dg, do).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(dg - do) <= step), tag + ": scale differs by more than one fp16 step"
    assert np.abs(qg - qo).max(initial=0) <= 1, tag + ": a code differs by more than one"
    vg = np.asarray(gpu_vals, np.float64).reshape(-1, 32)
    vo = np.asarray(orc_vals, np.float64).reshape(-1, 32)
    ag = np.abs(vg).max(axis=1, keepdims=True)
    ao = np.abs(vo).max(axis=1, keepdims=True)
    sg = np.where(ag > 0, vg * 127.0 / np.where(ag > 0, ag, 1), 0.0)
    so = np.where(ao > 0, vo * 127.0 / np.where(ao > 0, ao, 1), 0.0)
    flip = qg != qo
    if flip.any():
        assert np.all(np.abs(sg - so)[flip] < 0.01), tag + ": flip from a large value difference"
        frac = np.abs(so[flip]) - np.floor(np.abs(so[flip]))
        assert np.all(np.abs(frac - 0.5) < 0.01), tag + ": flip away from a rounding boundary"
    return int(flip.sum())


def abs_q5_matrix(blocks, rows: int, K: int) -> np.ndarray:
    """|W| (float64, [rows][K]) of a Q5_0 matrix, dequantized by the oracle."""
    return np.abs(oracle.dequantize_q5_0(np.ascontiguousarray(blocks, np.uint8).reshape(-1),
                                         rows * K).astype(np.float64)).reshape(rows, K)


# ------------------------------------------------------- oracle pieces -----
def oracle_from_xq(dims, wts, cache, x_s, xq_s, s: int, pos_s: int):
    """The oracle's layer for sequence s from the given Q8_0 codes of the
    normalized input: projections, RoPE, append into `cache` (mutated),
    attention over pos_s + 1 tokens, Q8_0 of the attention output, O
    projection + bias + residual x_s."""
    D, H, KV, hd = dims["D"], dims["H"], dims["KV"], dims["hd"]
    q0 = oracle.gemv_q5_0(wts["wq"], xq_s, wts["bq"], None, H * hd, D)
    k0 = oracle.gemv_q5_0(wts["wk"], xq_s, wts["bk"], None, KV * hd, D)
    v0 = oracle.gemv_q8_0(wts["wv"], xq_s, wts["bv"], None, KV * hd, D)
    q1, k1 = oracle.rope(q0, k0, wts["rope_cos"], wts["rope_sin"], pos_s, H, KV, hd)
    oracle.kv_append(cache, s, pos_s, k1, v0)
    a = oracle.attention(q1, cache, s, pos_s + 1, H)
    aq = oracle.quantize_q8_0(a)
    out = oracle.gemv_q5_0(wts["wo"], aq, wts["bo"], x_s, D, H * hd)
    return dict(q=q1, k=k1, v=v0, attn=a, aq=aq, out=out)


def branch_bound_check(got_s, x_s, cond_out, pure_out, aq_gpu, aq_cond, wo_abs, tag):
    """The branch (out - x) of one sequence against the oracle conditioned on
    the GPU's xq codes, within 2e-3 x RMS(branch) plus the aq flips' largest
    effect; and against the plain oracle, plus the oracle-evaluated effect of
    the xq flips (cond - pure). Returns the two relative errors."""
    x = np.asarray(x_s, np.float64)
    g = np.asarray(got_s, np.float64) - x
    c = np.asarray(cond_out, np.float64) - x
    p = np.asarray(pure_out, np.float64) - x
    assert np.all(np.isfinite(g)), tag + ": non-finite branch"
    flips = wo_abs @ np.abs(q8_values(aq_gpu) - q8_values(aq_cond))
    # the rounding of out = x + branch (two fp32 ulps at the output's size)
    ulps = 2 * np.spacing(np.abs(np.asarray(got_s, np.float32))).astype(np.float64)
    bc = TOL * rms(c) + flips + ulps
    ec = np.abs(g - c)
    assert np.all(ec <= bc), (f"{tag}: branch vs oracle on the GPU's xq codes, "
                              f"worst excess {float(np.max(ec - bc)):.3e}")
    bp = TOL * rms(p) + flips + np.abs(c - p) + ulps
    ep = np.abs(g - p)
    assert np.all(ep <= bp), (f"{tag}: branch vs the oracle, worst excess "
                              f"{float(np.max(ep - bp)):.3e}")
    return float(np.max(ec)) / max(rms(c), 1e-30), float(np.max(ep)) / max(rms(p), 1e-30)


def check_layer(cfg, wts, mk_cache, host_k, host_v, x_in, got, gpu, gpu_k, gpu_v, pos,
                slot_row, tag, wo_abs=None):
    """Every check of one layer's output on its input x_in ([m][D]):

    * stage by stage on the GPU's own intermediates (gpu: dict with xn, xq,
      q, k, v, attn, aq, [m][...] arrays read from the workspace): xn within
      1e-5 of the oracle's RMSNorm of x_in, xq and aq bytes exactly the
      oracle quantizer's on the GPU's fp32, q/k/v within 1e-5 of the oracle
      projections + RoPE of the GPU's xq, attention within 1e-4 of the
      oracle's on the GPU's q and cache, the O projection within 1e-5 of the
      branch plus two ulps of the output;
    * the plain oracle on x_in: out within 2e-3 x RMS, the attention output
      within 2e-3, xq codes differing only by boundary flips;
    * the branch against the conditioned and the plain oracle (module doc);
    * the cache: only the appended slots changed, each holding exactly the
      layer's k, v (slot_row(s, g) gives the flat element offset).

    mk_cache(k, v) builds an oracle.Cache over the given arrays; host_k/v are
    the cache contents before the layer ran; gpu_k/v after. Returns a dict of
    counts and relative errors."""
    m, D, H, KV, hd = cfg.m, cfg.D, cfg.H, cfg.KV, cfg.hd
    dims = dict(D=D, H=H, KV=KV, hd=hd, m=m, eps=cfg.eps)
    if wo_abs is None:
        wo_abs = abs_q5_matrix(wts["wo"], D, H * hd)
    gcache = mk_cache(gpu_k, gpu_v)
    for s in range(m):
        xs = x_in[s]
        assert_close_rms(gpu["xn"][s], oracle.rmsnorm(xs, wts["gamma"], cfg.eps), 1e-5,
                         tag + " xn")
        assert np.array_equal(gpu["xq"][s], oracle.quantize_q8_0(gpu["xn"][s])), tag + " xq bytes"
        q0 = oracle.gemv_q5_0(wts["wq"], gpu["xq"][s], wts["bq"], None, H * hd, D)
        k0 = oracle.gemv_q5_0(wts["wk"], gpu["xq"][s], wts["bk"], None, KV * hd, D)
        v0 = oracle.gemv_q8_0(wts["wv"], gpu["xq"][s], wts["bv"], None, KV * hd, D)
        q1, k1 = oracle.rope(q0, k0, wts["rope_cos"], wts["rope_sin"], pos[s], H, KV, hd)
        assert_close_rms(gpu["q"][s], q1, 1e-5, tag + " q")
        assert_close_rms(gpu["k"][s], k1, 1e-5, tag + " k")
        assert_close_rms(gpu["v"][s], v0, 1e-5, tag + " v")
        a0 = oracle.attention(gpu["q"][s], gcache, s, pos[s] + 1, H)
        assert_close_rms(gpu["attn"][s], a0, 1e-4, tag + " attention")
        assert np.array_equal(gpu["aq"][s], oracle.quantize_q8_0(gpu["attn"][s])), \
            tag + " aq bytes"
        o0 = oracle.gemv_q5_0(wts["wo"], gpu["aq"][s], wts["bo"], xs, D, H * hd)
        bound = 1e-5 * rms(o0.astype(np.float64) - xs) + 2 * np.spacing(np.abs(o0))
        assert np.all(np.abs(got[s].astype(np.float64) - o0) <= bound), tag + " O projection"

    # the plain oracle on the same input, and the one conditioned on the
    # GPU's xq codes
    ref, tr = oracle.decode_layer(dims, wts, mk_cache(host_k.copy(), host_v.copy()), x_in, x_in,
                                  pos, trace=True)
    assert_close_rms(got, ref, TOL, tag + " out")
    cc = mk_cache(host_k.copy(), host_v.copy())
    nx = na = 0
    errs = []
    for s in range(m):
        nx += check_flips(gpu["xq"][s], tr["xq"][s], gpu["xn"][s], tr["xn"][s], tag + " xq")
        assert_close_rms(gpu["attn"][s], tr["attn"][s], TOL, tag + " attention (independent)")
        cond = oracle_from_xq(dims, wts, cc, x_in[s], gpu["xq"][s], s, pos[s])
        na += check_flips(gpu["aq"][s], cond["aq"], gpu["attn"][s], cond["attn"], tag + " aq")
        errs.append(branch_bound_check(got[s], x_in[s], cond["out"], ref[s], gpu["aq"][s],
                                       cond["aq"], wo_abs, f"{tag} s={s}"))

    # the cache: only the appended slots changed; they hold the layer's k, v
    changed_k = ~((gpu_k == host_k) | (np.isnan(gpu_k) & np.isnan(host_k)))
    changed_v = ~((gpu_v == host_v) | (np.isnan(gpu_v) & np.isnan(host_v)))
    expect = np.zeros(host_k.size, bool)
    for s in range(m):
        for g in range(KV):
            r = slot_row(s, g)
            expect[r:r + hd] = True
            assert np.array_equal(gpu_k.reshape(-1)[r:r + hd].view(np.uint32),
                                  gpu["k"][s, g * hd:(g + 1) * hd].view(np.uint32)), tag + " k slot"
            assert np.array_equal(gpu_v.reshape(-1)[r:r + hd].view(np.uint32),
                                  gpu["v"][s, g * hd:(g + 1) * hd].view(np.uint32)), tag + " v slot"
    assert not np.any(changed_k.reshape(-1) & ~expect), tag + ": a k slot other than the appended one changed"
    assert not np.any(changed_v.reshape(-1) & ~expect), tag + ": a v slot other than the appended one changed"
    return dict(xq_flips=nx, aq_flips=na, branch_cond=max(e[0] for e in errs),
                branch_pure=max(e[1] for e in errs))


# ------------------------------------------------------- oracle chains -----
def nudged_floor(layer_fn, x0, nlayers, seeds=(1234, 4321)):
    """How far the oracle's own chain moves when every layer input is nudged
    by +-1 ulp (the size of fp32 reassociation): the largest relative
    deviation over the seeds. layer_fn(l, x) runs oracle layer l."""
    clean = x0.copy()
    for l in range(nlayers):
        clean = layer_fn(l, clean)
    worst = 0.0
    for seed in seeds:
        g = np.random.default_rng(seed)
        x = x0.copy()
        for l in range(nlayers):
            up = g.random(x.shape) < 0.5
            x = np.where(up, np.nextafter(x, np.float32(np.inf)),
                         np.nextafter(x, np.float32(-np.inf))).astype(np.float32)
            x = layer_fn(l, x)
        worst = max(worst, float(np.max(np.abs(x.astype(np.float64) - clean))) / rms(clean))
    return worst, clean


class OracleLoop:
    """The oracle's decode loop over a stack of layers with caches of its own
    (copies of the initial caches, appended to at every step), so that a GPU
    loop over several tokens is compared with an independent computation at
    every step. Layer l reads its cache through mk_cache(l, k, v)."""

    def __init__(self, cfg, layers_host, cos, sin, mk_cache):
        self.cfg = cfg
        self.dims = dict(D=cfg.D, H=cfg.H, KV=cfg.KV, hd=cfg.hd, m=cfg.m, eps=cfg.eps)
        self.wts = [dict(h, rope_cos=cos, rope_sin=sin) for h in layers_host]
        self.caches = [mk_cache(l, h["k"].copy(), h["v"].copy())
                       for l, h in enumerate(layers_host)]
        self.mk_cache = mk_cache

    def step(self, x0, pos):
        """Runs every layer at positions pos (appending to the oracle's
        caches); returns the output and the oracle's +-1-ulp noise floor of
        this step (0 for one layer), measured on copies of the caches."""
        n = len(self.caches)
        floor = 0.0
        if n > 1:
            snap = [(c.k.copy(), c.v.copy()) for c in self.caches]

            def layer_fn(l, x):
                return oracle.decode_layer(self.dims, self.wts[l],
                                           self.mk_cache(l, snap[l][0].copy(), snap[l][1].copy()),
                                           x, x, pos)
            floor, _ = nudged_floor(layer_fn, np.asarray(x0, np.float32), n, seeds=(77,))
        x = np.asarray(x0, np.float32).copy()
        for l in range(n):
            x = oracle.decode_layer(self.dims, self.wts[l], self.caches[l], x, x, pos)
        return x, floor
