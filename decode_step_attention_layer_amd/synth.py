"""Seeded synthetic inputs for the decode-step attention layer.

This module is shared by the tests, the benchmark and the smoke check. It only
draws numbers and lays them out in the input formats; it computes nothing the
layer computes. Weights are drawn in fp32 and turned into block bytes here,
because the layer consumes already-quantized weights: that conversion is data
preparation (a plain numpy rule, round-half-even), not the layer's Q8_0
activation quantizer.

Workloads (one per configuration; all values N(0,1) unless stated):
  c1  tiny: D=256, H=4, KV=2, hd=64, capacity 64, 16 prior tokens, pos 16,
      RoPE theta 1e4, one layer.
  c2  Qwen2-0.5B-shaped: D=896, H=14, KV=2, hd=64, capacity 2048, 1024 prior
      tokens, pos 1024, theta 1e4, 24 stacked layers.
  c3  7B-shaped: D=3584, H=28, KV=4, hd=128, capacity 8192, 4096 prior tokens,
      pos 4096, theta 1e4, 28 stacked layers.
  c4  long context: D=4096, H=32, KV=8, hd=128, capacity 33024, 32768 prior
      tokens, pos 32768, theta 5e5, one layer.
  c5  batched: c4's shape, m=8 sequences, paged cache with 16-token pages and a
      shuffled page table, per-sequence context L_s ~ U{512..8192}, pos_s = L_s,
      theta 5e5, one layer.
Weights ~ N(0, 0.02) before quantization, biases ~ N(0, 0.02), gamma ~ N(1, 0.1),
eps = 1e-6. Seeds: numpy default_rng(SeedSequence([config, layer, tensor])).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QK = 32
Q8_0_BYTES = 34
Q5_0_BYTES = 22

# tensor ids in the seed sequence
T_X, T_GAMMA, T_BQ, T_BK, T_BV, T_BO, T_WQ, T_WK, T_WV, T_WO = range(10)
T_KCACHE, T_VCACHE, T_LENS, T_PERM = 10, 11, 12, 13
T_KCODES, T_VCODES = 14, 15
T_KRING, T_VRING = 16, 17
T_SEL, T_SINK = 18, 19
SEL_WINDOW = 128               # selections: the last tokens, then index picks

# Reduced-precision caches: element types (the C ABI's CK_KV_*) and the fixed
# per-tensor scales of the synthetic fp8 caches.
KV_F32, KV_BF16, KV_FP8 = 0, 1, 2
FP8_K_SCALE, FP8_V_SCALE = 0.25, 0.5
KV_ELEM_BYTES = {KV_F32: 4, KV_BF16: 2, KV_FP8: 1}


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    D: int
    H: int
    KV: int
    hd: int
    theta: float
    layers: int = 1
    m: int = 1
    capacity: int = 0          # contiguous cache tokens per sequence
    pos: int = 0               # contiguous: the decode position (= prior tokens)
    page_size: int = 0         # > 0: paged cache
    min_ctx: int = 0           # paged: L_s ~ U{min_ctx..max_ctx}
    max_ctx: int = 0
    eps: float = 1e-6

    @property
    def G(self) -> int:
        return self.H // self.KV

    @property
    def max_pages_per_seq(self) -> int:
        return -(-(self.max_ctx + 1) // self.page_size) if self.page_size else 0

    @property
    def rope_rows(self) -> int:
        return self.max_pages_per_seq * self.page_size if self.page_size else self.capacity


CONFIGS = {
    "c1": Config("c1", 0, 256, 4, 2, 64, 1e4, layers=1, capacity=64, pos=16),
    "c2": Config("c2", 1, 896, 14, 2, 64, 1e4, layers=24, capacity=2048, pos=1024),
    "c3": Config("c3", 2, 3584, 28, 4, 128, 1e4, layers=28, capacity=8192, pos=4096),
    "c4": Config("c4", 3, 4096, 32, 8, 128, 5e5, layers=1, capacity=33024, pos=32768),
    "c5": Config("c5", 4, 4096, 32, 8, 128, 5e5, layers=1, m=8, page_size=16,
                 min_ctx=512, max_ctx=8192),
}


def rng(cfg_index: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_index, layer, tensor]))


def normal(g: np.random.Generator, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


# ----------------------------------------------------------- block packing --
def pack_q5_0(codes: np.ndarray, scales16: np.ndarray) -> np.ndarray:
    """codes uint8 [rows, nb, 32] in 0..31, scales fp16 [rows, nb] -> bytes
    [rows, nb*22]: fp16 d | qh (bit j = code_j >> 4, little-endian) | qs
    (byte j = low nibble of code j | low nibble of code j+16 << 4)."""
    rows, nb, _ = codes.shape
    lo = codes & 0x0F
    hi = ((codes >> 4) & 1).astype(np.uint32)
    qs = lo[..., :16] | (lo[..., 16:] << 4)
    qh = np.bitwise_or.reduce(hi << np.arange(32, dtype=np.uint32), axis=2).astype("<u4")
    out = np.empty((rows, nb, Q5_0_BYTES), np.uint8)
    out[..., 0:2] = np.ascontiguousarray(scales16.astype("<f2")).view(np.uint8).reshape(rows, nb, 2)
    out[..., 2:6] = np.ascontiguousarray(qh).view(np.uint8).reshape(rows, nb, 4)
    out[..., 6:22] = qs
    return out.reshape(rows, nb * Q5_0_BYTES)


def pack_q8_0(codes: np.ndarray, scales16: np.ndarray) -> np.ndarray:
    """codes int8 [rows, nb, 32], scales fp16 [rows, nb] -> bytes [rows, nb*34]."""
    rows, nb, _ = codes.shape
    out = np.empty((rows, nb, Q8_0_BYTES), np.uint8)
    out[..., 0:2] = np.ascontiguousarray(scales16.astype("<f2")).view(np.uint8).reshape(rows, nb, 2)
    out[..., 2:] = codes.astype(np.int8).view(np.uint8)
    return out.reshape(rows, nb * Q8_0_BYTES)


def weights_to_q5_0(W: np.ndarray):
    """Test-data conversion of fp32 weights [rows, K] to Q5_0 bytes. Per block
    the element of largest magnitude sets the scale d = that element / -16, so
    it maps to code 0; codes = clip(rint(w / d) + 16, 0, 31). Returns
    (bytes, codes, fp16 scales)."""
    rows, K = W.shape
    B = W.reshape(rows, K // QK, QK)
    idx = np.argmax(np.abs(B), axis=2)
    mv = np.take_along_axis(B, idx[..., None], axis=2)[..., 0]
    d = (mv / np.float32(-16.0)).astype(np.float32)
    safe = np.where(d == 0, np.float32(1), d)
    t = np.where(d[..., None] == 0, np.float32(0), B / safe[..., None])
    codes = np.clip(np.rint(t) + 16, 0, 31).astype(np.uint8)
    s16 = d.astype(np.float16)
    return pack_q5_0(codes, s16), codes, s16


def weights_to_q8_0(W: np.ndarray):
    """Test-data conversion of fp32 weights [rows, K] to Q8_0 bytes: d = absmax
    / 127, codes = clip(rint(w / d), -127, 127). Returns (bytes, codes, scales)."""
    rows, K = W.shape
    B = W.reshape(rows, K // QK, QK)
    d = (np.abs(B).max(axis=2) / np.float32(127.0)).astype(np.float32)
    safe = np.where(d == 0, np.float32(1), d)
    t = np.where(d[..., None] == 0, np.float32(0), B / safe[..., None])
    codes = np.clip(np.rint(t), -127, 127).astype(np.int8)
    s16 = d.astype(np.float16)
    return pack_q8_0(codes, s16), codes, s16


def rope_tables(rows: int, hd: int, theta: float):
    """cos/sin tables [rows][hd/2] fp32 for angle(p, i) = p * theta^(-2i/hd),
    evaluated in float64."""
    i = np.arange(hd // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / hd)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


# ---------------------------------------------------------------- layers ----
def layer_weights(cfg: Config, layer: int, keep_codes: bool = False) -> dict:
    """Quantized weights, biases and gamma of one layer of `cfg`."""
    D, H, KV, hd = cfg.D, cfg.H, cfg.KV, cfg.hd
    HD, KD = H * hd, KV * hd
    c, L = cfg.index, layer
    w = {}
    wq, cq, sq = weights_to_q5_0(normal(rng(c, L, T_WQ), (HD, D), 0.02))
    wk, ck, sk = weights_to_q5_0(normal(rng(c, L, T_WK), (KD, D), 0.02))
    wv, cv, sv = weights_to_q8_0(normal(rng(c, L, T_WV), (KD, D), 0.02))
    wo, co, so = weights_to_q5_0(normal(rng(c, L, T_WO), (D, HD), 0.02))
    w.update(wq=wq, wk=wk, wv=wv, wo=wo)
    if keep_codes:
        w.update(wq_codes=cq, wq_scales=sq, wk_codes=ck, wk_scales=sk,
                 wv_codes=cv, wv_scales=sv, wo_codes=co, wo_scales=so)
    w["gamma"] = normal(rng(c, L, T_GAMMA), D, 0.1, 1.0)
    w["bq"] = normal(rng(c, L, T_BQ), HD, 0.02)
    w["bk"] = normal(rng(c, L, T_BK), KD, 0.02)
    w["bv"] = normal(rng(c, L, T_BV), KD, 0.02)
    w["bo"] = normal(rng(c, L, T_BO), D, 0.02)
    return w


def token_input(cfg: Config) -> np.ndarray:
    """x [m][D] for the first layer; the residual input is x itself."""
    return normal(rng(cfg.index, 0, T_X), (cfg.m, cfg.D))


def context_lengths(cfg: Config) -> np.ndarray:
    """Prior tokens per sequence (= the decode position of each sequence)."""
    if cfg.page_size == 0:
        return np.full(cfg.m, cfg.pos, np.int32)
    g = rng(cfg.index, 0, T_LENS)
    return g.integers(cfg.min_ctx, cfg.max_ctx + 1, size=cfg.m).astype(np.int32)


def contiguous_cache(cfg: Config, layer: int, poison: float = float("nan")):
    """K and V [m][KV][capacity][hd]: tokens < pos ~ N(0,1), the rest `poison`."""
    shape = (cfg.m, cfg.KV, cfg.capacity, cfg.hd)
    out = []
    for tid in (T_KCACHE, T_VCACHE):
        a = np.full(shape, poison, np.float32)
        a[:, :, : cfg.pos, :] = normal(rng(cfg.index, layer, tid), (cfg.m, cfg.KV, cfg.pos, cfg.hd))
        out.append(a)
    return out[0], out[1]


def ring_cache(cfg: Config, layer: int, slots: int, poison: float = float("nan")):
    """K and V of a ring of `slots` tokens per (sequence, KV head):
    [m][KV][slots][hd]. A ring past its first lap holds `slots` earlier tokens
    in some order, so every slot is ~ N(0,1); before it (pos < slots) only
    slots < pos were written and the rest hold `poison`."""
    shape = (cfg.m, cfg.KV, slots, cfg.hd)
    out = []
    for tid in (T_KRING, T_VRING):
        a = normal(rng(cfg.index, layer, tid), shape)
        if cfg.pos < slots:
            a[:, :, cfg.pos:, :] = poison
        out.append(a)
    return out[0], out[1]


def selection(cfg: Config, layer: int, topk: int, lens=None) -> np.ndarray:
    """Sparse-attention selections [m][topk] int32, shaped like a sliding
    window plus an index's picks: per sequence of L prior tokens (attending
    L + 1 with the appended one) the last min(SEL_WINDOW, L + 1) positions,
    then distinct earlier positions drawn uniformly, up to topk entries in
    all, then -1."""
    if lens is None:
        lens = context_lengths(cfg)
    g = rng(cfg.index, layer, T_SEL)
    out = np.full((len(lens), topk), -1, np.int32)
    for s, L in enumerate(lens):
        n = int(L) + 1
        w = min(SEL_WINDOW, n, topk)
        win = np.arange(n - w, n, dtype=np.int32)
        k = min(topk - w, n - w)
        picks = g.choice(n - w, size=k, replace=False).astype(np.int32) if k > 0 else []
        row = np.concatenate([win, picks]).astype(np.int32)
        out[s, :row.size] = row
    return out


def sink_logits(cfg: Config, layer: int) -> np.ndarray:
    """Per-head attention-sink logits [H] ~ N(0, 1)."""
    return normal(rng(cfg.index, layer, T_SINK), (cfg.H,))


def paged_cache(cfg: Config, layer: int, poison: float = float("nan"), spare_pages: int = 0):
    """Paged K and V pools [P][KV][page][hd], the page table [m][max_pages]
    (int32, -1 = unmapped) and the context lengths. Sequence s owns
    ceil((L_s + 1) / page) pages (room for the appended token); physical ids are
    a seeded permutation, assigned in logical order. Slots at or past L_s and
    the `spare_pages` unused pages hold `poison`."""
    ps, KV, hd = cfg.page_size, cfg.KV, cfg.hd
    lens = context_lengths(cfg)
    npages = [-(-(int(L) + 1) // ps) for L in lens]
    P = sum(npages) + spare_pages
    perm = rng(cfg.index, layer, T_PERM).permutation(P).astype(np.int32)
    table = np.full((cfg.m, cfg.max_pages_per_seq), -1, np.int32)
    k = np.full((P, KV, ps, hd), poison, np.float32)
    v = np.full((P, KV, ps, hd), poison, np.float32)
    gk, gv = rng(cfg.index, layer, T_KCACHE), rng(cfg.index, layer, T_VCACHE)
    nxt = 0
    for s, L in enumerate(lens):
        L = int(L)
        ids = perm[nxt: nxt + npages[s]]
        nxt += npages[s]
        table[s, : npages[s]] = ids
        ks = normal(gk, (L, KV, hd))
        vs = normal(gv, (L, KV, hd))
        for lp, page in enumerate(ids):
            t0, t1 = lp * ps, min(L, (lp + 1) * ps)
            if t1 > t0:
                k[page, :, : t1 - t0, :] = ks[t0:t1].transpose(1, 0, 2)
                v[page, :, : t1 - t0, :] = vs[t0:t1].transpose(1, 0, 2)
    return k, v, table, lens


def cache_codes(values: np.ndarray, kv_dtype: int, cfg_index: int, layer: int,
                is_k: bool) -> np.ndarray:
    """Synthetic cache contents of a reduced-precision cache, built from the
    fp32 cache `values` (NaN marks poisoned slots). bf16: the upper half of
    each fp32 value (truncation, a plain bit extraction; NaN stays NaN); fp8:
    random E4M3 codes of magnitude 2^-3..7.5 with random signs, drawn from a
    stream of their own, and the NaN code 0x7F where the fp32 cache is
    poisoned. Test data only: the store rule under test is not involved."""
    if kv_dtype == KV_F32:
        return values
    if kv_dtype == KV_BF16:
        return (np.ascontiguousarray(values, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    g = rng(cfg_index, layer, T_KCODES if is_k else T_VCODES)
    exp_field = g.integers(4, 10, size=values.shape, dtype=np.uint8)     # 2^-3 .. 2^2
    mant = g.integers(0, 8, size=values.shape, dtype=np.uint8)
    sign = (g.integers(0, 2, size=values.shape, dtype=np.uint8) << 7).astype(np.uint8)
    codes = (sign | (exp_field << 3) | mant).astype(np.uint8)
    codes[np.isnan(values)] = 0x7F
    return codes


def rope_for(cfg: Config):
    return rope_tables(cfg.rope_rows, cfg.hd, cfg.theta)


def algorithmic_bytes(cfg: Config, lens=None, kv_dtype: int = KV_F32, window: int = 0,
                      topk: int = 0) -> dict:
    """Bytes one layer step must move: quantized weight blocks + K and V of
    every attended token (L = pos + 1 per sequence, at most `window` of them
    under a sliding window, min(L, topk) under a selection of topk entries)
    in the cache's type."""
    D, HD, KD = cfg.D, cfg.H * cfg.hd, cfg.KV * cfg.hd
    w = (HD * D // QK) * Q5_0_BYTES + (KD * D // QK) * Q5_0_BYTES \
        + (KD * D // QK) * Q8_0_BYTES + (D * HD // QK) * Q5_0_BYTES
    if lens is None:
        lens = context_lengths(cfg)
    att = np.asarray(lens, np.int64) + 1
    if window > 0:
        att = np.minimum(att, window)
    if topk > 0:
        att = np.minimum(att, topk)
    tokens = int(np.sum(att))
    kv = tokens * KD * KV_ELEM_BYTES[kv_dtype] * 2
    return {"weights": w, "kv": kv, "total": w + kv}


def seeded_vector(seed: int, n: int, std: float = 1.0) -> np.ndarray:
    return normal(np.random.default_rng(seed), n, std)

