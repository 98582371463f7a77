"""Python access to the C oracle of the decode-step attention layer.

TEST INFRASTRUCTURE ONLY. The oracle is the checker for the HIP path: only the
tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this module. The product path never does, and shares no code with it.

The C library (``oracle.c``) is a plain, single-threaded model of the layer on
the C-Kernel-Engine page "mega_fused_attention_decode_q5_0.c" (MAIN KERNEL,
steps 1-8), with the paged cache of the metrale page "prefill_attn_a.rs"
(``paged_decode_attn_*``). This module only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")

QK = 32
Q8_0_BYTES = 34
Q5_0_BYTES = 22


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, no contraction, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= max(
        os.path.getmtime(_SRC), os.path.getmtime(_HDR)
    ):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
        "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        f = ctypes.c_float
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = f
        L.orc_f32_to_f16.argtypes = [f]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_dequantize_q8_0.argtypes = [P, P, i]
        L.orc_dequantize_q5_0.argtypes = [P, P, i]
        L.orc_rmsnorm.argtypes = [P, P, P, i, f]
        L.orc_quantize_q8_0.argtypes = [P, P, i]
        L.orc_gemv_q5_0.argtypes = [P, P, P, P, P, i, i]
        L.orc_gemv_q8_0.argtypes = [P, P, P, P, P, i, i]
        L.orc_rope.argtypes = [P, P, P, P, i, i, i, i]
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = f
        L.orc_f32_to_bf16.argtypes = [f]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_f32.restype = f
        L.orc_f32_to_e4m3.argtypes = [f]
        L.orc_f32_to_e4m3.restype = ctypes.c_uint8
        L.orc_kv_append.argtypes = [ctypes.POINTER(OrcCache), i, i, P, P]
        L.orc_kv_append.restype = i
        L.orc_attention.argtypes = [P, ctypes.POINTER(OrcCache), i, i, i, P, P]
        L.orc_attention.restype = i
        L.orc_decode_layer.argtypes = [
            ctypes.POINTER(OrcDims), ctypes.POINTER(OrcWeights), ctypes.POINTER(OrcCache),
            P, P, P, P, ctypes.POINTER(OrcTrace),
        ]
        L.orc_decode_layer.restype = i
        L.orc_attention_sparse.argtypes = [P, ctypes.POINTER(OrcCache), i, i, i, P, i, P, P]
        L.orc_attention_sparse.restype = i
        L.orc_decode_layer_sparse.argtypes = [
            ctypes.POINTER(OrcDims), ctypes.POINTER(OrcWeights), ctypes.POINTER(OrcCache),
            P, P, P, P, i, P, P, ctypes.POINTER(OrcTrace),
        ]
        L.orc_decode_layer_sparse.restype = i
        _lib = L
    return _lib


class OrcCache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
        ("capacity", ctypes.c_int), ("page_size", ctypes.c_int),
        ("page_table", ctypes.c_void_p),
        ("max_pages_per_seq", ctypes.c_int), ("num_pages", ctypes.c_int),
        ("dtype", ctypes.c_int), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("ring", ctypes.c_int), ("window", ctypes.c_int),
    ]


KV_F32, KV_BF16, KV_FP8_E4M3 = 0, 1, 2
_KV_NP = {KV_F32: np.float32, KV_BF16: np.uint16, KV_FP8_E4M3: np.uint8}


class OrcDims(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int), ("H", ctypes.c_int), ("KV", ctypes.c_int),
                ("hd", ctypes.c_int), ("m", ctypes.c_int), ("eps", ctypes.c_float)]


class OrcWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("wq", "wk", "wv", "wo", "bq", "bk", "bv", "bo", "gamma",
                 "rope_cos", "rope_sin")] + [("rope_rows", ctypes.c_int)]


class OrcTrace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("xn", "xq", "q_pre", "k_pre", "q", "k", "v", "attn", "aq")]


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------- codec ----
def f16_to_f32(bits: int) -> float:
    return lib().orc_f16_to_f32(int(bits))


def f32_to_f16(x: float) -> int:
    return int(lib().orc_f32_to_f16(float(np.float32(x))))


# ---------------------------------------------------------------- steps ----
def dequantize_q8_0(blocks: np.ndarray, K: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    out = np.empty(K, np.float32)
    lib().orc_dequantize_q8_0(_p(blocks), _p(out), K)
    return out


def dequantize_q5_0(blocks: np.ndarray, K: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    out = np.empty(K, np.float32)
    lib().orc_dequantize_q5_0(_p(blocks), _p(out), K)
    return out


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    x, gamma = _f32(x), _f32(gamma)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(gamma), _p(y), x.shape[-1], eps)
    return y


def quantize_q8_0(x) -> np.ndarray:
    """fp32 [K] -> uint8 [K/32*34]."""
    x = _f32(x)
    K = x.shape[-1]
    assert K % QK == 0
    out = np.empty(K // QK * Q8_0_BYTES, np.uint8)
    lib().orc_quantize_q8_0(_p(x), _p(out), K)
    return out


def _gemv(fn, W, xq, bias, residual, rows, K):
    W = np.ascontiguousarray(W, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    bias = None if bias is None else _f32(bias)
    residual = None if residual is None else _f32(residual)
    y = np.empty(rows, np.float32)
    fn(_p(W), _p(xq), _p(bias), _p(residual), _p(y), rows, K)
    return y


def gemv_q5_0(W, xq, bias, residual, rows: int, K: int) -> np.ndarray:
    return _gemv(lib().orc_gemv_q5_0, W, xq, bias, residual, rows, K)


def gemv_q8_0(W, xq, bias, residual, rows: int, K: int) -> np.ndarray:
    return _gemv(lib().orc_gemv_q8_0, W, xq, bias, residual, rows, K)


def rope(q, k, cos_tab, sin_tab, pos: int, H: int, KV: int, hd: int):
    """Returns rotated copies of q [H*hd] and k [KV*hd] (either may be None)."""
    q = None if q is None else _f32(q).copy()
    k = None if k is None else _f32(k).copy()
    cos_tab, sin_tab = _f32(cos_tab), _f32(sin_tab)
    lib().orc_rope(_p(q), _p(k), _p(cos_tab), _p(sin_tab), pos, H, KV, hd)
    return q, k


@dataclass
class Cache:
    """KV cache arrays in the oracle's layout (contiguous or paged)."""
    k: np.ndarray
    v: np.ndarray
    kv_heads: int
    head_dim: int
    capacity: int = 0
    page_size: int = 0
    page_table: np.ndarray | None = None
    max_pages_per_seq: int = 0
    num_pages: int = 0
    dtype: int = KV_F32            # KV_F32 (float32 arrays), KV_BF16 (uint16), KV_FP8_E4M3 (uint8)
    k_scale: float = 1.0
    v_scale: float = 1.0
    ring: bool = False             # contiguous only: token t lives in slot t % capacity
    window: int = 0                # > 0: attention reads only the last `window` tokens

    def c(self) -> OrcCache:
        want = _KV_NP[self.dtype]
        assert self.k.dtype == want and self.v.dtype == want
        assert self.k.flags["C_CONTIGUOUS"] and self.v.flags["C_CONTIGUOUS"]
        if self.page_table is not None:
            assert self.page_table.dtype == np.int32 and self.page_table.flags["C_CONTIGUOUS"]
        self._keep = OrcCache(
            _p(self.k), _p(self.v), self.kv_heads, self.head_dim, self.capacity,
            self.page_size, _p(self.page_table), self.max_pages_per_seq, self.num_pages,
            self.dtype, self.k_scale, self.v_scale, int(self.ring), int(self.window),
        )
        return self._keep


def kv_append(cache: Cache, seq: int, pos: int, k, v) -> None:
    k, v = _f32(k), _f32(v)
    cc = cache.c()
    rc = lib().orc_kv_append(ctypes.byref(cc), seq, pos, _p(k), _p(v))
    if rc:
        raise ValueError("oracle kv_append: token has no valid home")


def attention(q, cache: Cache, seq: int, L: int, H: int, want_probs: bool = False):
    q = _f32(q)
    out = np.empty(H * cache.head_dim, np.float32)
    probs = np.empty(H * L, np.float64) if want_probs else None
    cc = cache.c()
    rc = lib().orc_attention(_p(q), ctypes.byref(cc), seq, L, H, _p(out), _p(probs))
    if rc:
        raise ValueError("oracle attention: unmapped page or bad length")
    if want_probs:
        return out, probs.reshape(H, L)
    return out


def attention_sparse(q, cache: Cache, seq: int, L: int, H: int, sel, sink=None):
    """Attention of one sequence over the selected token positions `sel`
    (-1 = absent), with per-head sink logits joining the denominator."""
    q = _f32(q)
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(-1)
    sink = None if sink is None else _f32(sink)
    out = np.empty(H * cache.head_dim, np.float32)
    cc = cache.c()
    rc = lib().orc_attention_sparse(_p(q), ctypes.byref(cc), seq, L, H, _p(sel), sel.size,
                                    _p(sink), _p(out))
    if rc:
        raise ValueError("oracle sparse attention: entry past the sequence or not held")
    return out


def decode_layer(dims: dict, weights: dict, cache: Cache, x, residual, pos, trace: bool = False,
                 sel=None, sink=None):
    """One decode step of the layer for m tokens. Mutates the cache (append).
    With sel ([m][topk] token positions, -1 = absent) the attention is the
    sparse one over that selection, with sink logits [H] (or none).

    dims: D, H, KV, hd, m, eps. weights: wq, wk, wv, wo (uint8 block bytes),
    bq, bk, bv, bo, gamma (fp32, biases may be None), rope_cos, rope_sin
    ([rows][hd/2] fp32). Returns out [m][D] (and a dict of intermediates).
    """
    D, H, KV, hd, m = dims["D"], dims["H"], dims["KV"], dims["hd"], dims["m"]
    od = OrcDims(D, H, KV, hd, m, dims["eps"])
    keep = {}

    def u8(name):
        a = np.ascontiguousarray(weights[name], dtype=np.uint8)
        keep[name] = a
        return _p(a)

    def f32(name):
        if weights.get(name) is None:
            return None
        a = _f32(weights[name])
        keep[name] = a
        return _p(a)

    ow = OrcWeights(u8("wq"), u8("wk"), u8("wv"), u8("wo"), f32("bq"), f32("bk"),
                    f32("bv"), f32("bo"), f32("gamma"), f32("rope_cos"), f32("rope_sin"),
                    int(np.asarray(weights["rope_cos"]).shape[0]))
    x = _f32(x).reshape(m, D)
    residual = None if residual is None else _f32(residual).reshape(m, D)
    pos = np.ascontiguousarray(pos, dtype=np.int32).reshape(m)
    out = np.empty((m, D), np.float32)
    tr = None
    bufs = {}
    if trace:
        nbD = D // QK * Q8_0_BYTES
        nbA = H * hd // QK * Q8_0_BYTES
        bufs = dict(
            xn=np.empty((m, D), np.float32), xq=np.empty((m, nbD), np.uint8),
            q_pre=np.empty((m, H * hd), np.float32), k_pre=np.empty((m, KV * hd), np.float32),
            q=np.empty((m, H * hd), np.float32), k=np.empty((m, KV * hd), np.float32),
            v=np.empty((m, KV * hd), np.float32), attn=np.empty((m, H * hd), np.float32),
            aq=np.empty((m, nbA), np.uint8),
        )
        tr = OrcTrace(*[_p(bufs[n]) for n in
                        ("xn", "xq", "q_pre", "k_pre", "q", "k", "v", "attn", "aq")])
    cc = cache.c()
    if sel is None:
        rc = lib().orc_decode_layer(ctypes.byref(od), ctypes.byref(ow), ctypes.byref(cc),
                                    _p(x), _p(residual), _p(pos), _p(out),
                                    ctypes.byref(tr) if tr is not None else None)
    else:
        sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(m, -1)
        sink = None if sink is None else _f32(sink)
        rc = lib().orc_decode_layer_sparse(ctypes.byref(od), ctypes.byref(ow), ctypes.byref(cc),
                                           _p(x), _p(residual), _p(pos), _p(sel), sel.shape[1],
                                           _p(sink), _p(out),
                                           ctypes.byref(tr) if tr is not None else None)
    if rc:
        raise ValueError("oracle decode_layer: bad argument, position or page")
    return (out, bufs) if trace else out


# ---- cache element codecs ---------------------------------------------------
def bf16_to_f32(b: int) -> float:
    return lib().orc_bf16_to_f32(int(b))


def f32_to_bf16(x: float) -> int:
    return int(lib().orc_f32_to_bf16(float(x)))


def e4m3_to_f32(c: int) -> float:
    return lib().orc_e4m3_to_f32(int(c))


def f32_to_e4m3(x: float) -> int:
    return int(lib().orc_f32_to_e4m3(float(x)))


def encode_cache(values: np.ndarray, dtype: int, scale: float = 1.0) -> np.ndarray:
    """Cache elements of `dtype` for fp32 values (the oracle's store rule,
    element by element; fp8 stores fp32(x / scale))."""
    x = np.ascontiguousarray(values, np.float32).reshape(-1)
    if dtype == KV_F32:
        return x.copy().reshape(values.shape)
    if dtype == KV_BF16:
        out = np.array([f32_to_bf16(v) for v in x], np.uint16)
    else:
        sc = np.float32(scale)
        out = np.array([f32_to_e4m3(np.float32(v) / sc) for v in x], np.uint8)
    return out.reshape(values.shape)


def decode_cache(codes: np.ndarray, dtype: int, scale: float = 1.0) -> np.ndarray:
    """fp32 values of cache elements (fp8: fp32(code value * scale))."""
    c = np.ascontiguousarray(codes).reshape(-1)
    if dtype == KV_F32:
        return c.astype(np.float32).reshape(codes.shape)
    if dtype == KV_BF16:
        out = np.array([bf16_to_f32(v) for v in c], np.float32)
    else:
        sc = np.float32(scale)
        out = np.array([np.float32(e4m3_to_f32(v)) * sc for v in c], np.float32)
    return out.reshape(codes.shape)
