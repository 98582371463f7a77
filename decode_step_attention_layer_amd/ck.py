"""ctypes binding of libck.so (the C ABI in include/ck.h).

Argument marshalling only: every function forwards to the C entry point of
the same name. Tensors are torch CUDA tensors (their device pointers are
passed), host position arrays are sequences of ints, ``stream`` is a
torch.cuda.Stream, a raw hipStream_t handle, or None for torch's current
stream. A non-zero return code raises CkError. If libck.so is missing or
cannot be loaded, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libck.so")

CK_OK = 0
CK_EINVAL = -1
CK_ENOSPC = -2
CK_EUNSUPPORTED = -3
CK_EHIP = -4
CK_MAX_SEQS = 16
CK_VARIANT_CHAIN = 0
CK_VARIANT_FUSED = 1
CK_VARIANT_PERSISTENT = 2
CK_VARIANT_TWO_LAUNCH = 3
CK_MAX_STEP_LAYERS = 32
CK_KV_F32 = 0
CK_KV_BF16 = 1
CK_KV_FP8_E4M3 = 2

EXPORTS = (
    "ck_strerror", "ck_version", "ck_rmsnorm", "ck_quantize_q8_0", "ck_gemv_q5_0_q8_0",
    "ck_gemv_q8_0_q8_0", "ck_rope", "ck_kv_append", "ck_attn_workspace_size",
    "ck_attn_decode_gqa", "ck_attn_partial", "ck_attn_merge", "ck_decode_layer_workspace_size",
    "ck_decode_layer",
    "ck_decode_layer_ws_offset", "ck_decode_step_workspace_size", "ck_decode_step",
    "ck_decode_step_status_offset", "ck_decode_layer_devpos", "ck_decode_step_devpos",
    "ck_attn_sparse", "ck_decode_layer_sparse", "ck_decode_layer_noalloc",
    "ck_decode_layer_noalloc_limit", "ck_decode_layer_part", "ck_read_probe",
    "ck_decode_layer_attn_plan",
)


class CkError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} ({code})")
        self.code = code


class CkKVCache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("page_table", ctypes.c_void_p),
        ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("window", ctypes.c_int32), ("ring", ctypes.c_int32),
    ]


class CkLayerDesc(ctypes.Structure):
    _fields_ = [
        ("D", ctypes.c_int32), ("H", ctypes.c_int32), ("KV", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("m", ctypes.c_int32), ("eps", ctypes.c_float),
        ("variant", ctypes.c_int32), ("attn_chunk", ctypes.c_int32),
    ]


class CkLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("wq", "wk", "wv", "wo", "bq", "bk", "bv", "bo", "gamma", "rope_cos", "rope_sin")] + [
        ("rope_rows", ctypes.c_int32)]


_lib = None


def load():
    """Open libck.so (built in-tree by decode_step_attention_layer_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libck.so not built: {LIB_PATH} is missing "
                           "(run python -m decode_step_attention_layer_amd.build)")
    # torch first: libck.so then binds to the HIP runtime torch loaded, so that
    # both share one runtime (devices, streams, graph capture)
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    IP = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "ck_strerror": ([I], ctypes.c_char_p),
        "ck_version": ([], I),
        "ck_rmsnorm": ([P, P, P, I, I, F, P], I),
        "ck_quantize_q8_0": ([P, P, I, I, P], I),
        "ck_gemv_q5_0_q8_0": ([P, P, P, P, P, I, I, I, P], I),
        "ck_gemv_q8_0_q8_0": ([P, P, P, P, P, I, I, I, P], I),
        "ck_rope": ([P, P, P, P, I, IP, I, I, I, I, P], I),
        "ck_kv_append": ([ctypes.POINTER(CkKVCache), P, P, IP, I, P], I),
        "ck_attn_workspace_size": ([I, I, I, I, I, I], S),
        "ck_attn_decode_gqa": ([P, ctypes.POINTER(CkKVCache), IP, P, I, I, F, I, P, S, P], I),
        "ck_attn_partial": ([P, ctypes.POINTER(CkKVCache), IP, I, I, F, I, P, S, P], I),
        "ck_attn_merge": ([P, S, IP, I, I, I, I, I, I, P, P, P], I),
        "ck_decode_layer_workspace_size": ([ctypes.POINTER(CkLayerDesc), I], S),
        "ck_decode_layer": ([ctypes.POINTER(CkLayerDesc), ctypes.POINTER(CkLayerWeights),
                             ctypes.POINTER(CkKVCache), P, P, IP, P, P, S, P], I),
        "ck_read_probe": ([P, S, P, P], I),
        "ck_decode_layer_attn_plan": ([ctypes.POINTER(CkLayerDesc), ctypes.POINTER(CkKVCache),
                                       IP, I, IP, IP], I),
        "ck_decode_layer_part": ([ctypes.POINTER(CkLayerDesc), ctypes.POINTER(CkLayerWeights),
                                  ctypes.POINTER(CkKVCache), P, P, IP, P, P, S, I, P], I),
        "ck_decode_layer_noalloc": ([ctypes.POINTER(CkLayerDesc),
                                     ctypes.POINTER(CkLayerWeights), ctypes.POINTER(CkKVCache),
                                     P, P, IP, P, P], I),
        "ck_decode_layer_noalloc_limit": ([], S),
        "ck_decode_layer_ws_offset": ([ctypes.POINTER(CkLayerDesc), I, ctypes.c_char_p],
                                      ctypes.c_long),
        "ck_decode_step_workspace_size": ([ctypes.POINTER(CkLayerDesc), I, I], S),
        "ck_decode_step": ([ctypes.POINTER(CkLayerDesc), ctypes.POINTER(CkLayerWeights),
                            ctypes.POINTER(CkKVCache), I, P, IP, P, P, S, P], I),
        "ck_decode_step_status_offset": ([ctypes.POINTER(CkLayerDesc), I], ctypes.c_long),
        "ck_decode_layer_devpos": ([ctypes.POINTER(CkLayerDesc), ctypes.POINTER(CkLayerWeights),
                                    ctypes.POINTER(CkKVCache), P, P, P, I, P, P, S, P], I),
        "ck_decode_step_devpos": ([ctypes.POINTER(CkLayerDesc), ctypes.POINTER(CkLayerWeights),
                                   ctypes.POINTER(CkKVCache), I, P, P, I, P, P, S, P], I),
        "ck_attn_sparse": ([P, ctypes.POINTER(CkKVCache), IP, P, I, P, P, I, I, F, I, P, S, P], I),
        "ck_decode_layer_sparse": ([ctypes.POINTER(CkLayerDesc), ctypes.POINTER(CkLayerWeights),
                                    ctypes.POINTER(CkKVCache), P, P, IP, P, I, P, I, P, P, P, S,
                                    P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def strerror(code: int) -> str:
    return load().ck_strerror(int(code)).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libck takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libck takes contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _pos(pos):
    vals = [int(p) for p in pos]
    return (ctypes.c_int32 * max(1, len(vals)))(*vals)


def _check(rc: int, where: str):
    if rc != CK_OK:
        raise CkError(rc, where)


# ------------------------------------------------------------ entry points --
def ck_version() -> int:
    return load().ck_version()


def ck_rmsnorm(x, gamma, y, m, D, eps, stream=None):
    _check(load().ck_rmsnorm(_ptr(x), _ptr(gamma), _ptr(y), m, D, eps, _stream(stream)),
           "ck_rmsnorm")


def ck_quantize_q8_0(x, y, m, K, stream=None):
    _check(load().ck_quantize_q8_0(_ptr(x), _ptr(y), m, K, _stream(stream)), "ck_quantize_q8_0")


def ck_gemv_q5_0_q8_0(W, xq, bias, residual, y, rows, K, m, stream=None):
    _check(load().ck_gemv_q5_0_q8_0(_ptr(W), _ptr(xq), _ptr(bias), _ptr(residual), _ptr(y),
                                    rows, K, m, _stream(stream)), "ck_gemv_q5_0_q8_0")


def ck_gemv_q8_0_q8_0(W, xq, bias, residual, y, rows, K, m, stream=None):
    _check(load().ck_gemv_q8_0_q8_0(_ptr(W), _ptr(xq), _ptr(bias), _ptr(residual), _ptr(y),
                                    rows, K, m, _stream(stream)), "ck_gemv_q8_0_q8_0")


def ck_rope(q, k, cos_tab, sin_tab, tab_rows, pos, m, H, KV, hd, stream=None):
    _check(load().ck_rope(_ptr(q), _ptr(k), _ptr(cos_tab), _ptr(sin_tab), tab_rows, _pos(pos),
                          m, H, KV, hd, _stream(stream)), "ck_rope")


def kv_cache(k, v, kv_heads, head_dim, capacity=0, page_size=0, page_table=None,
             max_pages_per_seq=0, num_pages=0, dtype=CK_KV_F32, k_scale=1.0,
             v_scale=1.0, window=0, ring=False) -> CkKVCache:
    c = CkKVCache(_ptr(k), _ptr(v), kv_heads, head_dim, capacity, page_size,
                  _ptr(page_table), max_pages_per_seq, num_pages, dtype, k_scale, v_scale,
                  window, int(ring))
    # the struct holds raw device pointers: it keeps the objects they point
    # into alive as long as it lives
    c._keep = (k, v, page_table)
    return c


def ck_kv_append(cache: CkKVCache, k, v, pos, m, stream=None):
    _check(load().ck_kv_append(ctypes.byref(cache), _ptr(k), _ptr(v), _pos(pos), m,
                               _stream(stream)), "ck_kv_append")


def ck_attn_workspace_size(m, H, KV, hd, max_tokens, chunk=0) -> int:
    return int(load().ck_attn_workspace_size(m, H, KV, hd, max_tokens, chunk))


def ck_attn_decode_gqa(q, cache: CkKVCache, pos, out, m, H, scale, chunk, ws, ws_bytes,
                       stream=None):
    _check(load().ck_attn_decode_gqa(_ptr(q), ctypes.byref(cache), _pos(pos), _ptr(out), m, H,
                                     scale, chunk, _ptr(ws), ws_bytes, _stream(stream)),
           "ck_attn_decode_gqa")


def ck_attn_partial(q, cache: CkKVCache, pos, m, H, scale, chunk, partials, nbytes,
                    stream=None):
    _check(load().ck_attn_partial(_ptr(q), ctypes.byref(cache), _pos(pos), m, H, scale, chunk,
                                  _ptr(partials), nbytes, _stream(stream)), "ck_attn_partial")


def ck_attn_merge(partials, nbytes, pos, m, H, KV, hd, chunk, out, out_q8=None, stream=None,
                  window=0):
    _check(load().ck_attn_merge(_ptr(partials), nbytes, _pos(pos), m, H, KV, hd, chunk, window,
                                _ptr(out), _ptr(out_q8), _stream(stream)), "ck_attn_merge")


def layer_desc(D, H, KV, head_dim, m=1, eps=1e-6, variant=CK_VARIANT_FUSED, attn_chunk=0):
    return CkLayerDesc(D, H, KV, head_dim, m, eps, variant, attn_chunk)


def layer_weights(wq, wk, wv, wo, bq, bk, bv, bo, gamma, rope_cos, rope_sin, rope_rows):
    return CkLayerWeights(_ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(bq), _ptr(bk), _ptr(bv),
                          _ptr(bo), _ptr(gamma), _ptr(rope_cos), _ptr(rope_sin), rope_rows)


def ck_decode_layer_workspace_size(desc: CkLayerDesc, max_ctx: int) -> int:
    return int(load().ck_decode_layer_workspace_size(ctypes.byref(desc), max_ctx))


def ck_decode_layer_ws_offset(desc: CkLayerDesc, max_ctx: int, name: str) -> int:
    return int(load().ck_decode_layer_ws_offset(ctypes.byref(desc), max_ctx, name.encode()))


def ck_decode_layer(desc: CkLayerDesc, weights: CkLayerWeights, cache: CkKVCache, x, residual,
                    pos, out, ws, ws_bytes, stream=None):
    _check(load().ck_decode_layer(ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(cache),
                                  _ptr(x), _ptr(residual), _pos(pos), _ptr(out), _ptr(ws),
                                  ws_bytes, _stream(stream)), "ck_decode_layer")


def ck_read_probe(src, nbytes, sink, stream=None):
    _check(load().ck_read_probe(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "ck_read_probe")


def ck_decode_layer_attn_plan(desc: CkLayerDesc, cache: CkKVCache, pos, topk=0):
    """(chunk, nchunks) of the attention a layer call plans at these positions."""
    chunk, nchunks = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().ck_decode_layer_attn_plan(ctypes.byref(desc), ctypes.byref(cache), _pos(pos),
                                            int(topk), ctypes.byref(chunk), ctypes.byref(nchunks)),
           "ck_decode_layer_attn_plan")
    return chunk.value, nchunks.value


def ck_decode_layer_part(desc: CkLayerDesc, weights: CkLayerWeights, cache: CkKVCache, x, residual,
                         pos, out, ws, ws_bytes, part, stream=None):
    _check(load().ck_decode_layer_part(ctypes.byref(desc), ctypes.byref(weights),
                                       ctypes.byref(cache), _ptr(x), _ptr(residual), _pos(pos),
                                       _ptr(out), _ptr(ws), ws_bytes, int(part), _stream(stream)),
           "ck_decode_layer_part")


def ck_decode_layer_noalloc(desc: CkLayerDesc, weights: CkLayerWeights, cache: CkKVCache, x,
                            residual, pos, out, stream=None):
    _check(load().ck_decode_layer_noalloc(ctypes.byref(desc), ctypes.byref(weights),
                                          ctypes.byref(cache), _ptr(x), _ptr(residual), _pos(pos),
                                          _ptr(out), _stream(stream)), "ck_decode_layer_noalloc")


def ck_decode_layer_noalloc_limit() -> int:
    return int(load().ck_decode_layer_noalloc_limit())


def ck_decode_step_workspace_size(desc: CkLayerDesc, layers: int, max_ctx: int) -> int:
    return int(load().ck_decode_step_workspace_size(ctypes.byref(desc), layers, max_ctx))


def ck_decode_step_status_offset(desc: CkLayerDesc, layers: int) -> int:
    return int(load().ck_decode_step_status_offset(ctypes.byref(desc), layers))


def ck_decode_step(desc: CkLayerDesc, weights, caches, x, pos, out, ws, ws_bytes, stream=None):
    """weights, caches: sequences of CkLayerWeights / CkKVCache, one per layer
    (or ctypes arrays of them)."""
    n = len(weights)
    if len(caches) != n:
        raise ValueError("one cache per layer")
    wa = weights if isinstance(weights, ctypes.Array) else (CkLayerWeights * n)(*weights)
    ca = caches if isinstance(caches, ctypes.Array) else (CkKVCache * n)(*caches)
    _check(load().ck_decode_step(ctypes.byref(desc), wa, ca, n, _ptr(x), _pos(pos), _ptr(out),
                                 _ptr(ws), ws_bytes, _stream(stream)), "ck_decode_step")


def ck_attn_sparse(q, cache: CkKVCache, pos, sel, topk, sink, out, m, H, scale, chunk, ws,
                   ws_bytes, stream=None):
    """sel: device int32 [m][topk] (-1 = absent); sink: device fp32 [H] or None."""
    _check(load().ck_attn_sparse(_ptr(q), ctypes.byref(cache), _pos(pos), _ptr(sel), topk,
                                 _ptr(sink), _ptr(out), m, H, scale, chunk, _ptr(ws), ws_bytes,
                                 _stream(stream)), "ck_attn_sparse")


def ck_decode_layer_sparse(desc: CkLayerDesc, weights: CkLayerWeights, cache: CkKVCache, x,
                           residual, sel, topk, sink, out, ws, ws_bytes, pos=None, pos_dev=None,
                           max_ctx=0, stream=None):
    """Exactly one of pos (host positions) and pos_dev (device int32 tensor)."""
    _check(load().ck_decode_layer_sparse(ctypes.byref(desc), ctypes.byref(weights),
                                         ctypes.byref(cache), _ptr(x), _ptr(residual),
                                         _pos(pos) if pos is not None else None, _ptr(pos_dev),
                                         max_ctx, _ptr(sel), topk, _ptr(sink), _ptr(out),
                                         _ptr(ws), ws_bytes, _stream(stream)),
           "ck_decode_layer_sparse")


def ck_decode_layer_devpos(desc: CkLayerDesc, weights: CkLayerWeights, cache: CkKVCache, x,
                           residual, pos_dev, max_ctx, out, ws, ws_bytes, stream=None):
    """pos_dev: a device int32 tensor of m positions, read when the kernels run."""
    _check(load().ck_decode_layer_devpos(ctypes.byref(desc), ctypes.byref(weights),
                                         ctypes.byref(cache), _ptr(x), _ptr(residual),
                                         _ptr(pos_dev), max_ctx, _ptr(out), _ptr(ws), ws_bytes,
                                         _stream(stream)), "ck_decode_layer_devpos")


def ck_decode_step_devpos(desc: CkLayerDesc, weights, caches, x, pos_dev, max_ctx, out, ws,
                          ws_bytes, stream=None):
    n = len(weights)
    if len(caches) != n:
        raise ValueError("one cache per layer")
    wa = weights if isinstance(weights, ctypes.Array) else (CkLayerWeights * n)(*weights)
    ca = caches if isinstance(caches, ctypes.Array) else (CkKVCache * n)(*caches)
    _check(load().ck_decode_step_devpos(ctypes.byref(desc), wa, ca, n, _ptr(x), _ptr(pos_dev),
                                        max_ctx, _ptr(out), _ptr(ws), ws_bytes, _stream(stream)),
           "ck_decode_step_devpos")
