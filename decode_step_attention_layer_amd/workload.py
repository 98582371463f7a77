"""Device-resident workloads for the decode layer: upload seeded inputs, wire
them into the C-ABI structs and run decode steps through libck.

Plumbing only (torch provides device memory and the stream); every step of
the layer runs in libck's kernels. A "step" runs every layer of the
configuration once, chaining x_{l+1} = out_l with residual_l = x_l.
"""
from __future__ import annotations

import concurrent.futures as cf
from dataclasses import dataclass, field

import numpy as np
import torch

from . import ck, synth


def to_dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclass
class DeviceLayer:
    tensors: dict
    weights: ck.CkLayerWeights
    cache: ck.CkKVCache
    host: dict = field(default_factory=dict)


class DeviceStack:
    """All layers of one configuration on one GPU, plus x, outputs and workspace."""

    def __init__(self, cfg: synth.Config, device="cuda", poison: float = float("nan"),
                 keep_host: bool = False, spare_pages: int = 0, layers: int | None = None,
                 threads: int = 8, kv_dtype: int = synth.KV_F32, window: int = 0,
                 ring: bool = False, topk: int = 0):
        self.cfg = cfg
        self.kv_dtype = kv_dtype
        # sliding window; a ring (contiguous caches only) has `window` slots
        assert not ring or (window > 0 and not cfg.page_size), "a ring is contiguous, window > 0"
        self.window = window
        self.ring = ring
        self.capacity = window if ring else cfg.capacity
        # sparse attention: per layer a selection [m][topk] and sink logits [H]
        self.topk = topk
        self.k_scale = synth.FP8_K_SCALE if kv_dtype == synth.KV_FP8 else 1.0
        self.v_scale = synth.FP8_V_SCALE if kv_dtype == synth.KV_FP8 else 1.0
        self.device = torch.device(device)
        self.nlayers = cfg.layers if layers is None else layers
        cos, sin = synth.rope_for(cfg)
        self.rope = (to_dev(cos, self.device), to_dev(sin, self.device))
        self.rope_rows = cos.shape[0]
        x = synth.token_input(cfg)
        self.x0_host = x
        self.x0 = to_dev(x, self.device)
        self.lens = synth.context_lengths(cfg)
        self.pos = [int(p) for p in self.lens]

        def make(layer):
            w = synth.layer_weights(cfg, layer)
            if cfg.page_size:
                k, v, table, lens = synth.paged_cache(cfg, layer, poison, spare_pages)
                assert np.array_equal(lens, self.lens)
                c = dict(k=k, v=v, table=table)
            elif ring:
                k, v = synth.ring_cache(cfg, layer, window, poison)
                c = dict(k=k, v=v)
            else:
                k, v = synth.contiguous_cache(cfg, layer, poison)
                c = dict(k=k, v=v)
            if kv_dtype != synth.KV_F32:
                c["k"] = synth.cache_codes(c["k"], kv_dtype, cfg.index, layer, True)
                c["v"] = synth.cache_codes(c["v"], kv_dtype, cfg.index, layer, False)
            if topk:
                c["sel"] = synth.selection(cfg, layer, topk, self.lens)
                c["sink"] = synth.sink_logits(cfg, layer)
            return layer, w, c

        self.layers: list[DeviceLayer] = []
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            for layer, w, c in ex.map(make, range(self.nlayers)):
                self.layers.append(self._upload(w, c, keep_host))
        D = cfg.D
        self.bufs = [torch.empty((cfg.m, D), dtype=torch.float32, device=self.device)
                     for _ in range(2)]
        self.max_ctx = max(self.pos) + 1

    def clone(self) -> "DeviceStack":
        """A second copy of every device tensor (same values, new memory), for
        benchmarks that rotate replicas to keep the working set out of the
        last-level cache."""
        twin = object.__new__(DeviceStack)
        twin.__dict__.update(self.__dict__)
        twin.layers = []
        cfg = self.cfg
        for L in self.layers:
            t = {n: v.clone() for n, v in L.tensors.items()}
            if cfg.page_size:
                cache = ck.kv_cache(t["k"], t["v"], cfg.KV, cfg.hd, 0, cfg.page_size, t["table"],
                                    cfg.max_pages_per_seq, L.cache.num_pages, **self._kvargs())
            else:
                cache = ck.kv_cache(t["k"], t["v"], cfg.KV, cfg.hd, self.capacity,
                                    **self._kvargs())
            weights = ck.layer_weights(t["wq"], t["wk"], t["wv"], t["wo"], t["bq"], t["bk"],
                                       t["bv"], t["bo"], t["gamma"], self.rope[0], self.rope[1],
                                       self.rope_rows)
            twin.layers.append(DeviceLayer(t, weights, cache, L.host))
        twin.bufs = [b.clone() for b in self.bufs]
        twin.x0 = self.x0.clone()
        twin._arrays = None
        twin.step_out = None
        return twin

    def _upload(self, w, c, keep_host):
        dev = self.device
        t = {n: to_dev(w[n], dev) for n in ("wq", "wk", "wv", "wo", "bq", "bk", "bv", "bo", "gamma")}
        t["k"] = to_dev(c["k"], dev)
        t["v"] = to_dev(c["v"], dev)
        for n in ("sel", "sink"):
            if n in c:
                t[n] = to_dev(c[n], dev)
        cfg = self.cfg
        if cfg.page_size:
            t["table"] = to_dev(c["table"], dev)
            cache = ck.kv_cache(t["k"], t["v"], cfg.KV, cfg.hd, 0, cfg.page_size, t["table"],
                                cfg.max_pages_per_seq, c["k"].shape[0], **self._kvargs())
        else:
            cache = ck.kv_cache(t["k"], t["v"], cfg.KV, cfg.hd, self.capacity, **self._kvargs())
        weights = ck.layer_weights(t["wq"], t["wk"], t["wv"], t["wo"], t["bq"], t["bk"], t["bv"],
                                   t["bo"], t["gamma"], self.rope[0], self.rope[1], self.rope_rows)
        host = dict(w, **{n: c[n] for n in ("k", "v", "table", "sel", "sink") if n in c}) \
            if keep_host else {}
        return DeviceLayer(t, weights, cache, host)

    def _kvargs(self) -> dict:
        return dict(dtype=self.kv_dtype, k_scale=self.k_scale, v_scale=self.v_scale,
                    window=self.window, ring=self.ring)

    def desc(self, variant=ck.CK_VARIANT_FUSED, attn_chunk=0) -> ck.CkLayerDesc:
        c = self.cfg
        return ck.layer_desc(c.D, c.H, c.KV, c.hd, c.m, c.eps, variant, attn_chunk)

    def workspace(self, desc: ck.CkLayerDesc) -> torch.Tensor:
        n = ck.ck_decode_layer_workspace_size(desc, max(self.max_ctx, self.topk))
        assert n > 0, "layer shape rejected by libck"
        return torch.empty(n, dtype=torch.uint8, device=self.device)

    def step(self, desc: ck.CkLayerDesc, ws: torch.Tensor, stream=None, x=None) -> torch.Tensor:
        """One decode step through every layer; returns the last layer's output."""
        cur = self.x0 if x is None else x
        for i, L in enumerate(self.layers):
            out = self.bufs[i % 2]
            if self.topk:
                ck.ck_decode_layer_sparse(desc, L.weights, L.cache, cur, cur, L.tensors["sel"],
                                          self.topk, L.tensors["sink"], out, ws, ws.numel(),
                                          pos=self.pos, stream=stream)
            else:
                ck.ck_decode_layer(desc, L.weights, L.cache, cur, cur, self.pos, out, ws,
                                   ws.numel(), stream)
            cur = out
        return cur

    # ----------------------------------------------------- whole-step entry --
    def step_workspace(self, desc: ck.CkLayerDesc) -> torch.Tensor:
        n = ck.ck_decode_step_workspace_size(desc, self.nlayers, self.max_ctx)
        assert n > 0, "step shape rejected by libck"
        return torch.empty(n, dtype=torch.uint8, device=self.device)

    def step_arrays(self):
        """ctypes arrays of the layers' weight and cache structs (built once)."""
        if getattr(self, "_arrays", None) is None:
            n = self.nlayers
            self._arrays = ((ck.CkLayerWeights * n)(*[L.weights for L in self.layers]),
                            (ck.CkKVCache * n)(*[L.cache for L in self.layers]))
        return self._arrays

    def decode_step(self, desc: ck.CkLayerDesc, ws: torch.Tensor, out: torch.Tensor | None = None,
                    stream=None, x=None) -> torch.Tensor:
        """One decode step through every layer with a single ck_decode_step call."""
        if out is None:
            if getattr(self, "step_out", None) is None:
                self.step_out = torch.empty((self.cfg.m, self.cfg.D), dtype=torch.float32,
                                            device=self.device)
            out = self.step_out
        w, c = self.step_arrays()
        ck.ck_decode_step(desc, w, c, self.x0 if x is None else x, self.pos, out, ws, ws.numel(),
                          stream)
        return out

    def step_status(self, desc: ck.CkLayerDesc, ws: torch.Tensor) -> int:
        """The persistent step's status word (0: completed)."""
        off = ck.ck_decode_step_status_offset(desc, self.nlayers)
        assert off >= 0
        return int(ws[off:off + 4].view(torch.int32).item())
