"""GPU parity of the whole decode layer (ck_decode_layer) against the oracle,
at the five workloads' full sizes and in the configuration the benchmark times,
and at three more paged batches (4, 5 and 12 tokens).

Per layer (parity.check_layer), with the oracle run on the same input the GPU
layer received:
  * stage by stage on identical inputs (the GPU's own intermediates read back
    from the workspace): xn within 1e-5, Q8_0 bytes of xn and of the attention
    output bit-exact, q/k/v within 1e-5, attention within 1e-4, O projection
    within 1e-5 of the branch RMS plus two ulps of the output;
  * out and the attention output within 2e-3 x RMS of the plain oracle (the
    required layer-output bound); every Q8_0 code of xq, and of the attention
    output against the oracle run from the GPU's xq codes, that differs must
    be a rounding-boundary flip (off by one, both scaled values within 1% of
    a quantum of the boundary);
  * the branch (out - residual) within 2e-3 x RMS(branch) of the oracle run
    from the GPU's xq codes, plus for each counted aq flip the movement it
    causes through Wo (|Wo[e, j]| times the code step), and of the plain
    oracle, plus the oracle-evaluated effect of the xq flips;
  * every KV-cache slot except the appended one is byte-identical (NaN poison
    included), and the appended slot holds exactly the k, v the layer computed;
  * chain and fused: the attention called on its own at the split the layer
    reports planning (ck_decode_layer_attn_plan) reproduces the layer's
    attention output bit for bit.
The persistent variant runs here as one-layer persistent steps (the same
kernel as a whole step, with one layer's items); the two-launch variant
(attention, merge and O projection in one launch) also leaves its status
word zero. End to end, the GPU chain of
all layers matches the independent oracle chain
within max(2e-3, 3 x the oracle's own +-1-ulp noise floor) x RMS: chaining
quantized layers turns last-bit differences into occasional code flips in
every layer, and the oracle chained against itself with +-1-ulp nudges shows
how far that alone carries (about 5e-3 after the 28 layers of the 7B shape).
"""
import numpy as np
import pytest

import oracle
from decode_step_attention_layer_amd import synth
import parity
from gpu_helpers import assert_close_rms, cuda, host, rms

pytestmark = pytest.mark.gpu

TOL = 2e-3
VARIANTS = [0, 1, 2, 3]
VARIANT_IDS = ["chain", "fused", "persistent", "two_launch"]


def gcache_row(cfg, L, s, g, t):
    """Float offset of (sequence, KV head, token) in the cache layout of ck.h."""
    hd, KV = cfg.hd, cfg.KV
    if cfg.page_size:
        page = int(L.host["table"][s, t // cfg.page_size])
        return ((page * KV + g) * cfg.page_size + t % cfg.page_size) * hd
    return ((s * KV + g) * cfg.capacity + t) * hd


def _ws_read(ws, off, nbytes, dtype):
    return ws[off: off + nbytes].cpu().numpy().view(dtype)


def _run_and_check(name, variant, attn_chunk=0, layers=None):
    import torch
    from decode_step_attention_layer_amd import ck
    from decode_step_attention_layer_amd.workload import DeviceStack

    dev = cuda()
    cfg = synth.CONFIGS[name] if name in synth.CONFIGS else BATCHES[name]
    stack = DeviceStack(cfg, dev, keep_host=True, spare_pages=4 if cfg.page_size else 0,
                        layers=layers)
    desc = stack.desc(variant, attn_chunk)
    ws = stack.workspace(desc)
    ws.fill_(0xFF)                       # NaN poison for any read of unwritten workspace
    m, D, H, KV, hd = cfg.m, cfg.D, cfg.H, cfg.KV, cfg.hd
    dims = dict(D=D, H=H, KV=KV, hd=hd, m=m, eps=cfg.eps)
    cos, sin = synth.rope_for(cfg)
    pos = stack.pos
    read = ws_reader(ck, desc, stack.max_ctx, ws, cfg)

    x_gpu_in = stack.x0
    x_host = stack.x0_host.copy()            # GPU chain input, host copy
    for li, L in enumerate(stack.layers):
        print(f"{name} variant={variant} layer {li}", flush=True)
        out = stack.bufs[li % 2]
        ck.ck_decode_layer(desc, L.weights, L.cache, x_gpu_in, x_gpu_in, pos, out, ws, ws.numel())
        torch.cuda.synchronize()
        got = host(out)
        if variant in (0, 1):
            _attention_at_reported_plan(ck, desc, stack, L, ws, pos, f"{name} layer {li}")
        if variant == 3:
            soff = ck.ck_decode_layer_ws_offset(desc, stack.max_ctx, "status")
            assert soff >= 0 and int(ws[soff:soff + 4].view(torch.int32).item()) == 0, \
                f"{name} layer {li}: a wait of the second launch timed out"
        wts = dict(L.host, rope_cos=cos, rope_sin=sin)
        st = parity.check_layer(cfg, wts, lambda k, v: ocache(cfg, L, k, v), L.host["k"],
                                L.host["v"], x_host, got, read(), host(L.tensors["k"]),
                                host(L.tensors["v"]), pos,
                                lambda s, g: gcache_row(cfg, L, s, g, pos[s]),
                                f"{name} layer {li}")
        print(f"{name} layer {li}: xq flips {st['xq_flips']}, aq flips {st['aq_flips']}, "
              f"branch rel err {st['branch_cond']:.2e} (conditioned) / "
              f"{st['branch_pure']:.2e} (plain oracle)")
        x_host = got
        x_gpu_in = out
    # End to end over a stack, against the independent oracle chain: the
    # bound is the oracle's own rounding-noise floor, how far the oracle
    # chained with every layer input nudged by +-1 ulp (the size of fp32
    # reassociation differences) diverges from itself, because nudged values
    # cross Q8_0 rounding boundaries in every layer.
    def layer_fn(l, x):
        Ll = stack.layers[l]
        return oracle.decode_layer(dims, dict(Ll.host, rope_cos=cos, rope_sin=sin),
                                   ocache(cfg, Ll, Ll.host["k"].copy(), Ll.host["v"].copy()),
                                   x, x, pos)

    if len(stack.layers) > 1:
        floor, x_orc = parity.nudged_floor(layer_fn, stack.x0_host, len(stack.layers))
        bound = max(TOL, 3.0 * floor)
        print(f"{name}: oracle +-1 ulp noise floor over {len(stack.layers)} layers {floor:.2e}")
    else:
        x_orc, bound = layer_fn(0, stack.x0_host.copy()), TOL
    e2e = assert_close_rms(x_host, x_orc, bound, f"{name} end to end")
    print(f"{name} variant={variant}: layers={len(stack.layers)} e2e rel err {e2e:.2e} "
          f"(bound {bound:.2e}, branch RMS {rms(x_orc - stack.x0_host):.3f})")


def _attention_at_reported_plan(ck, desc, stack, L, ws, pos, tag):
    """The chain and fused layers run the attention kernels: called on their
    own, on the layer's q (from the workspace) and the appended cache, at the
    split ck_decode_layer_attn_plan reports, they give the layer's attention
    output bit for bit (the scale rounded as the layer rounds it)."""
    import torch

    cfg = stack.cfg
    m, H, KV, hd = cfg.m, cfg.H, cfg.KV, cfg.hd
    chunk, nchunks = ck.ck_decode_layer_attn_plan(desc, L.cache, pos)
    assert (nchunks - 1) * chunk < max(pos) + 1 <= nchunks * chunk, (tag, chunk, nchunks)
    qoff = ck.ck_decode_layer_ws_offset(desc, stack.max_ctx, "q")
    aoff = ck.ck_decode_layer_ws_offset(desc, stack.max_ctx, "attn")
    nws = ck.ck_attn_workspace_size(m, H, KV, hd, max(pos) + 1, chunk)
    aw = torch.empty(nws, dtype=torch.uint8, device=ws.device)
    ao = torch.empty(m * H * hd, dtype=torch.float32, device=ws.device)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(hd)))
    ck.ck_attn_decode_gqa(ws.data_ptr() + qoff, L.cache, pos, ao, m, H, scale, chunk, aw, nws)
    torch.cuda.synchronize()
    layer_attn = _ws_read(ws, aoff, 4 * m * H * hd, np.float32)
    assert np.array_equal(host(ao).view(np.uint32), layer_attn.view(np.uint32)), \
        f"{tag}: attention at the reported split (chunk {chunk}) differs from the layer's"


def ocache(cfg, L, k, v):
    if cfg.page_size:
        return oracle.Cache(k, v, cfg.KV, cfg.hd, page_size=cfg.page_size,
                            page_table=L.host["table"], max_pages_per_seq=cfg.max_pages_per_seq,
                            num_pages=k.shape[0])
    return oracle.Cache(k, v, cfg.KV, cfg.hd, capacity=cfg.capacity)


def ws_reader(ck, desc, max_ctx, ws, cfg):
    """A function returning the layer intermediates kept in the workspace
    (offsets from ck_decode_layer_ws_offset), as [m][...] host arrays."""
    m, D, H, KV, hd = cfg.m, cfg.D, cfg.H, cfg.KV, cfg.hd
    off = {n: ck.ck_decode_layer_ws_offset(desc, max_ctx, n)
           for n in ("xn", "xq", "q", "k", "v", "attn", "aq")}
    sizes = dict(xn=(4 * m * D, np.float32), xq=(m * D // 32 * 34, np.uint8),
                 q=(4 * m * H * hd, np.float32), k=(4 * m * KV * hd, np.float32),
                 v=(4 * m * KV * hd, np.float32), attn=(4 * m * H * hd, np.float32),
                 aq=(m * H * hd // 32 * 34, np.uint8))

    def read():
        return {n: _ws_read(ws, off[n], nb, dt).reshape(m, -1) for n, (nb, dt) in sizes.items()}
    return read


@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_layer_c1(variant):
    _run_and_check("c1", variant)


@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_layer_c1_small_chunks(variant):
    _run_and_check("c1", variant, attn_chunk=64)


@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_layer_c2(variant):
    _run_and_check("c2", variant)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_layer_c3(variant):
    _run_and_check("c3", variant)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_layer_c4(variant):
    _run_and_check("c4", variant)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_layer_c5(variant):
    _run_and_check("c5", variant)


# Other batches of the paged path: the matrix-core projections from 4 tokens,
# the activation images' zero token slots from m to 15, the Q/K/V epilogue at
# other head counts and widths; b4s is small enough (heads x tokens x 32-dim
# parts within the compute units) for the merge to split heads over 32-dim
# workgroups while it writes the O projection's activation image.
BATCHES = {
    "b4": synth.Config("b4", 21, 3584, 28, 4, 128, 1e4, layers=1, m=4, page_size=16,
                       min_ctx=100, max_ctx=900),
    "b5": synth.Config("b5", 22, 4096, 32, 8, 128, 5e5, layers=1, m=5, page_size=16,
                       min_ctx=64, max_ctx=700),
    "b12": synth.Config("b12", 23, 896, 14, 2, 64, 1e4, layers=2, m=12, page_size=16,
                        min_ctx=30, max_ctx=300),
    "b4s": synth.Config("b4s", 24, 512, 8, 2, 64, 1e4, layers=2, m=4, page_size=16,
                        min_ctx=20, max_ctx=200),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
@pytest.mark.parametrize("name", sorted(BATCHES))
def test_layer_other_batches(name, variant):
    _run_and_check(name, variant)
