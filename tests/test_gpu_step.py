"""GPU parity of a whole decode step (ck_decode_step: every layer of a
workload in one call), in the three variants.

  * chain and fused: bit-identical to the same variant called layer by layer
    through ck_decode_layer (the same kernels, verified stage by stage in
    test_gpu_layer.py);
  * persistent (every layer in one persistent kernel): status word zero; end to
    end against the independent oracle chain within max(2e-3, 3 x the chain's
    rounding-noise floor) x RMS (the floor: the larger deviation of the oracle
    chained with +-1-ulp nudged inputs and of the verified fused GPU chain,
    from the oracle chain); the last
    layer's intermediates left in the workspace checked stage by stage on the
    GPU's own inputs (xq bytes exact, attention within 1e-4, its Q8_0 bytes
    exact); every cache slot other than the appended ones byte-identical, and
    the appended slots of every layer within max(2e-3, 3 x the same floor
    taken for k and v over the layers up to that one, 3 x one code flip) of
    the oracle chain's. One code flip: a rounding difference anywhere upstream
    can move one Q8_0 code of a layer's quantized input by one, which moves
    every appended k (v) element by up to max|W_k| (max|W_v|) times that
    block's scale; the floor estimates need not happen to contain a flip
    where the persistent chain has one;
  * two persistent steps in a row at successive positions: the second attends
    over the row the first appended, checked against the oracle on the GPU's
    own caches and input.
"""
import numpy as np
import pytest

import oracle
from decode_step_attention_layer_amd import synth
from gpu_helpers import assert_close_rms, cuda, host, rms

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _ocache(cfg, L, k, v):
    if cfg.page_size:
        return oracle.Cache(k, v, cfg.KV, cfg.hd, page_size=cfg.page_size,
                            page_table=L.host["table"], max_pages_per_seq=cfg.max_pages_per_seq,
                            num_pages=k.shape[0])
    return oracle.Cache(k, v, cfg.KV, cfg.hd, capacity=cfg.capacity)


def _dims(cfg):
    return dict(D=cfg.D, H=cfg.H, KV=cfg.KV, hd=cfg.hd, m=cfg.m, eps=cfg.eps)


def _oracle_chain(stack, x0, nudge_seed=None):
    """The oracle through every layer from x0 on fresh copies of the original
    caches; with nudge_seed, every layer input is first moved by +-1 ulp.
    Returns the output, per layer the appended (k, v) slots, and per layer
    the largest Q8_0 block scale of the layer's quantized input."""
    cfg = stack.cfg
    cos, sin = synth.rope_for(cfg)
    g = np.random.default_rng(nudge_seed) if nudge_seed is not None else None
    x = x0.copy()
    appended, dmax = [], []
    for L in stack.layers:
        if g is not None:
            up = g.random(x.shape) < 0.5
            x = np.where(up, np.nextafter(x, np.float32(np.inf)),
                         np.nextafter(x, np.float32(-np.inf))).astype(np.float32)
        xq = np.concatenate([oracle.quantize_q8_0(oracle.rmsnorm(r, L.host["gamma"], cfg.eps))
                             for r in x])
        dmax.append(float(np.max(np.abs(_block_scales(xq, 34)))))
        c = _ocache(cfg, L, L.host["k"].copy(), L.host["v"].copy())
        x = oracle.decode_layer(_dims(cfg), dict(L.host, rope_cos=cos, rope_sin=sin), c, x, x,
                                stack.pos)
        mask = _appended_mask(cfg, L, stack.pos)
        appended.append((c.k.reshape(-1)[mask].copy(), c.v.reshape(-1)[mask].copy()))
    return x, appended, dmax


def _block_scales(blocks, nbytes):
    """The binary16 scales (first two bytes) of Q8_0 (34-byte) or Q5_0
    (22-byte) blocks."""
    b = np.ascontiguousarray(blocks, np.uint8).reshape(-1, nbytes)
    return b[:, :2].copy().view("<f2")[:, 0].astype(np.float64)


def _max_weight(packed, q5):
    """An upper bound of |w| over a Q5_0 (|code - 16| <= 16) or Q8_0
    (|code| <= 128) weight matrix: the largest block scale times the code."""
    return float(np.max(np.abs(_block_scales(packed, 22 if q5 else 34)))) * (16 if q5 else 128)


def _rel_dev(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - b))) / rms(b)


def _appended_mask(cfg, L, pos):
    """Boolean masks over the flattened cache of the slots a step appends."""
    k = L.host["k"]
    mask = np.zeros(k.size, bool)
    hd, KV = cfg.hd, cfg.KV
    for s in range(cfg.m):
        for g in range(KV):
            t = pos[s]
            if cfg.page_size:
                page = int(L.host["table"][s, t // cfg.page_size])
                row = ((page * KV + g) * cfg.page_size + t % cfg.page_size) * hd
            else:
                row = ((s * KV + g) * cfg.capacity + t) * hd
            mask[row:row + hd] = True
    return mask


def _step_check(name, layers=None):
    import torch
    from decode_step_attention_layer_amd import ck
    from decode_step_attention_layer_amd.workload import DeviceStack

    dev = cuda()
    cfg = synth.CONFIGS[name]
    stack = DeviceStack(cfg, dev, keep_host=True, spare_pages=4 if cfg.page_size else 0,
                        layers=layers)
    m, D, H, hd = cfg.m, cfg.D, cfg.H, cfg.hd
    tag = f"{name} x{stack.nlayers}"

    # chain and fused: whole step == layer by layer, bit for bit
    for variant in (ck.CK_VARIANT_CHAIN, ck.CK_VARIANT_FUSED):
        d = stack.desc(variant)
        per_layer = stack.step(d, stack.workspace(d)).clone()
        whole = stack.decode_step(d, stack.step_workspace(d)).clone()
        torch.cuda.synchronize()
        assert torch.equal(whole, per_layer), f"{tag} variant {variant}: step != layer by layer"
        print(f"{tag} variant {variant}: whole step equals layer by layer", flush=True)
    fused_out = host(whole)
    fused_app = []
    for L in stack.layers:
        mask = _appended_mask(cfg, L, stack.pos)
        fused_app.append((host(L.tensors["k"]).reshape(-1)[mask],
                          host(L.tensors["v"]).reshape(-1)[mask]))

    # persistent
    d = stack.desc(ck.CK_VARIANT_PERSISTENT)
    ws = stack.step_workspace(d)
    ws.fill_(0xFF)
    print(f"{tag} persistent step", flush=True)
    out = host(stack.decode_step(d, ws))
    torch.cuda.synchronize()
    assert stack.step_status(d, ws) == 0, f"{tag}: persistent step reported a timed-out wait"

    # Bounds for a chain of layers: 3 x the rounding noise two independent
    # estimates show, never below 2e-3: the oracle chained against itself with
    # +-1-ulp nudged layer inputs, and the fused GPU chain (verified layer by
    # layer, stage by stage) against the oracle chain. For the appended k and
    # v of layer l, the larger deviation over layers 0..l (the noise only
    # accumulates down the chain).
    x_orc, app_orc, dmax = _oracle_chain(stack, stack.x0_host)
    bound = TOL
    kv_bounds = [(TOL, TOL)] * stack.nlayers
    if stack.nlayers > 1:
        x_nud, app_nud, _ = _oracle_chain(stack, stack.x0_host, 1234)
        floor = max(_rel_dev(x_nud, x_orc), _rel_dev(fused_out, x_orc))
        bound = max(TOL, 3.0 * floor)
        kv_bounds, fk, fv = [], 0.0, 0.0
        for L, dq, (kn, vn), (kf, vf), (ko, vo) in zip(stack.layers, dmax, app_nud, fused_app,
                                                       app_orc):
            fk = max(fk, _rel_dev(kn, ko), _rel_dev(kf, ko))
            fv = max(fv, _rel_dev(vn, vo), _rel_dev(vf, vo))
            flip_k = _max_weight(L.host["wk"], True) * dq / rms(ko)
            flip_v = _max_weight(L.host["wv"], False) * dq / rms(vo)
            kv_bounds.append((max(TOL, 3.0 * fk, 3.0 * flip_k), max(TOL, 3.0 * fv, 3.0 * flip_v)))
        print(f"{tag}: chain noise floor {floor:.2e}; one-flip k/v bound of the last layer "
              f"{kv_bounds[-1][0]:.2e} / {kv_bounds[-1][1]:.2e}", flush=True)
    e2e = assert_close_rms(out, x_orc, bound, f"{tag} persistent end to end")
    rel_fused = assert_close_rms(out, fused_out, bound, f"{tag} persistent vs fused")
    print(f"{tag} persistent: e2e rel err {e2e:.2e}, vs fused {rel_fused:.2e} (bound {bound:.2e})")

    # the last layer's intermediates, on the GPU's own inputs
    off = {n: ck.ck_decode_layer_ws_offset(d, stack.max_ctx, n)
           for n in ("xn", "xq", "q", "attn", "aq")}

    def rd(n, nbytes, dt):
        return ws[off[n]: off[n] + nbytes].cpu().numpy().view(dt)

    xn = rd("xn", 4 * m * D, np.float32).reshape(m, D)
    xq = rd("xq", m * D // 32 * 34, np.uint8).reshape(m, -1)
    gq = rd("q", 4 * m * H * hd, np.float32).reshape(m, H * hd)
    at = rd("attn", 4 * m * H * hd, np.float32).reshape(m, H * hd)
    aq = rd("aq", m * H * hd // 32 * 34, np.uint8).reshape(m, -1)
    Ll = stack.layers[-1]
    gcache = _ocache(cfg, Ll, host(Ll.tensors["k"]), host(Ll.tensors["v"]))
    for s in range(m):
        assert np.array_equal(xq[s], oracle.quantize_q8_0(xn[s])), f"{tag} last-layer xq bytes"
        a0 = oracle.attention(gq[s], gcache, s, stack.pos[s] + 1, H)
        assert_close_rms(at[s], a0, 1e-4, f"{tag} last-layer attention")
        assert np.array_equal(aq[s], oracle.quantize_q8_0(at[s])), f"{tag} last-layer aq bytes"

    # caches: only the appended slots changed; those match the oracle chain's
    # within that layer's noise-floor bound
    for li, L in enumerate(stack.layers):
        mask = _appended_mask(cfg, L, stack.pos)
        for j, (name_, orig) in enumerate((("k", L.host["k"]), ("v", L.host["v"]))):
            got = host(L.tensors[name_]).reshape(-1)
            orig = orig.reshape(-1)
            assert np.array_equal(got.view(np.uint32)[~mask], orig.view(np.uint32)[~mask]), \
                f"{tag} layer {li} {name_}: a slot other than the appended one changed"
            assert_close_rms(got[mask], app_orc[li][j], kv_bounds[li][j],
                             f"{tag} layer {li} appended {name_}")


def test_step_c1():
    _step_check("c1")


def test_step_c2():
    _step_check("c2")


@pytest.mark.timeout(900)
def test_step_c3():
    _step_check("c3")


@pytest.mark.timeout(600)
def test_step_c4():
    _step_check("c4")


@pytest.mark.timeout(600)
def test_step_c5():
    _step_check("c5")


@pytest.mark.parametrize("name", ["c1", "c2", "c5"])
def test_persistent_successive_positions(name):
    """Two one-layer persistent steps at positions p and p + 1: the second
    reads the row the first appended (written by an earlier launch)."""
    import torch
    from decode_step_attention_layer_amd import ck
    from decode_step_attention_layer_amd.workload import DeviceStack

    dev = cuda()
    cfg = synth.CONFIGS[name]
    stack = DeviceStack(cfg, dev, keep_host=True, spare_pages=4 if cfg.page_size else 0, layers=1)
    d = stack.desc(ck.CK_VARIANT_PERSISTENT)
    stack.max_ctx += 1
    ws = stack.step_workspace(d)
    L = stack.layers[0]
    cos, sin = synth.rope_for(cfg)
    wts = dict(L.host, rope_cos=cos, rope_sin=sin)
    x = stack.x0
    for step in range(2):
        if cfg.page_size:
            # map a spare page where the next position starts a new page
            table = L.host["table"]
            free = sorted(set(range(L.host["k"].shape[0])) - set(table[table >= 0].tolist()))
            for s_, p in enumerate(stack.pos):
                if table[s_, p // cfg.page_size] < 0:
                    table[s_, p // cfg.page_size] = free.pop(0)
            L.tensors["table"].copy_(torch.from_numpy(table))
        k_before, v_before = host(L.tensors["k"]), host(L.tensors["v"])
        out = torch.empty_like(x)
        stack.decode_step(d, ws, out=out, x=x)
        torch.cuda.synchronize()
        assert stack.step_status(d, ws) == 0
        c = _ocache(cfg, L, k_before, v_before)
        ref = oracle.decode_layer(_dims(cfg), wts, c, host(x), host(x), stack.pos)
        assert_close_rms(host(out), ref, TOL, f"{name} step {step} at {stack.pos}")
        stack.pos = [p + 1 for p in stack.pos]
        x = out
