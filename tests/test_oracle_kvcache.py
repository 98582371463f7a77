"""Pins of the oracle's reduced-precision KV cache (bf16, FP8 E4M3 with one
scale per tensor): the element codecs against torch's own bfloat16 and
float8_e4m3fn conversions (exhaustive decodes; encodes over random values,
hand-built ties, subnormals and the saturation the store uses), and the
cache-reading and -writing paths against the fp32 cache holding the decoded
values."""
import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def test_bf16_decode_exhaustive():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([oracle.bf16_to_f32(int(c)) for c in codes], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_encode_matches_torch():
    g = np.random.default_rng(5)
    x = np.concatenate([
        g.standard_normal(4000).astype(np.float32),
        (g.standard_normal(2000) * 1e-30).astype(np.float32),
        (g.standard_normal(2000) * 1e30).astype(np.float32),
        # exact ties: 1 + 2^-8 (to 1.0, even) and 1 + 3 * 2^-8 (to 1 + 2^-6, even)
        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 2.0**-130, 0.0, -0.0,
                  np.inf, -np.inf, 3.3895314e38], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)
    assert oracle.f32_to_bf16(1 + 2**-8) == 0x3F80 and oracle.f32_to_bf16(1 + 3 * 2**-8) == 0x3F82
    assert math.isnan(oracle.bf16_to_f32(oracle.f32_to_bf16(float("nan"))))


def test_e4m3_decode_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle.e4m3_to_f32(int(c)) for c in codes], np.float32)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)           # 0x7F, 0xFF
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert oracle.e4m3_to_f32(0x7E) == 448.0 and oracle.e4m3_to_f32(0x01) == 2.0**-9
    assert oracle.e4m3_to_f32(0x08) == 2.0**-6 and oracle.e4m3_to_f32(0x38) == 1.0


def test_e4m3_encode_matches_torch_in_range():
    g = np.random.default_rng(7)
    x = np.concatenate([
        g.standard_normal(5000).astype(np.float32) * 4,
        g.uniform(-464, 464, 3000).astype(np.float32),
        (g.standard_normal(2000) * 2**-8).astype(np.float32),
        # every half step of the subnormal and first normal spacings: ties
        np.array([k * 2.0**-10 for k in range(-40, 41)], np.float32),
        # ties in normal binades (midpoints between neighbours)
        np.array([1.0625, 1.1875, 3.25 + 0.125, 240.0 + 8.0, 448.0, 456.0, 464.0], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.f32_to_e4m3(float(v)) for v in x], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates_and_roundtrips():
    # beyond the rounding range the store saturates (torch would give NaN)
    for v, want in [(465.0, 0x7E), (1e30, 0x7E), (np.inf, 0x7E), (-500.0, 0xFE),
                    (-np.inf, 0xFE), (np.nan, 0x7F)]:
        assert oracle.f32_to_e4m3(float(v)) == want, v
    # every finite code survives decode then encode
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.f32_to_e4m3(oracle.e4m3_to_f32(c)) == c, hex(c)


@pytest.mark.parametrize("dtype", [oracle.KV_BF16, oracle.KV_FP8_E4M3], ids=["bf16", "fp8"])
@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
def test_reduced_cache_equals_fp32_cache_of_decoded_values(dtype, paged):
    """Append and attention on a bf16 / fp8 cache equal the same operations on
    an fp32 cache that holds the decoded values, bit for bit; the append
    stores exactly the codec's codes (fp8: of x / scale) and nothing else."""
    g = np.random.default_rng(11 + dtype + 2 * paged)
    KV, hd, H, L, pos = 2, 32, 4, 37, 36
    ks, vs = (0.03125, 0.0546875) if dtype == oracle.KV_FP8_E4M3 else (1.0, 1.0)
    if paged:
        ps, P, maxp = 8, 7, 6
        table = np.full((1, maxp), -1, np.int32)
        table[0, :5] = np.array([3, 0, 6, 2, 5], np.int32)
        shape = (P, KV, ps, hd)
        geo = dict(page_size=ps, page_table=table, max_pages_per_seq=maxp, num_pages=P)
    else:
        shape = (1, KV, 64, hd)
        geo = dict(capacity=64)
    vals_k = (g.standard_normal(shape) * 2).astype(np.float32)
    vals_v = (g.standard_normal(shape) * 2).astype(np.float32)
    ck_ = oracle.encode_cache(vals_k, dtype, ks)
    cv_ = oracle.encode_cache(vals_v, dtype, vs)
    red = oracle.Cache(ck_.copy(), cv_.copy(), KV, hd, dtype=dtype, k_scale=ks, v_scale=vs, **geo)
    f32 = oracle.Cache(oracle.decode_cache(ck_, dtype, ks), oracle.decode_cache(cv_, dtype, vs),
                       KV, hd, **geo)
    k_new = (g.standard_normal(KV * hd) * 3).astype(np.float32)
    v_new = (g.standard_normal(KV * hd) * 3).astype(np.float32)
    oracle.kv_append(red, 0, pos, k_new, v_new)
    # the appended slot holds the codes of the new values, every other slot is unchanged
    changed_k = red.k != ck_
    enc_k = oracle.encode_cache(k_new, dtype, ks)
    enc_v = oracle.encode_cache(v_new, dtype, vs)
    assert changed_k.sum() <= KV * hd
    if paged:
        page, slot = table[0, pos // 8], pos % 8
        got_k, got_v = red.k[page, :, slot, :], red.v[page, :, slot, :]
    else:
        got_k, got_v = red.k[0, :, pos, :], red.v[0, :, pos, :]
    assert np.array_equal(got_k.reshape(-1), enc_k) and np.array_equal(got_v.reshape(-1), enc_v)
    mask = np.ones(shape, bool)
    if paged:
        mask[page, :, slot, :] = False
    else:
        mask[0, :, pos, :] = False
    assert np.array_equal(red.k[mask], ck_[mask]) and np.array_equal(red.v[mask], cv_[mask])
    # the fp32 cache receives the decoded codes of the same append
    oracle.kv_append(f32, 0, pos, oracle.decode_cache(enc_k, dtype, ks),
                     oracle.decode_cache(enc_v, dtype, vs))
    q = g.standard_normal(H * hd).astype(np.float32)
    a = oracle.attention(q, red, 0, L, H)
    b = oracle.attention(q, f32, 0, L, H)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
