"""Pins of the oracle's binary16 codec and Q8_0 activation quantizer.

CPU only. The codec is checked exhaustively against numpy's IEEE binary16 type
and against hand-worked tie cases; the quantizer against hand-worked blocks
(tests/golden/q8_0_blocks.txt) and invariants that any correct
amax/127, round-half-away quantizer satisfies.
"""
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_cases(name):
    out = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            out.append([p.strip() for p in line.split("|")])
    return out


# ------------------------------------------------------------------ codec ---
def test_f16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([orc.f16_to_f32(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_encode_roundtrip_all_finite(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    fin = np.isfinite(vals)
    for b, v in zip(bits[fin][::7], vals[fin][::7].astype(np.float32)):
        assert orc.f32_to_f16(float(v)) == int(b)


def test_f16_encode_matches_numpy_rne(orc):
    g = np.random.default_rng(1234)
    mags = np.exp(g.uniform(np.log(1e-9), np.log(7e4), 20000)).astype(np.float32)
    sgn = np.where(g.random(20000) < 0.5, -1, 1).astype(np.float32)
    x = mags * sgn
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([orc.f32_to_f16(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("case", _read_cases("f16_cases.txt"), ids=lambda c: c[0])
def test_f16_encode_golden_ties(orc, case):
    x = np.float32(float(case[0]))
    assert float(x) == float(case[0]), "fixture input must be exact in fp32"
    assert orc.f32_to_f16(float(x)) == int(case[1], 16)


# -------------------------------------------------------------- quantizer ---
def _codes(blocks):
    b = blocks.reshape(-1, 34)
    d = b[:, :2].copy().view("<u2")[:, 0]
    q = b[:, 2:].view(np.int8)
    return d, q


@pytest.mark.parametrize("case", _read_cases("q8_0_blocks.txt"), ids=lambda c: c[0])
def test_q8_0_golden_blocks(orc, case):
    name, xs, dbits, qs = case
    x = np.zeros(32, np.float32)
    vals = [float(t) for t in xs.split()]
    x[: len(vals)] = vals
    q = np.zeros(32, np.int8)
    cv = [int(t) for t in qs.split()]
    q[: len(cv)] = cv
    d, got = _codes(orc.quantize_q8_0(x))
    assert int(d[0]) == int(dbits, 16), name
    assert np.array_equal(got[0], q), name


def _random_blocks(seed, nblocks, scale_spread=True):
    g = np.random.default_rng(seed)
    x = g.standard_normal((nblocks, 32)).astype(np.float32)
    if scale_spread:
        x *= np.exp(g.uniform(-6, 6, (nblocks, 1))).astype(np.float32)
    return x


def test_q8_0_invariants(orc):
    x = _random_blocks(7, 4096)
    d, q = _codes(orc.quantize_q8_0(x.reshape(-1)))
    q = q.astype(np.int32)
    # |q| <= 127 and the amax element maps to +-127 with the element's sign
    assert np.abs(q).max() <= 127
    j = np.argmax(np.abs(x), axis=1)
    rows = np.arange(x.shape[0])
    assert np.array_equal(q[rows, j], np.where(x[rows, j] > 0, 127, -127))
    # the stored scale is binary16(amax / 127)
    amax = np.abs(x).max(axis=1)
    ref_d = (amax / np.float32(127)).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(d, ref_d)
    # the dequantized block lies within half a quantum (+ fp16 scale rounding)
    d32 = (amax / np.float32(127)).astype(np.float64)
    d16 = d.view(np.float16).astype(np.float64)
    err = np.abs(x.astype(np.float64) - d16[:, None] * q)
    bound = 0.5 * d32[:, None] * (1 + 1e-6) + 127 * np.abs(d32 - d16)[:, None]
    assert np.all(err <= bound)


def test_q8_0_odd_symmetry(orc):
    x = _random_blocks(8, 1024).reshape(-1)
    dp, qp = _codes(orc.quantize_q8_0(x))
    dn, qn = _codes(orc.quantize_q8_0(-x))
    assert np.array_equal(dp, dn)
    assert np.array_equal(qp.astype(np.int32), -qn.astype(np.int32))


@pytest.mark.parametrize("k", [-3, -1, 1, 2, 5])
def test_q8_0_power_of_two_scaling(orc, k):
    # scaling a block by 2^k scales d by 2^k and leaves the codes unchanged, as
    # long as d stays a normal binary16 number
    x = _random_blocks(9, 512, scale_spread=False).reshape(-1)
    d0, q0 = _codes(orc.quantize_q8_0(x))
    d1, q1 = _codes(orc.quantize_q8_0(x * np.float32(2.0 ** k)))
    assert np.array_equal(q0, q1)
    f0 = d0.view(np.float16).astype(np.float64)
    f1 = d1.view(np.float16).astype(np.float64)
    assert np.array_equal(f1, f0 * 2.0 ** k)


def test_q8_0_zero_block_and_mixed(orc):
    x = np.zeros(96, np.float32)
    x[32:64] = np.linspace(-3, 3, 32, dtype=np.float32)
    d, q = _codes(orc.quantize_q8_0(x))
    assert d[0] == 0 and not q[0].any()
    assert d[2] == 0 and not q[2].any()
    assert d[1] != 0 and np.abs(q[1]).max() == 127


def test_q8_0_dequantize_decodes_codes(orc):
    x = _random_blocks(10, 64).reshape(-1)
    blocks = orc.quantize_q8_0(x)
    d, q = _codes(blocks)
    ref = (d.view(np.float16).astype(np.float32)[:, None] * q.astype(np.float32)).reshape(-1)
    assert np.array_equal(orc.dequantize_q8_0(blocks, x.size), ref)
