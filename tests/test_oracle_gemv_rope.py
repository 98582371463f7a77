"""Pins of the oracle's block GEMVs and RoPE.

GEMV: the block-integer dot (sum over blocks of d_w * d_x * integer sum) must
equal the float64 product of the dequantized matrix and vector (numpy matmul),
where the dequantized values come from the generator's own codes and scales,
not from the oracle's decoder. Zero weights must pass the bias (and the
residual) through bit for bit.

RoPE: rotate-half RoPE is multiplication of z_i = x_i + i x_{i+hd/2} by
e^{i angle}; checked against numpy complex arithmetic, plus norm preservation,
the inverse rotation, the identity at position 0 and angle addition.
"""
import numpy as np
import pytest

from decode_step_attention_layer_amd import synth


def _act(orc, seed, K):
    x = synth.seeded_vector(seed, K)
    xq = orc.quantize_q8_0(x)
    b = xq.reshape(-1, 34)
    d = b[:, :2].copy().view("<f2")[:, 0].astype(np.float64)
    q = b[:, 2:].view(np.int8).astype(np.float64)
    return xq, (d[:, None] * q).reshape(-1)


@pytest.mark.parametrize("rows,K", [(7, 32), (33, 256), (64, 896), (5, 4096)])
def test_gemv_q5_0_equals_dequantized_matmul(orc, rows, K):
    W = synth.seeded_vector(100 + rows, rows * K, 0.02).reshape(rows, K)
    wb, codes, s16 = synth.weights_to_q5_0(W)
    wdq = (s16.astype(np.float64)[..., None] * (codes.astype(np.float64) - 16)).reshape(rows, K)
    xq, xdq = _act(orc, 200 + K, K)
    bias = synth.seeded_vector(300, rows, 0.02)
    ref = wdq @ xdq
    got = orc.gemv_q5_0(wb, xq, bias, None, rows, K)
    # fp32(dot) + bias: allow one fp32 rounding of the dot plus the add
    tol = 2.0 ** -23 * (np.abs(ref) + np.abs(bias)) * 2 + 1e-30
    assert np.all(np.abs(got.astype(np.float64) - (ref + bias.astype(np.float64))) <= tol)


@pytest.mark.parametrize("rows,K", [(9, 64), (128, 512)])
def test_gemv_q8_0_equals_dequantized_matmul(orc, rows, K):
    W = synth.seeded_vector(400 + rows, rows * K, 0.02).reshape(rows, K)
    wb, codes, s16 = synth.weights_to_q8_0(W)
    wdq = (s16.astype(np.float64)[..., None] * codes.astype(np.float64)).reshape(rows, K)
    xq, xdq = _act(orc, 500 + K, K)
    ref = wdq @ xdq
    got = orc.gemv_q8_0(wb, xq, None, None, rows, K)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-30)


def test_q5_0_decoder_matches_generator_codes(orc):
    W = synth.seeded_vector(11, 4 * 128, 0.02).reshape(4, 128)
    wb, codes, s16 = synth.weights_to_q5_0(W)
    for r in range(4):
        got = orc.dequantize_q5_0(wb[r], 128)
        ref = (s16[r].astype(np.float32)[:, None] * (codes[r].astype(np.float32) - 16)).reshape(-1)
        assert np.array_equal(got, ref)


def test_q5_0_layout_single_bits(orc):
    # one code at a time, so a swapped nibble or qh bit order cannot cancel out
    for j in range(32):
        for code in (0, 1, 15, 16, 17, 31):
            codes = np.full((1, 1, 32), 16, np.uint8)
            codes[0, 0, j] = code
            wb = synth.pack_q5_0(codes, np.ones((1, 1), np.float16))
            got = orc.dequantize_q5_0(wb[0], 32)
            ref = np.zeros(32, np.float32)
            ref[j] = code - 16
            assert np.array_equal(got, ref), (j, code)


def test_gemv_zero_weights_pass_bias_and_residual(orc):
    rows, K = 48, 256
    xq, _ = _act(orc, 12, K)
    bias = synth.seeded_vector(13, rows, 0.02)
    res = synth.seeded_vector(14, rows)
    zq5 = np.zeros((rows, K // 32 * 22), np.uint8)
    zq8 = np.zeros((rows, K // 32 * 34), np.uint8)
    assert np.array_equal(orc.gemv_q5_0(zq5, xq, bias, None, rows, K), bias)
    assert np.array_equal(orc.gemv_q8_0(zq8, xq, bias, None, rows, K), bias)
    got = orc.gemv_q5_0(zq5, xq, bias, res, rows, K)
    assert np.array_equal(got, (bias + res).astype(np.float32))
    assert np.array_equal(orc.gemv_q5_0(zq5, xq, None, None, rows, K), np.zeros(rows, np.float32))


# ------------------------------------------------------------------ RoPE ---
def _rope_case(H, KV, hd, rows=64, theta=1e4, seed=21):
    cos, sin = synth.rope_tables(rows, hd, theta)
    q = synth.seeded_vector(seed, H * hd)
    k = synth.seeded_vector(seed + 1, KV * hd)
    return cos, sin, q, k


@pytest.mark.parametrize("hd", [64, 128])
def test_rope_is_complex_rotation(orc, hd):
    H, KV, pos = 4, 2, 37
    cos, sin, q, k = _rope_case(H, KV, hd)
    q2, k2 = orc.rope(q, k, cos, sin, pos, H, KV, hd)
    half = hd // 2
    ang = pos * 1e4 ** (-2.0 * np.arange(half) / hd)
    rot = np.exp(1j * ang)
    for src, dst, n in ((q, q2, H), (k, k2, KV)):
        s = src.astype(np.float64).reshape(n, hd)
        z = (s[:, :half] + 1j * s[:, half:]) * rot
        ref = np.concatenate([z.real, z.imag], axis=1).reshape(-1)
        assert np.max(np.abs(dst - ref)) < 2e-6 * max(1.0, np.max(np.abs(ref)))


def test_rope_norm_inverse_identity(orc):
    H, KV, hd = 3, 1, 64
    cos, sin, q, k = _rope_case(H, KV, hd, rows=128)
    half = hd // 2
    q2, k2 = orc.rope(q, k, cos, sin, 100, H, KV, hd)
    a, b = q.reshape(H, hd)[:, :half].astype(np.float64), q.reshape(H, hd)[:, half:].astype(np.float64)
    a2, b2 = q2.reshape(H, hd)[:, :half].astype(np.float64), q2.reshape(H, hd)[:, half:].astype(np.float64)
    assert np.allclose(a * a + b * b, a2 * a2 + b2 * b2, rtol=1e-6, atol=1e-12)
    # negated angles undo the rotation
    q3, k3 = orc.rope(q2, k2, cos, -sin, 100, H, KV, hd)
    assert np.max(np.abs(q3 - q)) < 1e-5 and np.max(np.abs(k3 - k)) < 1e-5
    # position 0 is the identity, bit for bit
    q0, k0 = orc.rope(q, k, cos, sin, 0, H, KV, hd)
    assert np.array_equal(q0, q) and np.array_equal(k0, k)


def test_rope_angle_addition(orc):
    H, KV, hd = 2, 1, 64
    cos, sin, q, k = _rope_case(H, KV, hd, rows=64)
    qa, ka = orc.rope(q, k, cos, sin, 13, H, KV, hd)
    qab, kab = orc.rope(qa, ka, cos, sin, 29, H, KV, hd)
    qs, ks = orc.rope(q, k, cos, sin, 42, H, KV, hd)
    assert np.max(np.abs(qab - qs)) < 2e-5 and np.max(np.abs(kab - ks)) < 2e-5


def test_rope_leaves_v_and_other_positions_alone(orc):
    # only q and k are rotated; passing no k leaves k untouched by construction
    H, KV, hd = 2, 1, 64
    cos, sin, q, k = _rope_case(H, KV, hd)
    q2, k2 = orc.rope(q, None, cos, sin, 5, H, KV, hd)
    assert k2 is None and not np.array_equal(q2, q)
