"""Pins of the oracle's building blocks against facts outside the oracle.

Each test checks one oracle function against a library routine that does not
share its code (numpy's IEEE half conversion, fp64 matrix products), a closed
form, or an invariant of the mathematics, so that a dropped term, a wrong sign
or index, or a transposed operand fails one of them.
"""
import math

import numpy as np
import pytest


# ---------------------------------------------------------------- fp16

def test_f16_decode_every_code(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_to_f32(codes)
    ref = codes.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_encode_matches_ieee_rne(orc):
    rng = np.random.default_rng(7)
    parts = [
        rng.standard_normal(200000).astype(np.float32) * np.float32(1000),
        (rng.standard_normal(200000) * 1e-6).astype(np.float32),     # fp16 subnormal range
        (rng.standard_normal(50000) * 1e-9).astype(np.float32),      # underflow to zero
        np.float32([65504, 65519.99, 65520, 65536, 1e30, -65520, np.inf, -np.inf, 0.0, -0.0,
                    2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 1e-45]),
    ]
    # exact midpoints between neighbouring halves (ties go to the even code)
    h = np.arange(0, 0x7bff, 7, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    parts.append(((lo + hi) / 2).astype(np.float32))
    x = np.concatenate(parts)
    ours = orc.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------- GEMV

def test_gemv_exact_on_integers(orc):
    """Small-integer operands make every product and partial sum exact in fp32,
    so the result must equal the integer matrix product bit for bit; a
    transposed or shifted operand cannot pass."""
    rng = np.random.default_rng(1)
    W = rng.integers(-8, 9, size=(37, 53))
    x = rng.integers(-8, 9, size=53)
    y = orc.gemv(W.astype(np.float16), x.astype(np.float32))
    assert np.array_equal(y, (W @ x).astype(np.float32))


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 8), (17, 256), (64, 1000)])
def test_gemv_within_fp32_bound_of_fp64(orc, rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    W = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float16)
    x = rng.standard_normal(cols).astype(np.float32)
    y = orc.gemv(W, x).astype(np.float64)
    ref = W.astype(np.float64) @ x.astype(np.float64)
    bound = cols * 2.0 ** -24 * (np.abs(W.astype(np.float64)) @ np.abs(x.astype(np.float64))) * 1.01
    assert np.all(np.abs(y - ref) <= bound + 1e-30)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_unit_rms_without_eps(orc):
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(2560) * 3.7).astype(np.float32)
    y = orc.rmsnorm(x, np.ones(2560, np.float16), 0.0).astype(np.float64)
    assert abs(math.sqrt(np.mean(y * y)) - 1.0) < 1e-6


def test_rmsnorm_rms_with_eps_and_gain(orc):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(256) * 0.01).astype(np.float32)
    eps = 1e-5
    ms = float(np.mean(x.astype(np.float64) ** 2))
    y = orc.rmsnorm(x, np.ones(256, np.float16), eps).astype(np.float64)
    assert abs(math.sqrt(np.mean(y * y)) - math.sqrt(ms / (ms + eps))) < 1e-6
    g = rng.standard_normal(256).astype(np.float16)
    yg = orc.rmsnorm(x, g, eps).astype(np.float64)
    assert np.allclose(yg, y * g.astype(np.float64), rtol=1e-6, atol=1e-9)
    # scale invariance (eps = 0): rmsnorm(c x) == rmsnorm(x)
    y1 = orc.rmsnorm(x, np.ones(256, np.float16), 0.0)
    y2 = orc.rmsnorm(x * np.float32(8.0), np.ones(256, np.float16), 0.0)
    assert np.array_equal(y1, y2)


# ---------------------------------------------------------------- RoPE

def test_rope_identity_at_position_zero(orc):
    v = np.random.default_rng(4).standard_normal(128).astype(np.float32)
    assert np.array_equal(orc.rope(v, 0), v)


def test_rope_closed_forms(orc):
    """dh=2: the one pair rotates by angle p (theta_0 = 1); dh=4: the second pair
    rotates by p / base^(1/2).  Fixes the sign convention and the frequencies."""
    for p in (1, 5, 100, 1023):
        y = orc.rope(np.float32([1, 0]), p).astype(np.float64)
        assert np.allclose(y, [math.cos(p), math.sin(p)], atol=1e-6)
        y = orc.rope(np.float32([0, 1, 0, 0]), p, base=10000.0).astype(np.float64)
        assert np.allclose(y, [0, math.cos(p / 100.0), 0, math.sin(p / 100.0)], atol=1e-6)
        y = orc.rope(np.float32([0, 0, 0, 1]), p).astype(np.float64)   # (i, i+dh/2) = (1, 3)
        assert np.allclose(y, [0, -math.sin(p / 100.0), 0, math.cos(p / 100.0)], atol=1e-6)


def test_rope_norm_and_relative_position(orc):
    rng = np.random.default_rng(5)
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal(128).astype(np.float32)
    for m, n in ((7, 3), (300, 299), (1000, 0), (50, 50)):
        rq, rk = orc.rope(q, m).astype(np.float64), orc.rope(k, n).astype(np.float64)
        pairs = lambda v: v[:64] ** 2 + v[64:] ** 2
        assert np.allclose(pairs(rq), pairs(q.astype(np.float64)), rtol=1e-5)
        lhs = float(rq @ rk)
        rhs = float(orc.rope(q, m - n).astype(np.float64) @ k.astype(np.float64))
        assert abs(lhs - rhs) < 1e-4 * (1 + abs(rhs))


# ---------------------------------------------------------------- attention

def _cache(rng, n, hkv, dh):
    k = rng.standard_normal((n, hkv, dh)).astype(np.float16)
    v = rng.standard_normal((n, hkv, dh)).astype(np.float16)
    return k, v


def test_attention_single_key_returns_value_row(orc):
    rng = np.random.default_rng(6)
    k, v = _cache(rng, 4, 2, 64)
    q = rng.standard_normal((2, 64)).astype(np.float32)
    o = orc.attention(q, k, v, 0)
    assert np.array_equal(o, v[0].astype(np.float32))


def test_attention_identical_keys_average_values(orc):
    rng = np.random.default_rng(7)
    n, dh = 9, 64
    k1 = rng.standard_normal(dh).astype(np.float16)
    k = np.broadcast_to(k1, (n, 1, dh)).copy()
    v = rng.standard_normal((n, 1, dh)).astype(np.float16)
    q = rng.standard_normal((1, dh)).astype(np.float32) * 10
    o = orc.attention(q, k, v, n - 1)
    assert np.allclose(o[0], v[:, 0].astype(np.float64).mean(0), atol=1e-5)


def test_attention_weights_match_fp64_softmax(orc):
    """One-hot value rows expose the attention weights: they must sum to one and
    equal softmax(q.k / sqrt(dh)) computed in fp64 by numpy."""
    rng = np.random.default_rng(8)
    n, dh, hq, hkv = 40, 64, 4, 2
    k = (rng.standard_normal((n, hkv, dh)) * 0.5).astype(np.float16)
    v = np.zeros((n, hkv, dh), np.float16)
    for j in range(n):
        v[j, :, j] = 1.0
    q = rng.standard_normal((hq, dh)).astype(np.float32)
    for pos in (0, 5, n - 1):
        o = orc.attention(q, k, v, pos).astype(np.float64)
        for h in range(hq):
            g = h // (hq // hkv)
            s = (k[: pos + 1, g].astype(np.float64) @ q[h].astype(np.float64)) / math.sqrt(dh)
            a = np.exp(s - s.max())
            a /= a.sum()
            assert abs(o[h, : pos + 1].sum() - 1.0) < (pos + 1) * 2.0 ** -23
            assert np.allclose(o[h, : pos + 1], a, rtol=1e-5, atol=1e-7)
            assert np.all(o[h, pos + 1:] == 0)


def test_attention_gqa_equals_mha_with_shared_heads(orc):
    rng = np.random.default_rng(9)
    n, dh, hq, hkv = 17, 64, 8, 2
    k, v = _cache(rng, n, hkv, dh)
    q = rng.standard_normal((hq, dh)).astype(np.float32)
    grp = hq // hkv
    k_full = np.repeat(k, grp, axis=1)     # query head h reads KV head h // grp
    v_full = np.repeat(v, grp, axis=1)
    assert np.array_equal(orc.attention(q, k, v, n - 1), orc.attention(q, k_full, v_full, n - 1))


# ---------------------------------------------------------------- misc

def test_silu_closed_form(orc):
    for z in (-20.0, -1.5, 0.0, 0.3, 7.0):
        assert abs(orc.silu(z) - z / (1 + math.exp(-z))) < 1e-6 * (1 + abs(z))
    assert orc.silu(0.0) == 0.0


def test_argmax_lowest_index_on_ties(orc):
    assert orc.argmax(np.float32([1, 3, 3, 2])) == 1
    assert orc.argmax(np.float32([5, 5, 5])) == 0
    assert orc.argmax(np.float32([-1, -0.5, -0.5])) == 1
    x = np.zeros(4096, np.float32)
    x[4095] = 1e-30
    assert orc.argmax(x) == 4095


def test_attention_window_weights_match_fp64_softmax(orc):
    """Sliding window: one-hot value rows expose the weights; rows before
    pos - window + 1 get none, the rest equal an fp64 softmax over the window."""
    rng = np.random.default_rng(18)
    n, dh, hq, hkv = 48, 96, 4, 2
    k = (rng.standard_normal((n, hkv, dh)) * 0.5).astype(np.float16)
    v = np.zeros((n, hkv, dh), np.float16)
    for j in range(n):
        v[j, :, j] = 1.0
    q = rng.standard_normal((hq, dh)).astype(np.float32)
    for pos, W in ((0, 4), (3, 4), (4, 4), (30, 7), (n - 1, 16), (n - 1, 1)):
        o = orc.attention(q, k, v, pos, W).astype(np.float64)
        lo = max(0, pos - W + 1)
        for h in range(hq):
            g = h // (hq // hkv)
            s = (k[lo: pos + 1, g].astype(np.float64) @ q[h].astype(np.float64)) / math.sqrt(dh)
            a = np.exp(s - s.max())
            a /= a.sum()
            assert np.all(o[h, :lo] == 0) and np.all(o[h, pos + 1:] == 0), (pos, W)
            assert np.allclose(o[h, lo: pos + 1], a, rtol=1e-5, atol=1e-7), (pos, W)


def test_attention_window_one_returns_current_value_row(orc):
    rng = np.random.default_rng(19)
    k, v = _cache(rng, 10, 2, 96)
    q = rng.standard_normal((4, 96)).astype(np.float32)
    o = orc.attention(q, k, v, 7, 1)
    assert np.array_equal(o, v[7][[0, 0, 1, 1]].astype(np.float32))
    # a window that covers every row is full attention
    assert np.array_equal(orc.attention(q, k, v, 7, 8), orc.attention(q, k, v, 7))
