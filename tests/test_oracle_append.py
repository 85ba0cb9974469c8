"""Pins for the oracle's KV append (scatter) and E4M3 encoder (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.append import append_kv, e4m3_encode, quantize_e4m3


def test_encode_inverts_decode_on_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    np.testing.assert_array_equal(e4m3_encode(vals), codes)


def test_encode_matches_torch_cast_within_range():
    """torch's float8_e4m3fn cast rounds to nearest-even; inside +-448 it must agree."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 40,
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 50_000).astype(np.float32),     # subnormal range
        rng.uniform(-448, 448, 50_000).astype(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_encode(x.astype(np.float64)), ref)


def test_ties_go_to_the_even_code():
    t = oracle.e4m3_decode_table()
    for c in [0x00, 0x01, 0x06, 0x07, 0x08, 0x30, 0x38, 0x39, 0x70, 0x7C, 0x7D]:
        mid = (t[c] + t[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert e4m3_encode(np.array([mid]))[0] == want, hex(c)
        assert e4m3_encode(np.array([-mid]))[0] == want | 0x80


def test_saturation_sign_and_nan():
    e = e4m3_encode(np.array([448.0, 449.0, 1e6, np.inf, -1e6, -np.inf, 0.0, -0.0, -1e-12, np.nan]))
    assert list(e) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x80, 0x7F]


def test_quantize_divides_in_float32():
    x = np.array([1.0, 3.3, -7.77], dtype=np.float32)
    s = 0.37
    q = (x / np.float32(s)).astype(np.float32)
    np.testing.assert_array_equal(quantize_e4m3(x, s), e4m3_encode(q.astype(np.float64)))


def test_append_then_gather_returns_the_new_tokens():
    rng = np.random.default_rng(1)
    nb, hkv, bs, d = 6, 2, 4, 8
    kp = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vp = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    T = 7
    kn = rng.standard_normal((T, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((T, hkv, d)).astype(np.float32)
    slots = np.array([5, 0, -1, 23, 12, 13, 1])
    k2, v2 = append_kv(kp, vp, kn, vn, slots, bs)
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        np.testing.assert_array_equal(k2[sl // bs, :, sl % bs], kn[t])
        np.testing.assert_array_equal(v2[sl // bs, :, sl % bs], vn[t])
    # every other slot is untouched
    touched = {int(s) for s in slots if s >= 0}
    for sl in range(nb * bs):
        if sl not in touched:
            np.testing.assert_array_equal(k2[sl // bs, :, sl % bs], kp[sl // bs, :, sl % bs])
    # a row whose table lists blocks 1 then 0 sees slot 5 (block 1, offset 1) as token 1
    K = oracle.gather_kv(k2, "f32", np.array([1, 0]), 2, 0, bs)
    np.testing.assert_array_equal(K[1], kn[0, 0])


def test_append_fp8_uses_per_head_scale():
    rng = np.random.default_rng(2)
    kp = np.zeros((2, 2, 4, 8), np.uint8)
    vp = np.zeros((2, 2, 4, 8), np.uint8)
    kn = rng.standard_normal((3, 2, 8)).astype(np.float32)
    vn = rng.standard_normal((3, 2, 8)).astype(np.float32)
    ks = np.array([0.5, 0.01], np.float32)
    vs = np.array([0.02, 0.25], np.float32)
    k2, v2 = append_kv(kp, vp, kn, vn, [2, 4, 7], 4, "fp8", ks, vs)
    np.testing.assert_array_equal(k2[1, 1, 0], quantize_e4m3(kn[1, 1], ks[1]))
    np.testing.assert_array_equal(v2[1, 0, 3], quantize_e4m3(vn[2, 0], vs[0]))
    # dequantised values are within half an E4M3 step (2^-4 relative) of the input
    deq = oracle.e4m3_decode(k2[0, 0, 2]) * ks[0]
    assert np.all(np.abs(deq - kn[0, 0]) <= 2.0 ** -4 * np.abs(kn[0, 0]) + 2.0 ** -10 * ks[0])


def _ties_ok(enc):
    t = oracle.e4m3_decode_table()
    for c in [0x00, 0x01, 0x07, 0x30, 0x38, 0x39, 0x7C, 0x7D]:
        mid = (t[c] + t[c + 1]) / 2
        if enc(np.array([mid]))[0] != (c if c % 2 == 0 else c + 1):
            return False
    return True


def _saturation_ok(enc):
    return list(enc(np.array([449.0, 470.0, 1e6]))) == [0x7E, 0x7E, 0x7E]


def test_planted_encoder_mistakes_are_caught():
    """Ties rounded away from zero, or overflow mapped to NaN, fail the pins above."""
    from oracle.append import _positive_codes

    def ties_away(x):
        x = np.asarray(x, dtype=np.float64)
        vals, codes = _positive_codes()
        a = np.minimum(np.abs(x), 448.0)
        hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
        lo = np.clip(hi - 1, 0, len(vals) - 1)
        c = np.where(vals[hi] - a <= a - vals[lo], codes[hi], codes[lo])
        return (c | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)

    def overflow_nan(x):
        x = np.asarray(x, dtype=np.float64)
        return np.where(np.abs(x) > 464.0, np.uint8(0x7F), e4m3_encode(x)).astype(np.uint8)

    assert _ties_ok(e4m3_encode) and _saturation_ok(e4m3_encode)
    assert not _ties_ok(ties_away)
    assert not _saturation_ok(overflow_nan)
