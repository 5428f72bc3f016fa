"""Pins of the FP8 (e4m3) KV-cache oracle against what the format and the
mathematics fix (no GPU): the value table against its closed-form landmarks
and torch's float8_e4m3fn, the encoder against torch's rounding and the
midpoint rule, saturation, the scatter's placement, and attention over
quantised pools against attention over values that e4m3 holds exactly."""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_kv as F


def test_value_table_landmarks():
    t = F.e4m3_value_table()
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9                     # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9                 # largest subnormal
    assert t[0x08] == 2.0 ** -6                     # smallest normal
    assert t[0x38] == 1.0                           # exponent field 7 = bias
    assert t[0x7E] == 448.0                         # largest finite
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.all(np.diff(t[:0x7F]) > 0)            # codes 0..126 ascending
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])


def test_value_table_matches_torch_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = F.e4m3_value_table()
    assert np.array_equal(np.isnan(ref), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(ref[ok], t[ok])


def test_encode_matches_torch_rounding_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(x), ref)


def test_encode_midpoints_go_to_the_even_code():
    t = F.e4m3_value_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)       # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (t[:-1] + t[1:]) / 2)
    codes = F.e4m3_encode(mids)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, expect)
    assert np.array_equal(F.e4m3_encode(-mids), expect | 0x80)
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_encode_saturates_and_keeps_nan_and_signed_zero():
    x = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, np.inf, -1e9, np.nan, -0.0, 0.0],
                 dtype=np.float32)
    c = F.e4m3_encode(x)
    assert c.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F, 0x80, 0x00]


def test_every_finite_code_survives_a_round_trip():
    t = F.e4m3_value_table()
    finite = [c for c in range(256) if not np.isnan(t[c])]
    assert F.e4m3_encode(t[finite].astype(np.float32)).tolist() == finite


def test_quantize_divides_in_fp32():
    """The quotient is rounded to fp32 before the e4m3 rounding: a value
    whose exact quotient lies just past a midpoint but whose fp32 quotient
    lands on it goes to the even code."""
    mid = np.float32(1.0 + 1.0 / 16.0)               # midpoint of 1.0 and 1.125
    scale = np.float32(3.0)
    x = np.float32(mid * scale)                      # 3.1875: exact
    assert float(np.float32(x) / scale) == float(mid)
    assert F.quantize(np.array([x]), scale).tolist() == [0x38]       # 1.0 (even)
    x2 = np.nextafter(x, np.float32(10.0))
    assert F.quantize(np.array([x2]), scale).tolist() == [0x39]      # 1.125


def test_scatter_places_quantised_rows_and_skips_negative_slots():
    rng = np.random.default_rng(1)
    nb, bs, hkv, d = 6, 4, 2, 8
    kc = np.full((nb, bs, hkv, d), 0x7F, dtype=np.uint8)
    vc = kc.copy()
    key = torch.from_numpy(rng.standard_normal((3, hkv, d)).astype(np.float32)).to(torch.bfloat16)
    val = torch.from_numpy(rng.standard_normal((3, hkv, d)).astype(np.float32)).to(torch.bfloat16)
    ks, vs = np.array([0.01, 0.02], np.float32), np.array([0.5, 0.25], np.float32)
    slots = np.array([5, -1, 22])
    k2, v2 = F.reshape_and_cache_fp8(key, val, kc, vc, slots, ks, vs)
    assert np.array_equal(k2[1, 1], F.quantize(key[0], ks.reshape(2, 1)))
    assert np.array_equal(v2[5, 2], F.quantize(val[2], vs.reshape(2, 1)))
    touched = np.zeros((nb, bs), bool)
    touched[1, 1] = touched[5, 2] = True
    assert np.all(k2[~touched] == 0x7F) and np.all(v2[~touched] == 0x7F)
    # the stored codes stand for the inputs within half an e4m3 step
    back = F.e4m3_decode(k2[1, 1]) * ks.reshape(2, 1)
    x = key[0].float().numpy()
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -4 + 2.0 ** -10 * ks.reshape(2, 1))


def _pool_of_small_integers(rng, nb, bs, hkv, d):
    return rng.integers(-8, 9, size=(nb, bs, hkv, d)).astype(np.float32)


def test_attention_over_exact_values_equals_decode():
    """K and V made of small integers are held exactly by e4m3 (scale 1): the
    fp8 attention equals the decode oracle on the original values; with
    other scales the pools are the same values times the scales."""
    rng = np.random.default_rng(2)
    nb, bs, hkv, d, H = 12, 4, 2, 16, 4
    K = _pool_of_small_integers(rng, nb, bs, hkv, d)
    V = _pool_of_small_integers(rng, nb, bs, hkv, d)
    q = torch.from_numpy(rng.standard_normal((3, H, d)).astype(np.float32) * 0.1)
    bt = np.array([[3, 7, 1], [0, 2, 4], [11, 5, 6]], dtype=np.int32)
    lens = np.array([9, 12, 1], dtype=np.int32)
    ones = np.ones(hkv, np.float32)
    kq, vq = F.e4m3_encode(K), F.e4m3_encode(V)
    got = F.decode_fp8(q, kq, vq, ones, ones, bt, lens, 0.25)
    ref = oracle.decode(q, torch.from_numpy(K), torch.from_numpy(V), bt, lens, 0.25)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    # k_scale c with scale / c is the same attention; v_scale scales the output
    ks = np.array([2.0, 0.5], np.float32)
    vs = np.array([4.0, 0.125], np.float32)
    got2 = F.decode_fp8(q, kq, vq, ks, vs, bt, lens, 0.25)
    ref2 = oracle.decode(q, torch.from_numpy(K * ks.reshape(1, 1, 2, 1)),
                         torch.from_numpy(V * vs.reshape(1, 1, 2, 1)), bt, lens, 0.25)
    assert np.allclose(got2, ref2, rtol=0, atol=1e-12)
    vs_h = np.repeat(vs, H // hkv).reshape(1, H, 1)
    assert np.allclose(F.decode_fp8(q, kq, vq, ones, vs, bt, lens, 0.25), got * vs_h,
                       rtol=0, atol=1e-12)


def test_multi_query_fp8_row_is_decode_fp8_of_its_prefix():
    rng = np.random.default_rng(3)
    nb, bs, hkv, d, H, Q = 10, 4, 2, 16, 4, 3
    kq = F.e4m3_encode(rng.standard_normal((nb, bs, hkv, d)).astype(np.float32))
    vq = F.e4m3_encode(rng.standard_normal((nb, bs, hkv, d)).astype(np.float32))
    q = torch.from_numpy(rng.standard_normal((2, Q, H, d)).astype(np.float32))
    bt = np.array([[3, 7, 1, 9], [0, 2, 4, 8]], dtype=np.int32)
    lens = np.array([11, 16], dtype=np.int32)
    ks, vs = np.array([0.7, 1.3], np.float32), np.array([0.9, 2.0], np.float32)
    out = F.multi_query_fp8(q, kq, vq, ks, vs, bt, lens, 0.3)
    for j in range(Q):
        ref = F.decode_fp8(q[:, j], kq, vq, ks, vs, bt, lens - Q + j + 1, 0.3)
        assert np.allclose(out[:, j], ref, rtol=0, atol=1e-12)


def test_shared_prefix_fp8_is_decode_fp8_over_the_joined_tables():
    """Two groups of two samples: each sample's row equals decode over its
    group's prefix blocks followed by its own, with the same scales."""
    rng = np.random.default_rng(8)
    nb, bs, hkv, d, H = 12, 4, 2, 16, 4
    kq = F.e4m3_encode(rng.standard_normal((nb, bs, hkv, d)).astype(np.float32))
    vq = F.e4m3_encode(rng.standard_normal((nb, bs, hkv, d)).astype(np.float32))
    q = torch.from_numpy(rng.standard_normal((4, H, d)).astype(np.float32))
    ks, vs = np.array([0.5, 1.5], np.float32), np.array([1.25, 0.75], np.float32)
    pt = np.array([[5, 2], [9, 0]], dtype=np.int32)
    pl = np.array([8, 4], dtype=np.int32)
    st = np.array([[1, 3], [7, 0], [11, 0], [6, 10]], dtype=np.int32)
    sl = np.array([5, 3, 0, 8], dtype=np.int32)
    out = F.decode_shared_prefix_fp8(q, kq, vq, ks, vs, pt, pl, st, sl, 2, 0.4)
    joined = np.array([[5, 2, 1, 3], [5, 2, 7, 0], [9, 11, 0, 0], [9, 6, 10, 0]], dtype=np.int32)
    lens = np.array([13, 11, 4, 12], dtype=np.int32)
    ref = F.decode_fp8(q, kq, vq, ks, vs, joined, lens, 0.4)
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def _table_pins_hold(t) -> bool:
    """The landmark and torch checks above, on a given value table."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ok = ~np.isnan(ref)
    return bool(t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6 and t[0x38] == 1.0
                and t[0x7E] == 448.0 and np.array_equal(np.isnan(t), ~ok)
                and np.array_equal(t[ok], ref[ok]))


def _encoder_pins_hold(enc) -> bool:
    """The midpoint, saturation and round-trip checks above, on an encoder."""
    t = F.e4m3_value_table()
    mids = ((t[:0x7E] + t[1:0x7F]) / 2).astype(np.float32)
    lo = np.arange(0x7E)
    finite = [c for c in range(256) if not np.isnan(t[c])]
    return bool(np.array_equal(enc(mids), np.where(lo % 2 == 0, lo, lo + 1))
                and enc(np.array([500.0, -1e9], np.float32)).tolist() == [0x7E, 0xFE]
                and enc(t[finite].astype(np.float32)).tolist() == finite)


def test_table_and_encoder_pins_hold_for_the_oracle():
    assert _table_pins_hold(F.e4m3_value_table())
    assert _encoder_pins_hold(F.e4m3_encode)


@pytest.mark.parametrize("mistake", ["scales_swapped", "scale_divides", "bias_8", "no_subnormals",
                                     "ties_away", "no_saturation"])
def test_pins_catch_planted_mistakes(mistake, monkeypatch):
    """Each plausible slip in the fp8 oracle fails one of the pins above."""
    t = F.e4m3_value_table()
    if mistake == "bias_8":
        assert not _table_pins_hold(np.array([v / 2 for v in t]))
        return
    if mistake == "no_subnormals":
        wrong = t.copy()
        wrong[1:8] = 0.0
        assert not _table_pins_hold(wrong)
        return
    if mistake == "ties_away":
        def enc(x):
            a = np.abs(np.asarray(x, np.float64))
            c = np.array([int(np.argmin(np.abs(t[:0x7F] - v) - 1e-300 * np.arange(0x7F)))
                          for v in a], dtype=np.uint8)          # ties to the larger code
            return np.where(a >= 448, np.uint8(0x7E), c) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
        assert not _encoder_pins_hold(enc)
        return
    if mistake == "no_saturation":
        def enc(x):
            x = np.asarray(x, np.float32)
            return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert not _encoder_pins_hold(enc)
        return
    rng = np.random.default_rng(4)
    nb, bs, hkv, d, H = 8, 4, 2, 16, 2
    K = _pool_of_small_integers(rng, nb, bs, hkv, d)
    V = _pool_of_small_integers(rng, nb, bs, hkv, d)
    kq, vq = F.e4m3_encode(K), F.e4m3_encode(V)
    q = torch.from_numpy(rng.standard_normal((2, H, d)).astype(np.float32) * 0.2)
    bt = np.array([[1, 2], [3, 4]], dtype=np.int32)
    lens = np.array([7, 8], dtype=np.int32)
    ks, vs = np.array([2.0, 0.5], np.float32), np.array([4.0, 0.125], np.float32)
    ref = oracle.decode(q, torch.from_numpy(K * ks.reshape(1, 1, 2, 1)),
                        torch.from_numpy(V * vs.reshape(1, 1, 2, 1)), bt, lens, 0.25)
    if mistake == "scales_swapped":
        bad = F.decode_fp8(q, kq, vq, vs, ks, bt, lens, 0.25)
    else:  # scale_divides
        bad = F.decode_fp8(q, kq, vq, 1 / ks, 1 / vs, bt, lens, 0.25)
    assert not np.allclose(bad, ref, atol=1e-6)
