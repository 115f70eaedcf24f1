"""Pins for the fp8 (E4M3) part of the CPU oracle.

Sources of truth used here, none of them the oracle itself:
* torch's float8_e4m3fn dtype (a library implementation of the same OCP
  format) for the value of every code and for round-to-nearest-even casts
  of in-range values;
* the format's closed forms (1.0, 448, the subnormal step 2^-9, the NaN
  codes, the count of finite codes);
* the rounding error bound (half the spacing of neighbouring codes);
* hand-computed attention results for two-token contexts, where each scale
  enters the closed form.
The last tests plant mistakes in the oracle and check that a pin fails.
"""

import math

import numpy as np
import pytest
import torch

import oracle.fp8 as f8
from oracle.paged_attention import BLOCK_SIZE
from workloads import bf16_bits_from_f32


def torch_values():
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_codes(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


# ----------------------------------------------------------------------------
# the code table


def test_table_matches_torch_e4m3fn():
    ref = torch_values()
    mine = f8.E4M3_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    # signed zeros too
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(mine[ok]))


@pytest.mark.parametrize("code,val", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0),
])
def test_closed_form_values(code, val):
    assert f8.e4m3_value(code) == val


def test_nan_codes_and_finite_count():
    assert math.isnan(f8.e4m3_value(0x7F)) and math.isnan(f8.e4m3_value(0xFF))
    assert np.isfinite(f8.E4M3_TABLE).sum() == 254
    assert math.copysign(1.0, f8.e4m3_value(0x80)) == -1.0


# ----------------------------------------------------------------------------
# encoding


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-14, np.log2(448.0), size=200_000)).astype(np.float32)
    x = (mags * rng.choice([-1, 1], size=mags.shape)).astype(np.float32)
    assert np.array_equal(f8.encode_f32(x), torch_codes(x))


def test_ties_go_to_even_codes():
    fin = f8.E4M3_TABLE[:0x7F]
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (fin[:-1] + fin[1:]) / 2)  # exact in fp32
    codes = f8.encode_f32(np.concatenate([mids, -mids]))
    assert np.all(codes % 2 == 0)
    assert np.array_equal(codes, torch_codes(np.concatenate([mids, -mids])))
    # worked cases: 1.0625 lies between 1.0 (0x38) and 1.125 (0x39)
    assert f8.encode_f32(np.float32(1.0625)) == 0x38
    assert f8.encode_f32(np.float32(1.1875)) == 0x3A  # between 1.125 and 1.25
    assert f8.encode_f32(np.float32(2.0 ** -10)) == 0x00  # between 0 and 2^-9
    assert f8.encode_f32(np.float32(1.5 * 2.0 ** -10)) == 0x01


def test_saturation_and_special_inputs():
    x = np.array([448.0, 449.0, 464.0, 500.0, 1e30, np.inf, -449.0, -np.inf], dtype=np.float32)
    assert list(f8.encode_f32(x)) == [0x7E] * 6 + [0xFE] * 2
    assert f8.encode_f32(np.float32(np.nan)) == 0x7F
    assert f8.encode_f32(np.float32(-1e-5)) == 0x80
    assert f8.encode_f32(np.float32(-0.0)) == 0x80
    assert f8.encode_f32(np.float32(0.0)) == 0x00


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(f8.encode_f32(f8.decode(codes).astype(np.float32)), codes)


def test_encoding_is_monotone_and_within_half_a_step():
    x = np.sort(np.random.default_rng(1).uniform(-460, 460, size=100_000)).astype(np.float32)
    v = f8.decode(f8.encode_f32(x))
    assert np.all(np.diff(v) >= 0)
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    # spacing of E4M3 at magnitude a: 2^-9 below 2^-6, else 2^(floor(log2 a) - 3)
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(np.abs(v) - a) <= step / 2)


def test_quantize_divides_in_fp32():
    # The code is the one of the fp32 quotient x / scale.  With scale =
    # fl32(x / m) for a midpoint m between two codes, the fp32 quotient often
    # lands exactly on m (a tie, so the even code) while the exact quotient
    # lies a little to one side, where a float64 division would pick the
    # nearer code: for some of these cases the odd one.
    fin = f8.E4M3_TABLE[:0x7F]
    tried = differs = 0
    for x in np.array([1.0, 3.0, -5.0, 0.75, 7.0, 2.5], dtype=np.float32):
        for lo in range(8, 0x7E, 7):
            m = (fin[lo] + fin[lo + 1]) / 2
            s = np.float32(float(x) / m)
            q32 = np.float32(x) / s
            q64 = float(x) / float(s)
            if float(abs(q32)) != m or abs(q64) == m:
                continue
            tried += 1
            code = int(f8.quantize(bf16_bits_from_f32(np.array([x], dtype=np.float32)), "bf16", s)[0])
            assert code == int(torch_codes(np.array([q32]))[0])
            assert (code & 0x7F) == (lo if lo % 2 == 0 else lo + 1)
            differs += (code & 0x7F) != (lo + 1 if abs(q64) > m else lo)
    assert tried > 10 and differs > 0


# ----------------------------------------------------------------------------
# cache write and attention


def _tiny_pools(D=16, Hkv=1):
    pk = f8.new_pool(3, Hkv, D, 0x7F)
    pv = f8.new_pool(3, Hkv, D, 0x7F)
    return pk, pv


def test_cache_write_stores_codes_in_slots_and_skips_negative():
    D = 16
    pk, pv = _tiny_pools(D)
    vals = np.linspace(-3, 3, 3 * D, dtype=np.float32).reshape(3, 1, D)
    k = bf16_bits_from_f32(vals)
    v = bf16_bits_from_f32(-vals)
    f8.reshape_and_cache(pk, pv, k, v, np.array([17, -1, 2]), 0.05, 0.1)
    want_k = torch_codes((k.astype(np.uint32) << 16).view(np.float32) / np.float32(0.05))
    assert np.array_equal(pk[1, 1], want_k[0])
    assert np.array_equal(pk[0, 2], want_k[2])
    assert np.all(pv[0, 1] == 0x7F)  # slot of the padding token stays untouched
    assert np.all(pk[0, 0] == 0x7F)


def _two_token(k_scale, v_scale, scale, kc=(0x38, 0x40), vc=(0x38, 0x48)):
    """One sequence, two tokens, D = 16, one head; q = e_0."""
    D = 16
    pk, pv = _tiny_pools(D)
    for t in range(2):
        pk[0, t, 0, :] = 0
        pk[0, t, 0, 0] = kc[t]
        pv[0, t, 0, :] = vc[t]
    q = np.zeros((1, 1, D), dtype=np.uint16)
    q[0, 0, 0] = 0x3F80  # bf16 1.0
    return f8.decode_attention(q, pk, pv, np.array([[0]], dtype=np.int32), np.array([2]), scale,
                               k_scale, v_scale)


def test_decode_two_token_closed_form():
    # keys 1.0 and 2.0 (times k_scale 0.5) give dots 0.5 and 1.0; with
    # scale = 2 ln 3 the weights are 1/4 and 3/4.  Values 1.0 and 4.0 times
    # v_scale 0.25 give 0.25 and 1.0: the output is 0.0625 + 0.75 = 0.8125.
    out = _two_token(0.5, 0.25, np.float32(2 * math.log(3)))
    sc = float(np.float32(2 * math.log(3)))
    w2 = 1 / (1 + math.exp(-0.5 * sc))
    assert abs(out[0, 0, 0] - ((1 - w2) * 0.25 + w2 * 1.0)) < 1e-15
    assert abs(out[0, 0, 0] - 0.8125) < 1e-6


def test_decode_equal_keys_gives_mean_of_dequantized_values():
    rng = np.random.default_rng(3)
    D, n = 32, 37
    pk = f8.new_pool(4, 1, D, 0x38)  # every key 1.0
    pv = f8.new_pool(4, 1, D, 0x00)
    codes = rng.integers(0, 0x7F, size=(n, D), dtype=np.uint8) | (rng.integers(0, 2, size=(n, D), dtype=np.uint8) << 7)
    table = np.array([[2, 0, 3]], dtype=np.int32)
    for t in range(n):
        pv[table[0, t // BLOCK_SIZE], t % BLOCK_SIZE, 0] = codes[t]
    q = bf16_bits_from_f32(rng.standard_normal((1, 1, D)).astype(np.float32))
    out = f8.decode_attention(q, pk, pv, table, np.array([n]), 0.125, 0.7, 0.03)
    want = np.array([[sum(f8.e4m3_value(codes[t, x]) for t in range(n)) / n * float(np.float32(0.03))
                      for x in range(D)]])
    assert np.allclose(out[0], want, rtol=0, atol=1e-14)


def test_prefill_last_row_equals_decode():
    rng = np.random.default_rng(5)
    D, Hkv, Hq, ctx, n_r = 16, 2, 4, 40, 5
    pk = rng.integers(0, 0x7F, size=(4, BLOCK_SIZE, Hkv, D), dtype=np.uint8)
    pv = rng.integers(0, 0x7F, size=(4, BLOCK_SIZE, Hkv, D), dtype=np.uint8) ^ np.uint8(0x80)
    table = np.array([[3, 1, 0]], dtype=np.int32)
    q = bf16_bits_from_f32(rng.standard_normal((n_r, Hq, D)).astype(np.float32))
    pf = f8.prefill_attention(q, pk, pv, table, np.array([0, n_r]), np.array([ctx]), 0.25, 0.02, 0.05)
    dc = f8.decode_attention(q[n_r - 1: n_r], pk, pv, table, np.array([ctx]), 0.25, 0.02, 0.05)
    assert np.allclose(pf[n_r - 1], dc[0], rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------
# planted mistakes


def test_planted_missing_k_scale_is_caught(monkeypatch):
    orig = f8.dequantize
    monkeypatch.setattr(f8, "dequantize", lambda c, s: orig(c, 1.0 if float(s) == 0.5 else s))
    with pytest.raises(AssertionError):
        test_decode_two_token_closed_form()


def test_planted_ties_away_from_zero_is_caught(monkeypatch):
    def bad(x):
        x = np.asarray(x, dtype=np.float32)
        a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
        fin = f8.E4M3_TABLE[:0x7F]
        hi = np.clip(np.searchsorted(fin, a), 0, 0x7E)
        lo = np.maximum(hi - 1, 0)
        mag = np.where(fin[hi] - a <= a - fin[lo], hi, lo).astype(np.uint8)
        return mag | ((x.view(np.uint32) >> 31).astype(np.uint8) << 7)

    monkeypatch.setattr(f8, "encode_f32", bad)
    with pytest.raises(AssertionError):
        test_ties_go_to_even_codes()


def test_planted_wrong_exponent_bias_is_caught(monkeypatch):
    bad = f8.E4M3_TABLE * 2.0
    monkeypatch.setattr(f8, "E4M3_TABLE", bad)
    with pytest.raises(AssertionError):
        test_table_matches_torch_e4m3fn()
