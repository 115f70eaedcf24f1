"""Pins for the fp8 (E4M3) part of the CPU oracle.

Sources of truth used here, none of them the oracle itself:
* torch's float8_e4m3fn dtype (a library implementation of the same OCP
  format) for the value of every code and for round-to-nearest-even casts
  of in-range values;
* the format's closed forms (1.0, 448, the subnormal step 2^-9, the NaN
  codes, the count of finite codes);
* the rounding error bound (half the spacing of neighbouring codes);
* hand-computed attention results for two-token contexts, where each scale
  enters the closed form;
* textbook attention written out with dense matrices over values that torch
  dequantizes (torch quantizes, torch gives each code's value): causal
  prefill masked with np.triu, and decode by scalar loops, both with several
  q heads per kv head, every query row and a prior context;
* GQA equal to MHA with the kv heads replicated.
The last tests plant mistakes in the oracle and check that a pin fails.
"""

import math

import numpy as np
import pytest
import torch

import oracle.fp8 as f8
from oracle.paged_attention import BLOCK_SIZE
from workloads import bf16_bits_from_f32, make_tiny_decode, make_tiny_prefill


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
# attention over fp8 pools against textbook attention over torch's values

# scales that keep N(0, 1) draws far inside +-448 (no saturation, which
# torch's cast does not do), neither a power of two
PIN_K_SCALE = np.float32(0.05)
PIN_V_SCALE = np.float32(0.04)


def _bf16_f32(raw):
    return (np.asarray(raw).astype(np.uint32) << 16).view(np.float32)


def torch_dequant(raw, scale):
    """Value each bf16 input stands for once stored in an fp8 pool: x / scale
    in fp32, cast to E4M3 by torch, the code's value (torch) times scale."""
    codes = torch_codes(_bf16_f32(raw) / np.float32(scale))
    return torch_values()[codes] * float(np.float32(scale))


def _fp8_pools(wl):
    pk = f8.new_pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, 0x7F)
    pv = f8.new_pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, 0x7F)
    for k, v, sl in ((wl.hist_k, wl.hist_v, wl.hist_slots), (wl.new_k, wl.new_v, wl.new_slots)):
        f8.reshape_and_cache(pk, pv, k, v, sl, PIN_K_SCALE, PIN_V_SCALE)
    return pk, pv


def _pin_prefill():
    return make_tiny_prefill(seed=31, prior=(0, 21, 40), chunk=(7, 16, 9), Hq=8, Hkv=2, D=16,
                             dtype="bf16")


def textbook_causal_fp8(wl):
    """softmax(scale Q K^T + causal mask) V per request and head, dense, the
    mask from np.triu over the request's full context, K and V from torch's
    dequantization of the request's logical-order rows."""
    Tq, Hq, D = wl.q.shape
    Hkv = wl.num_kv_heads
    G = Hq // Hkv
    sc = float(np.float32(wl.scale))
    out = np.zeros((Tq, Hq, D))
    koff = 0
    for r in range(wl.num_reqs):
        lo, hi = int(wl.query_start_loc[r]), int(wl.query_start_loc[r + 1])
        n_r, ctx = hi - lo, int(wl.context_lens[r])
        prior = ctx - n_r
        K = torch_dequant(np.concatenate([wl.hist_k[koff: koff + prior], wl.new_k[lo:hi]]), PIN_K_SCALE)
        V = torch_dequant(np.concatenate([wl.hist_v[koff: koff + prior], wl.new_v[lo:hi]]), PIN_V_SCALE)
        koff += prior
        Q = _bf16_f32(wl.q[lo:hi]).astype(np.float64)
        hidden = np.triu(np.ones((n_r, ctx), dtype=bool), k=prior + 1)
        for h in range(Hq):
            Z = sc * (Q[:, h, :] @ K[:, h // G, :].T)
            Z[hidden] = -np.inf
            P = np.exp(Z - Z.max(axis=1, keepdims=True))
            out[lo:hi, h] = (P / P.sum(axis=1, keepdims=True)) @ V[:, h // G, :]
    return out


def check_fp8_prefill_textbook(wl):
    pk, pv = _fp8_pools(wl)
    got = f8.prefill_attention(wl.q, pk, pv, wl.block_tables, wl.query_start_loc, wl.context_lens,
                               wl.scale, PIN_K_SCALE, PIN_V_SCALE)
    err = np.max(np.abs(got - textbook_causal_fp8(wl)))
    assert err <= 1e-12, f"fp8 prefill vs textbook: {err}"


def test_fp8_prefill_equals_textbook_causal_attention():
    check_fp8_prefill_textbook(_pin_prefill())


def _pin_decode():
    return make_tiny_decode(seed=33, ctx=(1, 16, 23, 50), Hq=8, Hkv=2, D=16, dtype="bf16")


def scalar_decode_fp8(wl):
    """Decode attention by scalar loops (math.fsum) over torch-dequantized
    logical-order K/V; q head h reads kv head h // G."""
    S, Hq, D = wl.q.shape
    Hkv = wl.num_kv_heads
    G = Hq // Hkv
    sc = float(np.float32(wl.scale))
    res = np.zeros((S, Hq, D))
    off = 0
    for s, n in enumerate(int(c) for c in wl.context_lens):
        K = torch_dequant(np.concatenate([wl.hist_k[off: off + n - 1], wl.new_k[s: s + 1]]), PIN_K_SCALE)
        V = torch_dequant(np.concatenate([wl.hist_v[off: off + n - 1], wl.new_v[s: s + 1]]), PIN_V_SCALE)
        off += n - 1
        qf = _bf16_f32(wl.q[s]).astype(np.float64)
        for h in range(Hq):
            g = h // G
            z = [sc * math.fsum(qf[h, x] * K[t, g, x] for x in range(D)) for t in range(n)]
            m = max(z)
            e = [math.exp(zz - m) for zz in z]
            l = math.fsum(e)
            for x in range(D):
                res[s, h, x] = math.fsum(e[t] * V[t, g, x] for t in range(n)) / l
    return res


def check_fp8_decode_scalar(wl):
    pk, pv = _fp8_pools(wl)
    got = f8.decode_attention(wl.q, pk, pv, wl.block_tables, wl.context_lens, wl.scale,
                              PIN_K_SCALE, PIN_V_SCALE)
    err = np.max(np.abs(got - scalar_decode_fp8(wl)))
    assert err <= 1e-12, f"fp8 decode vs scalar loops: {err}"


def test_fp8_decode_equals_scalar_attention_with_gqa():
    check_fp8_decode_scalar(_pin_decode())


def check_fp8_gqa_equals_mha(wl):
    pk, pv = _fp8_pools(wl)
    G = wl.num_q_heads // wl.num_kv_heads
    gqa = f8.decode_attention(wl.q, pk, pv, wl.block_tables, wl.context_lens, wl.scale,
                              PIN_K_SCALE, PIN_V_SCALE)
    mha = f8.decode_attention(wl.q, np.repeat(pk, G, axis=2), np.repeat(pv, G, axis=2),
                              wl.block_tables, wl.context_lens, wl.scale, PIN_K_SCALE, PIN_V_SCALE)
    assert np.array_equal(gqa, mha)
    # and the same for every row of a prefill chunk
    wp = _pin_prefill()
    pk, pv = _fp8_pools(wp)
    Gp = wp.num_q_heads // wp.num_kv_heads
    a = f8.prefill_attention(wp.q, pk, pv, wp.block_tables, wp.query_start_loc, wp.context_lens,
                             wp.scale, PIN_K_SCALE, PIN_V_SCALE)
    b = f8.prefill_attention(wp.q, np.repeat(pk, Gp, axis=2), np.repeat(pv, Gp, axis=2),
                             wp.block_tables, wp.query_start_loc, wp.context_lens, wp.scale,
                             PIN_K_SCALE, PIN_V_SCALE)
    assert np.array_equal(a, b)


def test_fp8_gqa_equals_mha_with_replicated_kv_heads():
    check_fp8_gqa_equals_mha(_pin_decode())


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


def _plain_fp8_prefill(future=0, modmap=False):
    """A prefill over fp8 pools written out with its own loops, with one of
    two planted mistakes: each row sees ``future`` keys past its position,
    or q head h reads kv head h % Hkv."""
    def run(q, pool_k, pool_v, block_tables, query_start_loc, context_lens, scale, k_scale, v_scale,
            q_dtype="bf16", rows=None):
        Tq, Hq, D = q.shape
        Hkv = pool_k.shape[2]
        G = Hq // Hkv
        out = np.zeros((Tq, Hq, D))
        for r in range(len(context_lens)):
            lo, hi = int(query_start_loc[r]), int(query_start_loc[r + 1])
            ctx = int(context_lens[r])
            nb = (ctx + BLOCK_SIZE - 1) // BLOCK_SIZE
            ids = np.asarray(block_tables[r][:nb], dtype=np.int64)
            K = f8.dequantize(pool_k[ids].reshape(nb * BLOCK_SIZE, Hkv, D)[:ctx], k_scale)
            V = f8.dequantize(pool_v[ids].reshape(nb * BLOCK_SIZE, Hkv, D)[:ctx], v_scale)
            for i in range(hi - lo):
                pos = ctx - (hi - lo) + i
                qrow = _bf16_f32(q[lo + i]).astype(np.float64)
                for h in range(Hq):
                    g = h % Hkv if modmap else h // G
                    z = float(np.float32(scale)) * (K[: pos + 1 + future, g] @ qrow[h])
                    w = np.exp(z - z.max())
                    out[lo + i, h] = (w @ V[: pos + 1 + future, g]) / w.sum()
        return out
    return run


def test_planted_fp8_prefill_future_key_is_caught(monkeypatch):
    # the unplanted loops pass the pin: the mistake, not the rewrite, fails it
    monkeypatch.setattr(f8, "prefill_attention", _plain_fp8_prefill())
    check_fp8_prefill_textbook(_pin_prefill())
    monkeypatch.setattr(f8, "prefill_attention", _plain_fp8_prefill(future=1))
    with pytest.raises(AssertionError):
        check_fp8_prefill_textbook(_pin_prefill())


def test_planted_fp8_prefill_wrong_gqa_map_is_caught(monkeypatch):
    monkeypatch.setattr(f8, "prefill_attention", _plain_fp8_prefill(modmap=True))
    with pytest.raises(AssertionError):
        check_fp8_prefill_textbook(_pin_prefill())


def test_planted_fp8_decode_wrong_gqa_map_is_caught(monkeypatch):
    plain = _plain_fp8_prefill(modmap=True)

    def decode_modmap(q, pool_k, pool_v, block_tables, context_lens, scale, k_scale, v_scale,
                      q_dtype="bf16", seqs=None):
        # decode is a one-row chunk per sequence
        qsl = np.arange(q.shape[0] + 1, dtype=np.int32)
        return plain(q, pool_k, pool_v, block_tables, qsl, context_lens, scale, k_scale, v_scale)

    monkeypatch.setattr(f8, "decode_attention", decode_modmap)
    with pytest.raises(AssertionError):
        check_fp8_decode_scalar(_pin_decode())
    with pytest.raises(AssertionError):
        check_fp8_gqa_equals_mha(_pin_decode())
