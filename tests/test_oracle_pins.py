"""Pins for the CPU oracle: each checks it against something other than itself.

Sources of truth used here:
* IEEE-754 closed forms for the raw-bit decoding;
* brute-force, unpaged attention written as scalar Python loops with
  ``math.exp`` / ``math.fsum`` on the generator's logical-order tensors;
* invariants the pages imply: paging only moves bytes (physical permutation
  and shared blocks change nothing), softmax weights sum to one;
* closed forms (zero scale gives the mean of V, one token returns its V row);
* the online-softmax rescale identity (zihan-zhang.net vLLM study, 4.3.1);
* the textbook masked causal attention (same page, 1.1.1) for prefill;
* the block and byte counts the pages print (tests/golden/).

The last group plants mistakes in the oracle and checks that a pin fails.
"""

import math

import numpy as np
import pytest

import oracle
from workloads import make_tiny_decode, make_tiny_prefill, make_tiny_shared, poison_bits


# ----------------------------------------------------------------------------
# helpers


def build_pools(wl, fast=False):
    pk = oracle.new_pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype, poison_bits(wl.dtype))
    pv = oracle.new_pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype, poison_bits(wl.dtype))
    write = oracle.reshape_and_cache_fast if fast else oracle.reshape_and_cache
    write(pk, pv, wl.hist_k, wl.hist_v, wl.hist_slots)
    write(pk, pv, wl.new_k, wl.new_v, wl.new_slots)
    return pk, pv


def logical_kv(wl):
    """Per-sequence raw K/V in logical order, straight from the generator (no
    paging): history rows of sequence s are its positions 0..ctx-2 in order,
    followed (for the next sequence) by the next sequence's; the new row is
    position ctx-1.  Valid for workloads without shared prompts."""
    out = []
    off = 0
    for s, n in enumerate(wl.context_lens):
        n = int(n)
        K = np.concatenate([wl.hist_k[off: off + n - 1], wl.new_k[s: s + 1]])
        V = np.concatenate([wl.hist_v[off: off + n - 1], wl.new_v[s: s + 1]])
        off += n - 1
        out.append((K, V))
    return out


def as_float(raw, dtype):
    """Scalar IEEE decoding via struct, independent of ``oracle.widen``."""
    import struct

    if dtype == "bf16":
        return [struct.unpack("<f", struct.pack("<I", int(r) << 16))[0] for r in np.ravel(raw)]
    return [struct.unpack("<f", struct.pack("<I", int(r)))[0] for r in np.ravel(raw)]


def brute_decode(wl):
    """Dense attention by scalar loops over the unpaged logical tensors."""
    S, Hq, D = wl.q.shape
    G = Hq // wl.num_kv_heads
    scale = float(np.float32(wl.scale))
    res = np.zeros((S, Hq, D))
    for s, (K, V) in enumerate(logical_kv(wl)):
        n = K.shape[0]
        qf = np.array(as_float(wl.q[s], wl.dtype)).reshape(Hq, D)
        Kf = np.array(as_float(K, wl.dtype)).reshape(n, wl.num_kv_heads, D)
        Vf = np.array(as_float(V, wl.dtype)).reshape(n, wl.num_kv_heads, D)
        for h in range(Hq):
            g = h // G
            z = [scale * math.fsum(qf[h, x] * Kf[t, g, x] for x in range(D)) for t in range(n)]
            m = max(z)
            e = [math.exp(zz - m) for zz in z]
            l = math.fsum(e)
            for x in range(D):
                res[s, h, x] = math.fsum(e[t] * Vf[t, g, x] for t in range(n)) / l
    return res


def check_bruteforce(wl, tol=1e-12):
    pk, pv = build_pools(wl)
    got = oracle.decode(wl.q, pk, pv, wl.block_tables, wl.context_lens, wl.scale, wl.dtype)
    ref = brute_decode(wl)
    err = np.max(np.abs(got - ref))
    assert err <= tol, f"oracle vs brute force: max abs err {err}"


def textbook_causal(wl):
    """softmax(Q K^T * scale + causal mask) V per request and head, with the
    mask built by np.triu over the request's full context; dense matrices."""
    Tq, Hq, D = wl.q.shape
    G = Hq // wl.num_kv_heads
    sc = float(np.float32(wl.scale))
    out = np.zeros((Tq, Hq, D))
    koff = 0
    for r in range(wl.num_reqs):
        lo, hi = int(wl.query_start_loc[r]), int(wl.query_start_loc[r + 1])
        n_r = hi - lo
        ctx = int(wl.context_lens[r])
        prior = ctx - n_r
        Kraw = np.concatenate([wl.hist_k[koff: koff + prior], wl.new_k[lo:hi]])
        Vraw = np.concatenate([wl.hist_v[koff: koff + prior], wl.new_v[lo:hi]])
        koff += prior
        K = np.array(as_float(Kraw, wl.dtype)).reshape(ctx, wl.num_kv_heads, D)
        V = np.array(as_float(Vraw, wl.dtype)).reshape(ctx, wl.num_kv_heads, D)
        Q = np.array(as_float(wl.q[lo:hi], wl.dtype)).reshape(n_r, Hq, D)
        # key t is hidden from query i when t > prior + i
        hidden = np.triu(np.ones((n_r, ctx), dtype=bool), k=prior + 1)
        for h in range(Hq):
            g = h // G
            Z = sc * (Q[:, h, :] @ K[:, g, :].T)
            Z[hidden] = -np.inf
            Z = Z - Z.max(axis=1, keepdims=True)
            P = np.exp(Z)
            P /= P.sum(axis=1, keepdims=True)
            out[lo:hi, h] = P @ V[:, g, :]
    return out


def build_prefill_pools(wl):
    pk = oracle.new_pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype, poison_bits(wl.dtype))
    pv = oracle.new_pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype, poison_bits(wl.dtype))
    oracle.reshape_and_cache(pk, pv, wl.hist_k, wl.hist_v, wl.hist_slots)
    oracle.reshape_and_cache(pk, pv, wl.new_k, wl.new_v, wl.new_slots)
    return pk, pv


def check_prefill_textbook(wl, tol=1e-12):
    pk, pv = build_prefill_pools(wl)
    got = oracle.prefill_chunk(wl.q, pk, pv, wl.block_tables, wl.query_start_loc,
                               wl.context_lens, wl.scale, wl.dtype)
    ref = textbook_causal(wl)
    err = np.max(np.abs(got - ref))
    assert err <= tol, f"prefill oracle vs textbook: {err}"


# ----------------------------------------------------------------------------
# raw decoding: IEEE-754 closed forms


@pytest.mark.parametrize("bits,val", [(0x3F80, 1.0), (0xC000, -2.0), (0x3F81, 1.0 + 2.0 ** -7),
                                      (0x0001, 2.0 ** -133), (0x7F80, math.inf),
                                      (0x8000, -0.0), (0x4049, 3.140625)])
def test_widen_bf16_closed_forms(bits, val):
    got = oracle.widen(np.array([bits], np.uint16), "bf16")[0]
    assert got == val and math.copysign(1, got) == math.copysign(1, val)


@pytest.mark.parametrize("bits,val", [(0x3F800000, 1.0), (0x00000001, 2.0 ** -149),
                                      (0xBF000000, -0.5), (0x3F800001, 1.0 + 2.0 ** -23)])
def test_widen_f32_closed_forms(bits, val):
    assert oracle.widen(np.array([bits], np.uint32), "f32")[0] == val


# ----------------------------------------------------------------------------
# cache write + addressing


def test_write_then_gather_round_trip():
    """Tokens written through slot_mapping come back in logical order through
    the block table; exactly the targeted slots change; the rest stay poison."""
    wl = make_tiny_decode(seed=3, ctx=(1, 16, 17, 32, 33, 100), Hq=2, Hkv=2, D=4, dtype="f32")
    # tag every token's row with a unique integer so the check is on identity
    Th = wl.hist_k.shape[0]
    wl.hist_k = np.arange(Th * 2 * 4, dtype=np.uint32).reshape(Th, 2, 4)
    wl.hist_v = wl.hist_k + np.uint32(1 << 30)
    wl.new_k = (np.arange(wl.num_seqs * 8, dtype=np.uint32) + np.uint32(1 << 20)).reshape(-1, 2, 4)
    wl.new_v = wl.new_k + np.uint32(1 << 30)
    pk, pv = build_pools(wl)
    for s, (K, V) in enumerate(logical_kv(wl)):
        n = int(wl.context_lens[s])
        assert np.array_equal(oracle.gather(pk, wl.block_tables[s], n), K)
        assert np.array_equal(oracle.gather(pv, wl.block_tables[s], n), V)
    poison = poison_bits("f32")
    changed = (pk != poison).all(axis=(2, 3))
    assert changed.sum() == int(wl.context_lens.sum())
    assert ((pk == poison).all(axis=(2, 3)) | changed).all()


def test_negative_slots_write_nothing():
    pk = oracle.new_pool(4, 1, 2, "bf16", 0x7FA5)
    pv = oracle.new_pool(4, 1, 2, "bf16", 0x7FA5)
    k = np.array([[[1, 2]], [[3, 4]], [[5, 6]]], np.uint16)
    oracle.reshape_and_cache(pk, pv, k, k, np.array([-1, 17, -5], np.int64))
    assert (pk[1, 1, 0] == [3, 4]).all()
    assert (pk != 0x7FA5).sum() == 2


def test_fast_and_loop_cache_write_agree():
    wl = make_tiny_decode(seed=5, ctx=(7, 40, 64), Hq=4, Hkv=2, D=8, dtype="bf16")
    a = build_pools(wl, fast=False)
    b = build_pools(wl, fast=True)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_gather_reads_ceil_blocks_only():
    """A 32-token context with a table [a, b, -1]: two blocks, never the pad
    (the pages' loop bound seq_len // 16 + 1 would read a third one)."""
    pool = oracle.new_pool(3, 1, 1, "f32", 0)
    pool[:, :, 0, 0] = np.arange(48).reshape(3, 16)
    got = oracle.gather(pool, np.array([2, 0, -1], np.int32), 32)[:, 0, 0]
    assert got.tolist() == list(range(32, 48)) + list(range(0, 16))
    with pytest.raises(IndexError):
        oracle.gather(pool, np.array([2, 0, -1], np.int32), 33)


def test_physical_layout_matches_written_formula():
    """The pool byte orders equal the written index formulas, by explicit loops."""
    nb, hkv, d = 3, 2, 4
    pool = np.arange(nb * 16 * hkv * d, dtype=np.uint32).reshape(nb, 16, hkv, d)
    kb = oracle.k_pool_bytes(pool)
    vb = oracle.v_pool_bytes(pool)
    for b in range(nb):
        for o in range(16):
            for g in range(hkv):
                for x in range(d):
                    assert kb[((b * hkv + g) * 16 + o) * d + x] == pool[b, o, g, x]
                    assert vb[((b * hkv + g) * d + x) * 16 + o] == pool[b, o, g, x]
    assert np.array_equal(oracle.k_pool_from_bytes(kb, nb, hkv, d), pool)
    assert np.array_equal(oracle.v_pool_from_bytes(vb, nb, hkv, d), pool)


def test_address_rule_exhaustive():
    """Every logical index below 4096 lands where block_table[i // 16], i % 16
    says (vLLM: from PagedAttention to Speculative Decoding, 3.3)."""
    rng = np.random.default_rng(0)
    table = rng.permutation(300)[:256].astype(np.int32)
    pool = oracle.new_pool(300, 1, 1, "f32", 0xFFFFFFFF)
    slots = table[np.arange(4096) // 16].astype(np.int64) * 16 + np.arange(4096) % 16
    vals = np.arange(4096, dtype=np.uint32).reshape(4096, 1, 1)
    oracle.reshape_and_cache_fast(pool, pool.copy(), vals, vals, slots)
    got = oracle.gather(pool, table, 4096)[:, 0, 0]
    assert np.array_equal(got, np.arange(4096))


# ----------------------------------------------------------------------------
# attention values


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_oracle_matches_bruteforce_tiny(dtype):
    wl = make_tiny_decode(seed=1, ctx=(1, 5, 17, 33), Hq=4, Hkv=2, D=8, dtype=dtype)
    check_bruteforce(wl)


def test_oracle_matches_bruteforce_config1_shape():
    """The tiny fp32 benchmark shape: ctx {5,17,33,64}, 4q/2kv, d=64."""
    wl = make_tiny_decode(seed=9, ctx=(5, 17, 33, 64), Hq=4, Hkv=2, D=64, dtype="f32",
                          num_blocks=32)
    check_bruteforce(wl, tol=1e-12)


def test_permutation_of_physical_blocks_changes_nothing():
    a = make_tiny_decode(seed=2, ctx=(3, 16, 31, 77), Hq=4, Hkv=1, D=16, dtype="bf16", layout_variant=0)
    b = make_tiny_decode(seed=2, ctx=(3, 16, 31, 77), Hq=4, Hkv=1, D=16, dtype="bf16", layout_variant=1)
    assert not np.array_equal(a.block_tables, b.block_tables)
    ra = oracle.decode(a.q, *build_pools(a), a.block_tables, a.context_lens, a.scale, a.dtype)
    rb = oracle.decode(b.q, *build_pools(b), b.block_tables, b.context_lens, b.scale, b.dtype)
    assert np.array_equal(ra, rb)


def test_softmax_weights_sum_to_one():
    wl = make_tiny_decode(seed=4, ctx=(2, 19, 64, 65), Hq=4, Hkv=2, D=32, dtype="bf16")
    _, w = oracle.decode(wl.q, *build_pools(wl), wl.block_tables, wl.context_lens, wl.scale,
                         wl.dtype, return_weights=True)
    for (s, h), ws in w.items():
        assert ws.shape[0] == wl.context_lens[s]
        assert (ws >= 0).all()
        assert abs(math.fsum(ws) - 1.0) < 1e-12


def test_single_token_context_returns_its_v_row():
    wl = make_tiny_decode(seed=6, ctx=(1, 1, 1), Hq=4, Hkv=2, D=16, dtype="bf16")
    out = oracle.decode(wl.q, *build_pools(wl), wl.block_tables, wl.context_lens, wl.scale, wl.dtype)
    for s in range(3):
        for h in range(4):
            v = np.array(as_float(wl.new_v[s, h // 2], "bf16"))
            assert np.array_equal(out[s, h], v)


def test_shared_prefix_equals_private_copies():
    a = make_tiny_shared(private_copies=False)
    b = make_tiny_shared(private_copies=True)
    # the shared layout really shares: some block ids repeat across rows
    ids = a.block_tables[:, :2].ravel()
    assert len(set(ids.tolist())) < ids.size
    ra = oracle.decode(a.q, *build_pools(a), a.block_tables, a.context_lens, a.scale, a.dtype)
    rb = oracle.decode(b.q, *build_pools(b), b.block_tables, b.context_lens, b.scale, b.dtype)
    assert np.array_equal(ra, rb)


def test_gqa_equals_mha_with_replicated_kv_heads():
    wl = make_tiny_decode(seed=8, ctx=(9, 40), Hq=8, Hkv=2, D=16, dtype="f32")
    pk, pv = build_pools(wl)
    gqa = oracle.decode(wl.q, pk, pv, wl.block_tables, wl.context_lens, wl.scale, wl.dtype)
    # replicate kv head g into heads g*4 .. g*4+3 (contiguous groups)
    pk8 = np.repeat(pk, 4, axis=2)
    pv8 = np.repeat(pv, 4, axis=2)
    mha = oracle.decode(wl.q, pk8, pv8, wl.block_tables, wl.context_lens, wl.scale, wl.dtype)
    assert np.array_equal(gqa, mha)


def test_zero_scale_gives_mean_of_v_rows():
    wl = make_tiny_decode(seed=10, ctx=(7, 50), Hq=2, Hkv=1, D=8, dtype="f32")
    out = oracle.decode(wl.q, *build_pools(wl), wl.block_tables, wl.context_lens, 0.0, wl.dtype)
    for s, (K, V) in enumerate(logical_kv(wl)):
        Vf = np.array(as_float(V, "f32")).reshape(V.shape)
        assert np.allclose(out[s, 0], Vf[:, 0, :].mean(axis=0), rtol=0, atol=1e-13)


def test_constant_v_gives_that_constant():
    wl = make_tiny_decode(seed=12, ctx=(30,), Hq=2, Hkv=1, D=4, dtype="bf16")
    wl.hist_v[:] = 0x4040  # 3.0
    wl.new_v[:] = 0x4040
    out = oracle.decode(wl.q, *build_pools(wl), wl.block_tables, wl.context_lens, wl.scale, wl.dtype)
    assert np.allclose(out, 3.0, rtol=0, atol=1e-14)


def test_split_and_rescale_combine_matches_whole():
    """The online-softmax rescale (zihan-zhang.net vLLM study, 4.3.1), applied
    to arbitrary contiguous splits of one context and recombined, reaches the
    oracle's single-pass result; this is the identity split-K relies on."""
    wl = make_tiny_decode(seed=13, ctx=(300,), Hq=2, Hkv=1, D=16, dtype="bf16")
    pk, pv = build_pools(wl)
    whole = oracle.decode(wl.q, pk, pv, wl.block_tables, wl.context_lens, wl.scale, wl.dtype)
    K = oracle.widen(oracle.gather(pk, wl.block_tables[0], 300), "bf16")[:, 0, :]
    V = oracle.widen(oracle.gather(pv, wl.block_tables[0], 300), "bf16")[:, 0, :]
    sc = float(np.float32(wl.scale))
    rng = np.random.default_rng(0)
    for h in range(2):
        qv = oracle.widen(wl.q[0, h], "bf16")
        cuts = np.sort(rng.choice(np.arange(1, 300), size=6, replace=False))
        parts = np.split(np.arange(300), cuts)
        m, l, o = -np.inf, 0.0, np.zeros(16)
        for idx in parts:
            z = sc * (K[idx] @ qv)
            m_new = max(m, z.max())
            p = np.exp(z - m_new)
            alpha = math.exp(m - m_new) if m != -np.inf else 0.0
            o = o * alpha + p @ V[idx]
            l = l * alpha + p.sum()
            m = m_new
        assert np.max(np.abs(o / l - whole[0, h])) < 1e-12


# ----------------------------------------------------------------------------
# prefill


def test_prefill_prior_zero_equals_textbook_causal_attention():
    wl = make_tiny_prefill(seed=14, prior=(0, 0), chunk=(5, 21), Hq=4, Hkv=2, D=16, dtype="bf16")
    check_prefill_textbook(wl)


def test_prefill_with_prior_equals_textbook_causal_attention():
    wl = make_tiny_prefill(seed=15, prior=(0, 5, 40), chunk=(7, 16, 33), Hq=4, Hkv=2, D=16, dtype="f32")
    check_prefill_textbook(wl)


def test_prefill_last_row_equals_decode():
    wl = make_tiny_prefill(seed=16, prior=(3, 30), chunk=(9, 18), Hq=4, Hkv=2, D=16, dtype="bf16")
    pk, pv = build_prefill_pools(wl)
    pre = oracle.prefill_chunk(wl.q, pk, pv, wl.block_tables, wl.query_start_loc,
                               wl.context_lens, wl.scale, wl.dtype)
    last = wl.query_start_loc[1:] - 1
    dec = oracle.decode(wl.q[last], pk, pv, wl.block_tables, wl.context_lens, wl.scale, wl.dtype)
    assert np.array_equal(pre[last], dec)


def test_prefill_two_chunks_equal_one_chunk():
    wl = make_tiny_prefill(seed=17, prior=(10,), chunk=(40,), Hq=2, Hkv=1, D=16, dtype="bf16")
    pk, pv = build_prefill_pools(wl)
    whole = oracle.prefill_chunk(wl.q, pk, pv, wl.block_tables, wl.query_start_loc,
                                 wl.context_lens, wl.scale, wl.dtype)
    # first chunk: 15 queries ending at position 24; second: the remaining 25
    first = oracle.prefill_chunk(wl.q[:15], pk, pv, wl.block_tables, np.array([0, 15]),
                                 np.array([25]), wl.scale, wl.dtype)
    second = oracle.prefill_chunk(wl.q[15:], pk, pv, wl.block_tables, np.array([0, 25]),
                                  np.array([50]), wl.scale, wl.dtype)
    assert np.array_equal(np.concatenate([first, second]), whole)


# ----------------------------------------------------------------------------
# printed block and byte counts (tests/golden/page_counts.txt)


def _golden(name):
    import os

    rows = []
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_block_counts_printed_on_pages():
    from workloads import make_tiny_decode as mk

    for kind, tokens, blocks in _golden("block_counts.txt"):
        wl = mk(seed=1, ctx=(int(tokens),), Hq=1, Hkv=1, D=2, dtype="f32")
        assert int((wl.block_tables[0] >= 0).sum()) == int(blocks), kind


def test_kv_byte_accounting_printed_on_pages():
    for kind, layers, hkv, d, tokens, eb, expect in _golden("kv_bytes.txt"):
        wl = make_tiny_decode(seed=1, ctx=(int(tokens),), Hq=int(hkv), Hkv=int(hkv), D=int(d),
                              dtype="bf16" if int(eb) == 2 else "f32", num_blocks=None) \
            if int(tokens) <= 64 else None
        per_token_layer = 2 * int(hkv) * int(d) * int(eb)
        if wl is not None:
            assert wl.kv_bytes == per_token_layer * int(tokens)
        assert per_token_layer * int(layers) * int(tokens) == int(expect), kind


# ----------------------------------------------------------------------------
# planted mistakes: each must make some pin above fail


def _expect_pin_failure(monkeypatch, target, replacement, pin):
    monkeypatch.setattr(oracle.paged_attention, target, replacement)
    monkeypatch.setattr(oracle, target, replacement, raising=False)
    with pytest.raises((AssertionError, IndexError)):
        pin()


def test_planted_missing_scale_is_caught(monkeypatch):
    def attend_noscale(qvec, K, V, scale):
        z = K @ qvec
        w = np.exp(z - z.max())
        return (w @ V) / w.sum(), w / w.sum()

    wl = make_tiny_decode(seed=1, ctx=(1, 5, 17, 33), Hq=4, Hkv=2, D=8, dtype="f32")
    _expect_pin_failure(monkeypatch, "attend", attend_noscale, lambda: check_bruteforce(wl))


def test_planted_wrong_gqa_mapping_is_caught(monkeypatch):
    real = oracle.paged_attention.decode

    def decode_modmap(q, pool_k, pool_v, block_tables, context_lens, scale, dtype, **kw):
        # kv head h % Hkv instead of h // G: permute q heads before the real call
        S, Hq, D = q.shape
        Hkv = pool_k.shape[2]
        G = Hq // Hkv
        perm = [(h % Hkv) * G + h // Hkv for h in range(Hq)]
        out = real(q[:, perm], pool_k, pool_v, block_tables, context_lens, scale, dtype, **kw)
        inv = np.argsort(perm)
        return out[:, inv]

    wl = make_tiny_decode(seed=1, ctx=(1, 5, 17, 33), Hq=4, Hkv=2, D=8, dtype="f32")
    _expect_pin_failure(monkeypatch, "decode", decode_modmap, lambda: check_bruteforce(wl))


def test_planted_wrong_block_index_is_caught(monkeypatch):
    def gather_shifted(pool, table_row, n):
        nb = (n + 15) // 16
        ids = np.roll(np.asarray(table_row[:nb], dtype=np.int64), 1)
        return pool[ids].reshape(nb * 16, pool.shape[2], pool.shape[3])[:n]

    wl = make_tiny_decode(seed=1, ctx=(1, 5, 17, 33), Hq=4, Hkv=2, D=8, dtype="f32")
    _expect_pin_failure(monkeypatch, "gather", gather_shifted, lambda: check_bruteforce(wl))


def test_planted_causal_off_by_one_is_caught(monkeypatch):
    real_attend = oracle.paged_attention.attend

    def attend_drop_last(qvec, K, V, scale):
        if K.shape[0] > 1:
            K, V = K[:-1], V[:-1]
        return real_attend(qvec, K, V, scale)

    wl = make_tiny_prefill(seed=14, prior=(0, 0), chunk=(5, 21), Hq=4, Hkv=2, D=16, dtype="bf16")
    _expect_pin_failure(monkeypatch, "attend", attend_drop_last, lambda: check_prefill_textbook(wl))


def test_planted_wrong_v_layout_is_caught(monkeypatch):
    def v_bytes_untransposed(pool_v):
        return np.ascontiguousarray(pool_v.transpose(0, 2, 1, 3)).reshape(-1)

    _expect_pin_failure(monkeypatch, "v_pool_bytes", v_bytes_untransposed,
                        test_physical_layout_matches_written_formula)


def test_planted_causal_future_key_is_caught(monkeypatch):
    # each query row also sees the key just past its own position
    def prefill_future(q, pool_k, pool_v, block_tables, query_start_loc, context_lens, scale, dtype,
                       rows=None, **kw):
        Tq, Hq, D = q.shape
        Hkv = pool_k.shape[2]
        out = np.zeros((Tq, Hq, D))
        for r in range(len(context_lens)):
            lo, hi = int(query_start_loc[r]), int(query_start_loc[r + 1])
            ctx = int(context_lens[r])
            K = oracle.widen(oracle.gather(pool_k, block_tables[r], ctx), dtype)
            V = oracle.widen(oracle.gather(pool_v, block_tables[r], ctx), dtype)
            for i in range(hi - lo):
                pos = ctx - (hi - lo) + i
                qrow = oracle.widen(q[lo + i], dtype)
                for h in range(Hq):
                    g = h // (Hq // Hkv)
                    out[lo + i, h], _ = oracle.attend(qrow[h], K[: pos + 2, g], V[: pos + 2, g],
                                                      float(np.float32(scale)))
        return out

    wl = make_tiny_prefill(seed=15, prior=(3, 20), chunk=(6, 13), Hq=4, Hkv=2, D=16, dtype="bf16")
    _expect_pin_failure(monkeypatch, "prefill_chunk", prefill_future, lambda: check_prefill_textbook(wl))
