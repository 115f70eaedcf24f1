"""Chunked prefill (bf16 matrix cores) on the GPU against the fp64 oracle.

Tolerance: |gpu - ref| <= 2e-2 + 2e-2|ref| (bf16 inputs, fp32 accumulation,
probabilities rounded to bf16 before the P.V product).  Pools are
NaN-poisoned before any write: a stray read of an unreferenced block or of a
slot past the context shows up as a non-finite output.
"""

import numpy as np
import pytest

import oracle
from workloads import (make_decode, make_mixed, make_prefill, make_tiny_decode, make_tiny_prefill,
                       poison_bits)

from gpu_util import (assert_close, gpu_decode, gpu_pool_for, gpu_prefill, log, oracle_pools,
                      raw_bits, to_f64)

pytestmark = pytest.mark.gpu


def _oracle_prefill(wl, rows=None):
    pk, pv = oracle_pools(wl, oracle)
    return oracle.prefill_chunk(wl.q, pk, pv, wl.block_tables, wl.query_start_loc,
                                wl.context_lens, wl.scale, wl.dtype, rows=rows)


SHAPES = [
    # D, Hq, Hkv, prior, chunk
    (128, 32, 8, (0, 5, 40), (7, 16, 33)),
    (128, 32, 8, (0,), (1,)),
    (128, 32, 8, (16, 100, 0, 63), (1, 15, 130, 64)),
    (128, 64, 8, (3, 200), (17, 70)),
    (128, 8, 4, (31, 0), (40, 129)),
    (128, 4, 4, (10,), (200,)),
    (128, 16, 2, (0, 77), (300, 5)),
    (64, 16, 2, (9, 0), (20, 65)),
    (64, 8, 8, (130,), (33,)),
    (64, 32, 4, (0, 1), (64, 129)),
    (128, 32, 8, (0, 50, 2000), (16, 9, 12)),  # both column blocks of the paired shape
]


@pytest.mark.parametrize("D,Hq,Hkv,prior,chunk", SHAPES)
def test_tiny_prefill_shapes(D, Hq, Hkv, prior, chunk):
    log(f"prefill tiny D={D} Hq={Hq} Hkv={Hkv} prior={prior} chunk={chunk}")
    wl = make_tiny_prefill(seed=61 + D + Hq + sum(chunk), prior=prior, chunk=chunk, Hq=Hq,
                           Hkv=Hkv, D=D)
    out = to_f64(gpu_prefill(wl, gpu_pool_for(wl)))
    assert_close(out, _oracle_prefill(wl), "bf16", f"prefill D={D} {Hq}/{Hkv}")


def test_prefill_prior_zero_is_plain_causal_attention():
    log("prefill prior 0")
    wl = make_tiny_prefill(seed=3, prior=(0, 0), chunk=(100, 33), Hq=32, Hkv=8, D=128)
    out = to_f64(gpu_prefill(wl, gpu_pool_for(wl)))
    assert_close(out, _oracle_prefill(wl), "bf16", "prior 0")


def test_prefill_permutation_of_physical_blocks_is_bitwise_invariant():
    log("prefill permutation invariance")
    a = make_tiny_prefill(seed=4, prior=(40, 300), chunk=(70, 129), Hq=32, Hkv=8, D=128,
                          layout_variant=0)
    b = make_tiny_prefill(seed=4, prior=(40, 300), chunk=(70, 129), Hq=32, Hkv=8, D=128,
                          layout_variant=1)
    assert not np.array_equal(a.block_tables, b.block_tables)
    oa = gpu_prefill(a, gpu_pool_for(a))
    ob = gpu_prefill(b, gpu_pool_for(b))
    assert np.array_equal(raw_bits(oa), raw_bits(ob))


def test_prefill_last_row_matches_decode():
    """A chunk's last query sees the whole context, exactly as decode does."""
    log("prefill last row vs decode")
    wl = make_tiny_prefill(seed=5, prior=(90, 500, 0), chunk=(10, 64, 33), Hq=32, Hkv=8, D=128)
    pool = gpu_pool_for(wl)
    pre = to_f64(gpu_prefill(wl, pool))
    last = wl.query_start_loc[1:] - 1

    class _Dec:  # decode view of the same pool: one query per request (its last row)
        pass

    d = _Dec()
    d.q = wl.q[last]
    d.dtype, d.num_kv_heads, d.scale = wl.dtype, wl.num_kv_heads, wl.scale
    d.block_tables, d.context_lens = wl.block_tables, wl.context_lens
    dec = to_f64(gpu_decode(d, pool))
    assert_close(pre[last], dec, "bf16", "last row vs decode")


def test_prefill_two_half_chunks_equal_one_chunk():
    """Splitting a chunk into two requests over the same table (the first half
    with a shorter context) gives the same rows within tolerance."""
    log("prefill split chunk")
    wl = make_tiny_prefill(seed=6, prior=(200,), chunk=(96,), Hq=32, Hkv=8, D=128)
    pool = gpu_pool_for(wl)
    whole = to_f64(gpu_prefill(wl, pool))
    ref = _oracle_prefill(wl)
    assert_close(whole, ref, "bf16", "whole chunk")
    # same block table twice: first 48 rows at ctx 248, next 48 at ctx 296
    wl2 = make_tiny_prefill(seed=6, prior=(200,), chunk=(96,), Hq=32, Hkv=8, D=128)
    wl2.block_tables = np.repeat(wl.block_tables, 2, axis=0)
    split = to_f64(gpu_prefill(wl2, pool, query_start_loc=np.array([0, 48, 96], np.int32),
                               context_lens=np.array([248, 296], np.int32)))
    assert_close(split, ref, "bf16", "two half chunks")


def test_prefill_unreferenced_rows_stay_finite_with_poison():
    log("prefill poison")
    wl = make_tiny_prefill(seed=7, prior=(1, 17, 33), chunk=(15, 1, 31), Hq=8, Hkv=2, D=128)
    out = to_f64(gpu_prefill(wl, gpu_pool_for(wl)))
    assert np.isfinite(out).all()
    assert_close(out, _oracle_prefill(wl), "bf16", "poison")


def test_config5_prefill_full():
    """The long-context mixed batch's prefill half at full size: 4 requests,
    512-token chunks against 4096 prior tokens; every row and head against
    the oracle."""
    log("prefill config 5 (full)")
    wl = make_prefill(5)
    out = to_f64(gpu_prefill(wl, gpu_pool_for(wl)))
    log("  oracle ...")
    err = assert_close(out, _oracle_prefill(wl), "bf16", "config 5 prefill")
    log(f"  max abs err {err:.3g}")


def test_config5_mixed_step_one_pool():
    """The long-context mixed batch as one step over one pool: decodes append
    their newest tokens and attend while the prefill chunks write their K/V
    and attend, on two streams at once.  Both outputs against the oracle
    (every decode row, every prefill row), both pools byte for byte against
    the oracle's after the step's writes, and the same step back to back on
    one stream bitwise equal to the concurrent one."""
    import torch

    from gpu_util import MixedStep

    log("mixed step config 5 (two streams, one pool)")
    dec, pre = make_mixed(0)
    step = MixedStep(dec, pre)
    step.run(concurrent=True)
    torch.cuda.synchronize()
    d_conc, p_conc = raw_bits(step.dout), raw_bits(step.pout)
    pk = oracle.new_pool(dec.num_blocks, dec.num_kv_heads, dec.head_dim, dec.dtype, poison_bits(dec.dtype))
    pv = oracle.new_pool(dec.num_blocks, dec.num_kv_heads, dec.head_dim, dec.dtype, poison_bits(dec.dtype))
    for wl in (dec, pre):
        oracle.reshape_and_cache_fast(pk, pv, wl.hist_k, wl.hist_v, wl.hist_slots)
        oracle.reshape_and_cache_fast(pk, pv, wl.new_k, wl.new_v, wl.new_slots)
    per_block = dec.num_kv_heads * 16 * dec.head_dim * 2
    chunk = 2048
    for b0 in range(0, dec.num_blocks, chunk):
        b1 = min(dec.num_blocks, b0 + chunk)
        kb = step.pool.k[b0 * per_block: b1 * per_block].cpu().numpy().view(np.uint16)
        vb = step.pool.v[b0 * per_block: b1 * per_block].cpu().numpy().view(np.uint16)
        assert np.array_equal(kb, oracle.k_pool_bytes(pk[b0:b1])), f"K blocks {b0}..{b1 - 1}"
        assert np.array_equal(vb, oracle.v_pool_bytes(pv[b0:b1])), f"V blocks {b0}..{b1 - 1}"
    ref_d = oracle.decode(dec.q, pk, pv, dec.block_tables, dec.context_lens, dec.scale, dec.dtype)
    err = assert_close(to_f64(step.dout), ref_d, "bf16", "mixed step decode half")
    log(f"  decode half max abs err {err:.3g}")
    log("  prefill oracle ...")
    ref_p = oracle.prefill_chunk(pre.q, pk, pv, pre.block_tables, pre.query_start_loc,
                                 pre.context_lens, pre.scale, pre.dtype)
    err = assert_close(to_f64(step.pout), ref_p, "bf16", "mixed step prefill half")
    log(f"  prefill half max abs err {err:.3g}")
    # back to back on one stream, from a fresh pool: the same bits
    del step
    seq = MixedStep(dec, pre)
    seq.run(concurrent=False)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(seq.dout), d_conc)
    assert np.array_equal(raw_bits(seq.pout), p_conc)


# ---- split-K over the keys: parts of a tile's keys leave partial states,
# merged by a second kernel with the online-softmax rescale

SPLIT_SHAPES = [
    # D, Hq, Hkv, prior, chunk, partition_size
    (128, 32, 8, (0, 5, 40, 700), (7, 16, 33, 3), 64),      # narrow; parts inside the chunk
    (128, 32, 8, (300, 0, 1000), (5, 5, 5), 128),           # narrow, k + 1 rows
    (128, 32, 8, (0, 90, 300), (200, 64, 97), 64),          # wide; causal diagonal across parts
    (128, 8, 1, (33, 1500), (40, 1), 256),                  # G 8, ragged
    (64, 16, 4, (2000, 17), (3, 70), 192),                  # D 64
]


@pytest.mark.parametrize("D,Hq,Hkv,prior,chunk,part", SPLIT_SHAPES)
def test_prefill_split_matches_oracle(D, Hq, Hkv, prior, chunk, part):
    from gpu_util import prefill_splits

    log(f"prefill split D={D} {Hq}/{Hkv} prior={prior} chunk={chunk} part={part}")
    wl = make_tiny_prefill(seed=40 + part, prior=prior, chunk=chunk, Hq=Hq, Hkv=Hkv, D=D)
    assert prefill_splits(wl, wl.max_q_len, part) > 1
    pool = gpu_pool_for(wl)
    ref = _oracle_prefill(wl)
    got = to_f64(gpu_prefill(wl, pool, partition_size=part, workspace_fill=float("nan")))
    err = assert_close(got, ref, "bf16", "split prefill")
    log(f"  max abs err {err:.3g}")
    whole = to_f64(gpu_prefill(wl, pool, partition_size=-1))
    assert_close(whole, ref, "bf16", "unsplit prefill")


@pytest.mark.parametrize("prior,chunk", [((0, 90), (130, 64)), ((5, 40), (20, 33)), ((0, 300), (5, 3))])
@pytest.mark.parametrize("factor", [0.0, -1.0, 8.0])
def test_prefill_scale_edge_cases(prior, chunk, factor):
    """Zero, negative and large softmax scales on the wide, narrow and
    paired shapes: a zero scale is uniform attention over the visible keys,
    a negative one flips the sign of every score."""
    import dataclasses

    wl = make_tiny_prefill(seed=77, prior=prior, chunk=chunk, Hq=32, Hkv=8, D=128)
    wl = dataclasses.replace(wl, scale=float(wl.scale) * factor)
    log(f"prefill scale x{factor} prior={prior} chunk={chunk}")
    got = to_f64(gpu_prefill(wl, gpu_pool_for(wl)))
    err = assert_close(got, _oracle_prefill(wl), "bf16", f"scale x{factor}")
    log(f"  max abs err {err:.3g}")


def test_prefill_split_last_row_still_matches_decode():
    wl = make_tiny_prefill(seed=9, prior=(3000, 1200), chunk=(5, 5), Hq=32, Hkv=8, D=128)
    pool = gpu_pool_for(wl)
    pre = to_f64(gpu_prefill(wl, pool, partition_size=512))
    last = wl.query_start_loc[1:] - 1

    class _Dec:
        pass

    d = _Dec()
    d.q = wl.q[last]
    d.dtype, d.num_kv_heads, d.scale = wl.dtype, wl.num_kv_heads, wl.scale
    d.block_tables, d.context_lens = wl.block_tables, wl.context_lens
    dec = to_f64(gpu_decode(d, pool))
    assert_close(pre[last], dec, "bf16", "split last row vs decode")
