"""Cache writes on the GPU must equal the oracle's pool byte for byte,
including every slot nobody wrote (which keeps its NaN poison)."""

import numpy as np
import pytest

import oracle
from workloads import make_decode, make_tiny_decode, poison_bits

from gpu_util import gpu_pool_for, log, mixed_slots, oracle_pools

pytestmark = pytest.mark.gpu


def _compare_pools(wl, pool):
    pk, pv = oracle_pools(wl, oracle)
    assert np.array_equal(pool.k_bits(), oracle.k_pool_bytes(pk)), "K pool differs"
    assert np.array_equal(pool.v_bits(), oracle.v_pool_bytes(pv)), "V pool differs"


@pytest.mark.parametrize("dtype,D,Hkv", [("f32", 64, 2), ("bf16", 128, 8), ("bf16", 64, 1),
                                         ("f32", 128, 3)])
def test_cache_write_tiny_bit_exact(dtype, D, Hkv):
    log(f"cache write tiny {dtype} D={D} Hkv={Hkv}")
    wl = make_tiny_decode(seed=31, ctx=(1, 15, 16, 17, 40), Hq=Hkv, Hkv=Hkv, D=D, dtype=dtype)
    _compare_pools(wl, gpu_pool_for(wl))


def test_cache_write_negative_and_out_of_range_slots_write_nothing():
    log("cache write with padding slots")
    wl = make_tiny_decode(seed=32, ctx=(20, 33), Hq=2, Hkv=2, D=128, dtype="bf16")
    slots = wl.hist_slots.copy()
    slots[::3] = -1                      # padding tokens
    slots[1] = wl.num_blocks * 16 + 5    # beyond the pool: ignored
    wl.hist_slots = slots
    pool = gpu_pool_for(wl)
    # the oracle skips negative slots; the out-of-range one must not appear either
    keep = slots.copy()
    keep[1] = -1
    wl.hist_slots = keep
    _compare_pools(wl, pool)


def test_cache_write_config1():
    log("cache write config 1")
    wl = make_decode(1)
    _compare_pools(wl, gpu_pool_for(wl))


def test_cache_write_config2_full_pool():
    """The Llama-3.1-8B-shaped layer: history plus the step's 64 new tokens."""
    log("cache write config 2 (full pool)")
    wl = make_decode(2)
    _compare_pools(wl, gpu_pool_for(wl))


def test_cache_write_block_aligned_runs_and_scattered_tokens_mixed():
    """Groups of 16 input tokens that fill one block in order (written as whole
    tiles) next to a misaligned run, a run with a padding token, scattered
    tokens and a short last group: byte-exact either way."""
    from gpu_util import GpuPool

    log("cache write aligned runs + scattered tokens")
    rng = np.random.default_rng(5)
    for dtype, D, Hkv in (("bf16", 128, 8), ("f32", 64, 2), ("bf16", 64, 3)):
        nb = 40
        runs = [16 * 5 + np.arange(16),            # aligned run: whole block 5
                16 * 2 + np.arange(16),            # aligned run: whole block 2
                16 * 7 + 3 + np.arange(16),        # consecutive but misaligned (blocks 7, 8)
                16 * 11 + np.arange(16),           # aligned run with a padding token
                rng.choice(np.arange(16 * 20, 16 * 30), 16, replace=False),  # scattered
                16 * 33 + np.arange(15)]           # short last group
        slots = np.concatenate(runs).astype(np.int64)
        slots[3 * 16 + 6] = -1
        T = slots.shape[0]
        raw = np.uint16 if dtype == "bf16" else np.uint32
        k = rng.integers(0, 2 ** 15 if dtype == "bf16" else 2 ** 30, (T, Hkv, D)).astype(raw)
        v = rng.integers(0, 2 ** 15 if dtype == "bf16" else 2 ** 30, (T, Hkv, D)).astype(raw)
        pool = GpuPool(nb, Hkv, D, dtype)
        pool.write(k, v, slots)
        pk = oracle.new_pool(nb, Hkv, D, dtype, poison_bits(dtype))
        pv = oracle.new_pool(nb, Hkv, D, dtype, poison_bits(dtype))
        oracle.reshape_and_cache(pk, pv, k, v, slots)
        assert np.array_equal(pool.k_bits(), oracle.k_pool_bytes(pk)), f"K pool {dtype} {D}"
        assert np.array_equal(pool.v_bits(), oracle.v_pool_bytes(pv)), f"V pool {dtype} {D}"


def test_cache_write_bulk_fill_config3_pool_full():
    """The 70B layer's whole history written in one call (524,288 tokens,
    every block a full aligned run): both whole pools (40,960 blocks, 1.25
    GiB each) compared byte for byte, in host-side chunks of blocks."""
    log("cache write bulk fill config 3 (whole pools)")
    wl = make_decode(3)
    pool = gpu_pool_for(wl, with_new=False)
    pk = oracle.new_pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype, poison_bits(wl.dtype))
    pv = oracle.new_pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype, poison_bits(wl.dtype))
    oracle.reshape_and_cache_fast(pk, pv, wl.hist_k, wl.hist_v, wl.hist_slots)
    per_block = wl.num_kv_heads * 16 * wl.head_dim * 2  # bytes of one block in one pool
    chunk = 2048
    for b0 in range(0, wl.num_blocks, chunk):
        b1 = min(wl.num_blocks, b0 + chunk)
        kb = pool.k[b0 * per_block: b1 * per_block].cpu().numpy().view(np.uint16)
        vb = pool.v[b0 * per_block: b1 * per_block].cpu().numpy().view(np.uint16)
        assert np.array_equal(kb, oracle.k_pool_bytes(pk[b0:b1])), f"K blocks {b0}..{b1 - 1}"
        assert np.array_equal(vb, oracle.v_pool_bytes(pv[b0:b1])), f"V blocks {b0}..{b1 - 1}"

def _run_slots(rng, nb, lengths, offsets):
    """Slots of consecutive runs (one per request), each starting at the given
    offset inside a fresh random block and continuing through the next
    blocks; concatenated in request order, so most input groups of 16 start
    mid-block and some hold the end of one run and the start of the next."""
    blocks = list(rng.permutation(nb))
    out = []
    for n, o in zip(lengths, offsets):
        nbk = (o + n + 15) // 16
        mine = [blocks.pop() for _ in range(nbk)]
        pos = o + np.arange(n)
        out.append(np.asarray(mine, dtype=np.int64)[pos // 16] * 16 + pos % 16)
    return np.concatenate(out).astype(np.int64)


@pytest.mark.parametrize("dtype,D,Hkv", [("bf16", 128, 8), ("f32", 64, 2), ("bf16", 64, 3)])
def test_cache_write_runs_starting_mid_block(dtype, D, Hkv):
    """Consecutive slots that start anywhere in a block (a prefill chunk's or
    a ragged history's tokens): whole pools byte-exact, untouched slots keep
    their poison; adjacent runs fill complementary halves of shared blocks."""
    from gpu_util import GpuPool

    log(f"cache write runs starting mid-block {dtype} D={D} Hkv={Hkv}")
    rng = np.random.default_rng(D * 7 + Hkv)
    nb = 200
    lengths = [2047 % 300 + 1, 16, 17, 31, 1, 64, 100, 15, 33, 250]
    offsets = [3, 0, 15, 8, 7, 1, 12, 0, 5, 9]
    slots = _run_slots(rng, nb, lengths, offsets)
    T = slots.shape[0]
    raw = np.uint16 if dtype == "bf16" else np.uint32
    k = rng.integers(0, 2 ** 15 if dtype == "bf16" else 2 ** 30, (T, Hkv, D)).astype(raw)
    v = rng.integers(0, 2 ** 15 if dtype == "bf16" else 2 ** 30, (T, Hkv, D)).astype(raw)
    pool = GpuPool(nb, Hkv, D, dtype)
    pool.write(k, v, slots)
    pk = oracle.new_pool(nb, Hkv, D, dtype, poison_bits(dtype))
    pv = oracle.new_pool(nb, Hkv, D, dtype, poison_bits(dtype))
    oracle.reshape_and_cache(pk, pv, k, v, slots)
    assert np.array_equal(pool.k_bits(), oracle.k_pool_bytes(pk)), "K pool"
    assert np.array_equal(pool.v_bits(), oracle.v_pool_bytes(pv)), "V pool"


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("dtype,D,Hkv", [("bf16", 128, 8), ("f32", 64, 2), ("bf16", 64, 3)])
def test_cache_write_random_segments(dtype, D, Hkv, seed):
    """Random mixtures of runs, scattered tokens, padding and out-of-range
    slots in one call: whole pools byte-exact against the oracle."""
    from gpu_util import GpuPool

    log(f"cache write random segments {dtype} D={D} Hkv={Hkv} seed={seed}")
    rng = np.random.default_rng(1000 * seed + D + Hkv)
    nb = 400
    slots = mixed_slots(rng, nb, 120)
    T = slots.shape[0]
    raw = np.uint16 if dtype == "bf16" else np.uint32
    k = rng.integers(0, 2 ** 15 if dtype == "bf16" else 2 ** 30, (T, Hkv, D)).astype(raw)
    v = rng.integers(0, 2 ** 15 if dtype == "bf16" else 2 ** 30, (T, Hkv, D)).astype(raw)
    pool = GpuPool(nb, Hkv, D, dtype)
    pool.write(k, v, slots)
    pk = oracle.new_pool(nb, Hkv, D, dtype, poison_bits(dtype))
    pv = oracle.new_pool(nb, Hkv, D, dtype, poison_bits(dtype))
    # slots past the pool are ignored (the oracle skips negative ones)
    oracle.reshape_and_cache(pk, pv, k, v, np.where(slots >= nb * 16, -1, slots))
    assert np.array_equal(pool.k_bits(), oracle.k_pool_bytes(pk)), "K pool"
    assert np.array_equal(pool.v_bits(), oracle.v_pool_bytes(pv)), "V pool"


def test_cache_write_run_halves_of_one_block_in_two_calls():
    """One block filled by two runs, offsets 0..6 in the first call and 7..15
    (continuing into the next block) in the second: the first call's
    elements survive the second's partial chunk writes."""
    from gpu_util import GpuPool

    log("cache write two runs into one block")
    rng = np.random.default_rng(3)
    nb, Hkv, D = 8, 2, 128
    pool = GpuPool(nb, Hkv, D, "bf16")
    pk = oracle.new_pool(nb, Hkv, D, "bf16", poison_bits("bf16"))
    pv = oracle.new_pool(nb, Hkv, D, "bf16", poison_bits("bf16"))
    for sl in (np.arange(3 * 16, 3 * 16 + 7), np.arange(3 * 16 + 7, 3 * 16 + 7 + 20)):
        sl = sl.astype(np.int64)
        k = rng.integers(0, 2 ** 15, (len(sl), Hkv, D)).astype(np.uint16)
        v = rng.integers(0, 2 ** 15, (len(sl), Hkv, D)).astype(np.uint16)
        pool.write(k, v, sl)
        oracle.reshape_and_cache(pk, pv, k, v, sl)
    assert np.array_equal(pool.k_bits(), oracle.k_pool_bytes(pk))
    assert np.array_equal(pool.v_bits(), oracle.v_pool_bytes(pv))
