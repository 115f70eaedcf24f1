"""Cache writes on the GPU must equal the oracle's pool byte for byte,
including every slot nobody wrote (which keeps its NaN poison)."""

import numpy as np
import pytest

import oracle
from workloads import make_decode, make_tiny_decode

from gpu_util import gpu_pool_for, log, oracle_pools

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
