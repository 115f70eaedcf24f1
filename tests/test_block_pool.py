"""The library's host block pool (pa_pool_*) against the reference model in
oracle/block_pool.py: the same seeded operation sequences must give the same
cached-token counts, slots, copy-on-write pairs, block tables and free
counts, step by step (the model is pinned in test_oracle_block_pool.py).
Host only: no GPU."""

import random

import pytest

import paged_kv_cache_396_amd as pa
from oracle.block_pool import BlockPool as RefPool, NoFreeBlocks


def run_both(num_blocks, seed, n_ops, vocab=6):
    rng = random.Random(seed)
    ref, lib = RefPool(num_blocks), pa.BlockPool(num_blocks)
    live, next_id = [], 0
    stats = {"cow": 0, "hits": 0, "nofree": 0}

    def alloc(r, toks):
        try:
            want = ref.allocate_slots(r, toks)
        except NoFreeBlocks:
            with pytest.raises(pa.PAError) as e:
                lib.allocate_slots(r, toks)
            assert e.value.status == pa.PA_ERR_NO_BLOCKS
            stats["nofree"] += 1
            return False
        got = lib.allocate_slots(r, toks)
        assert got == (list(want[0]), list(want[1]))
        stats["cow"] += len(want[1])
        return True

    for _ in range(n_ops):
        op = rng.random()
        if op < 0.3 or not live:
            plen = rng.randrange(0, 70)
            base = rng.randrange(3)
            prompt = [(base * 7 + i * (1 + base)) % vocab for i in range(plen)]
            c = ref.add_request(next_id, prompt)
            assert lib.add_request(next_id, prompt) == c
            stats["hits"] += c > 0
            if alloc(next_id, prompt[c:]):
                live.append(next_id)
            else:
                ref.free_request(next_id)
                lib.free_request(next_id)
            next_id += 1
        elif op < 0.6:
            r = rng.choice(live)
            alloc(r, [rng.randrange(vocab) for _ in range(rng.randrange(1, 20))])
        elif op < 0.75:
            r = rng.choice(live)
            ref.fork(r, next_id)
            lib.fork(r, next_id)
            live.append(next_id)
            next_id += 1
        else:
            r = live.pop(rng.randrange(len(live)))
            ref.free_request(r)
            lib.free_request(r)
        assert lib.num_free() == ref.num_free()
        for r in live:
            assert lib.block_table(r) == ref.block_table(r)
            assert lib.num_tokens(r) == ref.num_tokens(r)
    return stats


@pytest.mark.parametrize("seed", range(8))
def test_pool_matches_reference_model(seed):
    stats = run_both(40, seed, 400)
    assert stats["cow"] and stats["hits"] and stats["nofree"]


def test_pool_large_mixed_sequence():
    stats = run_both(600, 123, 3000, vocab=4)
    assert stats["cow"] > 10 and stats["hits"] > 10


def test_pool_errors():
    p = pa.BlockPool(4)
    assert p.add_request(7, [1, 2, 3]) == 0
    with pytest.raises(pa.PAError) as e:
        p.add_request(7, [1])
    assert e.value.status == -10
    for call in (lambda: p.allocate_slots(8, [1]), lambda: p.fork(8, 9), lambda: p.free_request(8),
                 lambda: p.block_table(8), lambda: p.num_tokens(8)):
        with pytest.raises(pa.PAError) as e:
            call()
        assert e.value.status == -9
    with pytest.raises(pa.PAError) as e:
        p.fork(7, 7)
    assert e.value.status == -10
    # 3 usable blocks: 49 tokens need 4
    with pytest.raises(pa.PAError) as e:
        p.allocate_slots(7, list(range(49)))
    assert e.value.status == pa.PA_ERR_NO_BLOCKS
    assert p.num_tokens(7) == 0 and p.num_free() == 3
    with pytest.raises(pa.PAError):
        pa.BlockPool(1)
