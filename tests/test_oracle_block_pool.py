"""Pins for the block-pool reference model (oracle/block_pool.py): each check
holds the model to a fact the pages state or to an invariant of reference
counting, not to its own code.

* Parallel sampling shares every prompt block; a sample that writes into the
  shared, partly filled last block gets its own copy first (zihan-zhang.net
  vLLM study, 3.2.2).
* Prefix matching is cumulative: a prompt that differs in its first token
  matches nothing; one that shares the first k full blocks matches exactly
  those (same page, 3.6.1).
* Freed blocks keep their key and are reused from the least recently used
  end; reuse removes the old key (same page, 3.6.2 and 5.5).
* Allocation that cannot be served changes nothing (same page, 5.5).
* Invariants after random operation sequences: reference counts equal the
  number of tables that hold a block; the free queue is exactly the
  unreferenced blocks; every indexed key names a block holding that content;
  blocks shared by live requests hold the same tokens in every filled slot.

The last tests plant mistakes in a copy of the model and check that a pin
fails.
"""

import random

import numpy as np
import pytest

from oracle.block_pool import BLOCK, BlockPool, NoFreeBlocks, copy_blocks


def _contents(pool, req):
    """Logical token of every filled slot of req: {(block, offset): token}."""
    r = pool.reqs[req]
    return {(r["blocks"][i // BLOCK], i % BLOCK): r["tokens"][i] for i in range(r["n"])}


def check_invariants(pool):
    refs = [0] * pool.num_blocks
    for r in pool.reqs.values():
        assert len(r["blocks"]) == (r["n"] + BLOCK - 1) // BLOCK
        assert len(r["tokens"]) == r["n"]
        for b in r["blocks"]:
            assert 1 <= b < pool.num_blocks
            refs[b] += 1
    assert refs == pool.ref
    assert set(pool.free) == {b for b in range(1, pool.num_blocks) if refs[b] == 0}
    assert len(pool.free) == len(set(pool.free))
    for k, b in pool.index.items():
        assert pool.key[b] == k and len(k) % BLOCK == 0
    # shared blocks hold the same tokens for every live holder
    seen = {}
    for req in pool.reqs:
        for slot, tok in _contents(pool, req).items():
            assert seen.setdefault(slot, tok) == tok, f"slot {slot} holds two different tokens"


def test_parallel_sampling_shares_prompt_then_copies_on_write():
    pool = BlockPool(32)
    prompt = list(range(1000, 1040))  # 2 full blocks + 8 tokens
    cached = pool.add_request(0, prompt)
    assert cached == 0
    slots, copies = pool.allocate_slots(0, prompt)
    assert copies == [] and len(slots) == 40
    for s in range(1, 4):
        pool.fork(0, s)
    assert [pool.ref[b] for b in pool.block_table(0)] == [4, 4, 4]
    shared_last = pool.block_table(0)[-1]
    for s in range(1, 4):
        slots, copies = pool.allocate_slots(s, [s])
        assert len(copies) == 1 and copies[0][0] == shared_last
        assert pool.block_table(s)[:2] == pool.block_table(0)[:2]   # full blocks stay shared
        assert slots == [copies[0][1] * BLOCK + 8]                    # position 40 -> offset 8
    # the last holder writes in place
    slots, copies = pool.allocate_slots(0, [0])
    assert copies == [] and slots == [shared_last * BLOCK + 8]
    check_invariants(pool)


def test_prefix_match_is_cumulative():
    pool = BlockPool(64)
    a = list(range(64))
    pool.add_request(0, a)
    pool.allocate_slots(0, a)
    # same first 3 blocks, then different
    b = a[:48] + [999] * 20
    assert pool.add_request(1, b) == 48
    assert pool.block_table(1) == pool.block_table(0)[:3]
    # different first token: nothing matches
    c = [7] + a[1:]
    assert pool.add_request(2, c) == 0
    # a prompt equal to a cached one keeps its last block to compute
    assert pool.add_request(3, a) == 48
    check_invariants(pool)


def test_freed_blocks_are_reused_least_recently_used_first_and_lose_their_key():
    pool = BlockPool(1 + 4)
    a = list(range(32))
    pool.add_request(0, a)
    pool.allocate_slots(0, a)            # blocks 1, 2 (ascending first-use order)
    assert pool.block_table(0) == [1, 2]
    pool.free_request(0)                 # last block first: free queue 3, 4, 2, 1
    assert list(pool.free) == [3, 4, 2, 1]
    assert len(pool.index) == 2          # the keys survive the free
    # the cached blocks revive on a hit
    assert pool.add_request(1, a + [5]) == 32
    assert list(pool.free) == [3, 4]
    pool.free_request(1)
    # two new blocks come from the head; then the next takes block 2 and evicts its key
    pool.add_request(2, [])
    pool.allocate_slots(2, list(range(500, 548)))
    assert pool.block_table(2) == [3, 4, 2]
    assert tuple(a[:32]) not in pool.index         # a's second block key left with block 2
    assert pool.index[tuple(a[:16])] == 1          # a's first block is still cached
    assert pool.add_request(3, a + [1]) == 16      # only a's first block is still cached
    check_invariants(pool)


def test_allocation_failure_changes_nothing():
    pool = BlockPool(1 + 3)
    pool.add_request(0, [])
    pool.allocate_slots(0, list(range(40)))        # 3 blocks
    before = (list(pool.free), list(pool.ref), dict(pool.index), pool.block_table(0), pool.num_tokens(0))
    with pytest.raises(NoFreeBlocks):
        pool.allocate_slots(0, list(range(9)))     # needs a 4th block
    assert (list(pool.free), list(pool.ref), dict(pool.index), pool.block_table(0),
            pool.num_tokens(0)) == before
    # copy-on-write counts the copy's block too
    pool2 = BlockPool(1 + 2)
    pool2.add_request(0, [])
    pool2.allocate_slots(0, list(range(8)))
    pool2.fork(0, 1)
    pool2.allocate_slots(1, [1])                   # CoW uses the last free block
    with pytest.raises(NoFreeBlocks):
        pool2.fork(0, 2) or pool2.allocate_slots(2, [2])
    check_invariants(pool2)


def random_ops(pool, rng, n_ops, vocab=6):
    """A seeded random mix of admit / append / fork / free (small vocabulary,
    so that prompts repeat and prefixes hit)."""
    live, next_id, log = [], 0, []
    for _ in range(n_ops):
        op = rng.random()
        try:
            if op < 0.3 or not live:
                plen = rng.randrange(0, 70)
                base = rng.randrange(3)
                prompt = [(base * 7 + i * (1 + base)) % vocab for i in range(plen)]
                c = pool.add_request(next_id, prompt)
                log.append(("add", next_id, c))
                try:
                    s, cp = pool.allocate_slots(next_id, prompt[c:])
                    log.append(("alloc", next_id, tuple(s), tuple(cp)))
                except NoFreeBlocks:
                    pool.free_request(next_id)
                    log.append(("nofree", next_id))
                    next_id += 1
                    continue
                live.append(next_id)
                next_id += 1
            elif op < 0.6:
                r = rng.choice(live)
                toks = [rng.randrange(vocab) for _ in range(rng.randrange(1, 20))]
                s, cp = pool.allocate_slots(r, toks)
                log.append(("alloc", r, tuple(s), tuple(cp)))
            elif op < 0.75:
                r = rng.choice(live)
                pool.fork(r, next_id)
                live.append(next_id)
                log.append(("fork", r, next_id))
                next_id += 1
            else:
                r = live.pop(rng.randrange(len(live)))
                pool.free_request(r)
                log.append(("free", r))
        except NoFreeBlocks:
            log.append(("nofree",))
        check_invariants(pool)
    return log


@pytest.mark.parametrize("seed", range(6))
def test_invariants_hold_under_random_operations(seed):
    pool = BlockPool(40)
    log = random_ops(pool, random.Random(seed), 300)
    assert any(e[0] == "alloc" and e[3] for e in log)       # copy-on-write happened
    assert any(e[0] == "add" and e[2] > 0 for e in log)     # prefix hits happened
    assert any(e[0] == "nofree" for e in log)               # the pool ran dry at times


def test_copy_blocks_copies_every_head_and_nothing_else():
    rng = np.random.default_rng(0)
    pk = rng.integers(0, 1 << 16, size=(6, 16, 2, 8), dtype=np.uint16)
    pv = rng.integers(0, 1 << 16, size=(6, 16, 2, 8), dtype=np.uint16)
    k0, v0 = pk.copy(), pv.copy()
    copy_blocks(pk, pv, [(1, 4), (2, 5)])
    assert np.array_equal(pk[4], k0[1]) and np.array_equal(pv[5], v0[2])
    assert np.array_equal(pk[[0, 1, 2, 3]], k0[[0, 1, 2, 3]])
    assert np.array_equal(pv[[0, 1, 2, 3]], v0[[0, 1, 2, 3]])


# ----------------------------------------------------------------------------
# planted mistakes: each must break a pin


class _NoCow(BlockPool):
    def allocate_slots(self, req, new_tokens):
        r = self.reqs[req]
        saved = self.ref[r["blocks"][-1]] if r["blocks"] else None
        if r["blocks"]:
            self.ref[r["blocks"][-1]] = 1  # pretend nobody else holds it
        try:
            return super().allocate_slots(req, new_tokens)
        finally:
            if saved is not None and r["blocks"]:
                self.ref[r["blocks"][-1]] = saved


class _KeepStaleKey(BlockPool):
    def _take(self):
        b, _ = self.free.popitem(last=False)
        self.key[b] = None  # forgets to drop the index entry
        self.ref[b] = 1
        return b


@pytest.mark.parametrize("bad", [_NoCow, _KeepStaleKey])
def test_planted_mistakes_fail_a_pin(bad):
    failed = False
    for seed in range(6):
        try:
            random_ops(bad(40), random.Random(seed), 300)
        except AssertionError:
            failed = True
            break
    assert failed
