"""Reference model of the KV block pool (host policy) and of the block copy.

TEST INFRASTRUCTURE ONLY.  Only the tests may import this module.  It shares
no code with the library and imports nothing from it.

What it follows (the pages are cited by title and section):

* Blocks are shared between sequences through reference counts; when a
  sequence must write into a block that others still hold (the partly
  filled last block of a forked sample), it first gets a private copy
  (zihan-zhang.net vLLM study, 3.2.2: sharing and copy-on-write;
  plumephp.com vLLM deep dive, 4.2).
* A full block is indexed by a prefix-cumulative key: two blocks match only
  if everything from the start of the sequence through the block is equal
  (same page, 3.6.1).  Here the key is that token prefix itself, so a match
  is exact by construction.
* Freed blocks keep their key and join the tail of the free queue; a block
  is taken from the head (least recently used), and only then does its old
  key leave the index: eviction is a side effect of allocation (same page,
  3.6.2 and 5.5).
* A new request first collects the cached blocks of its prompt, stopping at
  the first miss (same page, 5.5, get_computed_blocks); allocation for new
  tokens fails without changing anything when the free queue is too short
  (same page, 5.5, allocate_slots).
* Block 0 is a placeholder that is never handed out (same page, 5.5).

Readings where the pages are silent:
* The first free queue holds blocks 1 .. N-1 in ascending order.
* The lookup of a new request's prompt stops before the block that holds the
  prompt's last token, so at least one token is computed.
* A request's blocks are released last block first, so its first blocks end
  nearest the tail and are evicted last.
* When a newly filled block's key is already indexed (same content computed
  twice), the index keeps the older block.
* Slot of token i of a request: block_table[i // 16] * 16 + i % 16 (vLLM:
  from PagedAttention to Speculative Decoding, 3.3).
"""

from __future__ import annotations

from collections import OrderedDict

import numpy as np

BLOCK = 16


class NoFreeBlocks(Exception):
    pass


class BlockPool:
    def __init__(self, num_blocks: int):
        if num_blocks < 2:
            raise ValueError("a pool needs the placeholder block and at least one more")
        self.num_blocks = num_blocks
        self.ref = [0] * num_blocks
        self.key = [None] * num_blocks          # token prefix that fills this block, if full and indexed
        self.free = OrderedDict((b, None) for b in range(1, num_blocks))  # head = least recently used
        self.index: dict[tuple, int] = {}
        self.reqs: dict[int, dict] = {}

    # -- helpers --------------------------------------------------------
    def _take(self) -> int:
        b, _ = self.free.popitem(last=False)
        if self.key[b] is not None:
            del self.index[self.key[b]]
            self.key[b] = None
        self.ref[b] = 1
        return b

    def num_free(self) -> int:
        return len(self.free)

    def block_table(self, req: int) -> list[int]:
        return list(self.reqs[req]["blocks"])

    def num_tokens(self, req: int) -> int:
        return self.reqs[req]["n"]

    # -- operations -----------------------------------------------------
    def add_request(self, req: int, prompt) -> int:
        """Registers ``req`` with its prompt; returns how many prompt tokens
        are already cached (a multiple of 16).  Those tokens have slots."""
        if req in self.reqs:
            raise KeyError(f"request {req} exists")
        prompt = [int(t) for t in prompt]
        blocks = []
        for j in range((len(prompt) - 1) // BLOCK if prompt else 0):
            k = tuple(prompt[: BLOCK * (j + 1)])
            b = self.index.get(k)
            if b is None:
                break
            if self.ref[b] == 0:
                del self.free[b]
            self.ref[b] += 1
            blocks.append(b)
        n = BLOCK * len(blocks)
        self.reqs[req] = {"blocks": blocks, "tokens": prompt[:n], "n": n}
        return n

    def allocate_slots(self, req: int, new_tokens):
        """Slots for the request's next tokens, whose ids are ``new_tokens``
        (the uncached rest of a prompt, or newly sampled tokens).  Returns
        (slots, copies): copies are (src, dst) block pairs to copy before the
        new tokens are written (copy-on-write of a shared last block).
        Raises NoFreeBlocks, changing nothing, when blocks run out."""
        r = self.reqs[req]
        new_tokens = [int(t) for t in new_tokens]
        n_new = len(new_tokens)
        T = r["n"]
        known = r["tokens"][:T] + new_tokens
        cow = T % BLOCK != 0 and self.ref[r["blocks"][-1]] > 1
        need = (T + n_new + BLOCK - 1) // BLOCK - len(r["blocks"]) + (1 if cow else 0)
        if need > len(self.free):
            raise NoFreeBlocks
        copies = []
        if cow:
            old = r["blocks"][-1]
            new = self._take()
            self.ref[old] -= 1
            r["blocks"][-1] = new
            copies.append((old, new))
        while len(r["blocks"]) * BLOCK < T + n_new:
            r["blocks"].append(self._take())
        slots = [r["blocks"][(T + i) // BLOCK] * BLOCK + (T + i) % BLOCK for i in range(n_new)]
        r["tokens"] = known
        r["n"] = T + n_new
        # index the blocks this call filled
        for j in range(T // BLOCK, r["n"] // BLOCK):
            b = r["blocks"][j]
            if self.key[b] is None:
                k = tuple(known[: BLOCK * (j + 1)])
                if k not in self.index:
                    self.index[k] = b
                    self.key[b] = k
        return slots, copies

    def fork(self, parent: int, child: int) -> None:
        """``child`` shares every block of ``parent`` (parallel sampling)."""
        if child in self.reqs:
            raise KeyError(f"request {child} exists")
        p = self.reqs[parent]
        for b in p["blocks"]:
            self.ref[b] += 1
        self.reqs[child] = {"blocks": list(p["blocks"]), "tokens": list(p["tokens"][: p["n"]]),
                            "n": p["n"]}

    def free_request(self, req: int) -> None:
        r = self.reqs.pop(req)
        for b in reversed(r["blocks"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free[b] = None  # tail: most recently used


def copy_blocks(pool_k: np.ndarray, pool_v: np.ndarray, pairs) -> None:
    """Copy every kv head's K and V of block src into block dst, in place
    (logical pools [num_blocks, 16, Hkv, D]).  The copy of a shared block
    made before a sample writes into it (zihan-zhang.net vLLM study, 3.2.2)."""
    for src, dst in pairs:
        pool_k[dst] = pool_k[src]
        pool_v[dst] = pool_v[src]
