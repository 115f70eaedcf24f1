"""CPU fp64 oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline may import this module.  It shares no code with the HIP library and
imports nothing from it.

Plain, slow, obviously correct NumPy.  Tensors are exchanged as raw bit
patterns (``uint16`` for bf16, ``uint32`` for fp32), exactly as the seeded
workload generators produce them.

What each function follows (the pages are cited by title and section):

* Attention itself: softmax(Q K^T / sqrt(d)) V with a causal mask, each position
  seeing only itself and earlier tokens (zihan-zhang.net vLLM study, 1.1.1).
* Paging: the KV cache is cut into fixed 16-token blocks that need not be
  contiguous; a per-sequence block table maps logical block to physical block
  (vLLM: from PagedAttention to Speculative Decoding, 3.2; zihan-zhang.net
  vLLM study, 3.2).
* Addressing: logical token ``i`` lives in physical block
  ``block_table[i // block_size]`` at offset ``i % block_size`` (vLLM: from
  PagedAttention to Speculative Decoding, 3.3).
* Writing new K/V goes through ``slot_mapping``; the pages name it without
  defining it (same page, 3.3).  Reading taken here: slot = block * 16 + offset,
  a negative slot marks a padding token and writes nothing.
* Chunked prefill: a long prompt is processed chunk by chunk; a chunk's
  queries are the last tokens of the context and attend causally to every
  earlier token (zihan-zhang.net vLLM study, 3.5; flattened batch metadata, 5.6).
* GQA: query head ``h`` reads kv head ``h // (Hq / Hkv)`` (contiguous groups).

Because paging only changes where bytes live, the oracle reaches the exact
dense-attention result: it gathers each sequence's blocks into contiguous
K/V and runs the textbook formula in float64.  There is no online softmax and
no split-K here.

The library's physical pool layout (one K pool and one V pool) is re-derived
here from its written definition, independently of the library:

* K pool: element (block b, kv head g, token offset o, dim x) at
  ``((b * Hkv + g) * 16 + o) * D + x``.
* V pool: element (b, g, o, x) at ``((b * Hkv + g) * D + x) * 16 + o``
  (dim-major inside a tile: the 16 tokens of one dim are consecutive).
"""

from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


# ----------------------------------------------------------------------------
# raw bits <-> float64


def widen(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of each raw element.

    bf16 is the top half of an IEEE binary32, so shifting its 16 bits into the
    high half of a 32-bit word gives the float32 with the same value.
    """
    raw = np.asarray(raw)
    if dtype == "bf16":
        f32 = (raw.astype(np.uint32) << np.uint32(16)).view(np.float32)
    elif dtype == "f32":
        f32 = raw.astype(np.uint32).view(np.float32)
    else:
        raise ValueError(dtype)
    return f32.astype(np.float64)


def raw_type(dtype: str):
    return np.uint16 if dtype == "bf16" else np.uint32


# ----------------------------------------------------------------------------
# the block pool, logical view [num_blocks, 16, Hkv, D]


def new_pool(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str, fill: int) -> np.ndarray:
    """A pool whose every slot holds the raw pattern ``fill``."""
    return np.full((num_blocks, BLOCK_SIZE, num_kv_heads, head_dim), fill, dtype=raw_type(dtype))


def reshape_and_cache(pool_k: np.ndarray, pool_v: np.ndarray, k: np.ndarray, v: np.ndarray,
                      slot_mapping: np.ndarray) -> None:
    """Copy token ``i``'s K and V rows (all kv heads) into its slot, in place.

    Slot ``s >= 0`` names block ``s // 16`` and offset ``s % 16``; negative
    slots are skipped.  A pure bit copy: no value is converted.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for i in range(slots.shape[0]):
        s = int(slots[i])
        if s < 0:
            continue
        pool_k[s // BLOCK_SIZE, s % BLOCK_SIZE] = k[i]
        pool_v[s // BLOCK_SIZE, s % BLOCK_SIZE] = v[i]


def reshape_and_cache_fast(pool_k, pool_v, k, v, slot_mapping) -> None:
    """The same copy as ``reshape_and_cache`` done with one fancy-index
    assignment (slots in one call are distinct), for large pools."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    s = slots[keep]
    pool_k[s // BLOCK_SIZE, s % BLOCK_SIZE] = k[keep]
    pool_v[s // BLOCK_SIZE, s % BLOCK_SIZE] = v[keep]


def k_pool_bytes(pool_k: np.ndarray) -> np.ndarray:
    """The K pool in the library's physical order [block][kv head][token][dim]."""
    return np.ascontiguousarray(pool_k.transpose(0, 2, 1, 3)).reshape(-1)


def v_pool_bytes(pool_v: np.ndarray) -> np.ndarray:
    """The V pool in the library's physical order [block][kv head][dim][token]."""
    return np.ascontiguousarray(pool_v.transpose(0, 2, 3, 1)).reshape(-1)


def k_pool_from_bytes(flat: np.ndarray, num_blocks, num_kv_heads, head_dim) -> np.ndarray:
    t = np.asarray(flat).reshape(num_blocks, num_kv_heads, BLOCK_SIZE, head_dim)
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3))


def v_pool_from_bytes(flat: np.ndarray, num_blocks, num_kv_heads, head_dim) -> np.ndarray:
    t = np.asarray(flat).reshape(num_blocks, num_kv_heads, head_dim, BLOCK_SIZE)
    return np.ascontiguousarray(t.transpose(0, 3, 1, 2))


# ----------------------------------------------------------------------------
# gather + dense attention


def gather(pool: np.ndarray, table_row: np.ndarray, n: int) -> np.ndarray:
    """Raw K (or V) of logical tokens 0..n-1 of one sequence, [n, Hkv, D].

    Logical token i sits in block table_row[i // 16] at offset i % 16; only the
    ceil(n / 16) blocks that hold tokens are read.
    """
    nb = (n + BLOCK_SIZE - 1) // BLOCK_SIZE
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    if ids.shape[0] != nb or (ids < 0).any() or (ids >= pool.shape[0]).any():
        raise IndexError("block table does not cover the context with valid block ids")
    blocks = pool[ids]  # [nb, 16, Hkv, D]
    return blocks.reshape(nb * BLOCK_SIZE, pool.shape[2], pool.shape[3])[:n]


def attend(qvec: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """softmax(scale * K q) weights and the weighted sum of V rows (float64)."""
    z = scale * (K @ qvec)
    m = z.max()
    w = np.exp(z - m)
    l = w.sum()
    return (w @ V) / l, w / l


def _value_fns(dtype, k_value, v_value):
    """How raw pool elements become float64 values: widened as ``dtype`` unless
    the caller gives its own mapping (an 8-bit pool's dequantization)."""
    kf = k_value if k_value is not None else (lambda raw: widen(raw, dtype))
    vf = v_value if v_value is not None else (lambda raw: widen(raw, dtype))
    return kf, vf


def decode(q, pool_k, pool_v, block_tables, context_lens, scale, dtype, num_kv_heads=None,
           return_weights=False, seqs=None, k_value=None, v_value=None):
    """Decode attention for every (sequence, q head): one query per sequence,
    the whole context visible (the newest token included).

    ``q`` is raw [S, Hq, D]; the result is float64 [S, Hq, D].  A sequence of
    length 0 yields zeros.  ``seqs`` restricts the work to some sequences
    (others stay zero).  ``k_value`` / ``v_value`` map gathered raw pool
    elements to float64 (default: widen them as ``dtype``, the q dtype too).
    """
    S, Hq, D = q.shape
    Hkv = pool_k.shape[2] if num_kv_heads is None else num_kv_heads
    G = Hq // Hkv
    sc = float(np.float32(scale))
    kf, vf = _value_fns(dtype, k_value, v_value)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    weights = {}
    for s in (range(S) if seqs is None else seqs):
        n = int(context_lens[s])
        if n == 0:
            continue
        K = kf(gather(pool_k, block_tables[s], n))
        V = vf(gather(pool_v, block_tables[s], n))
        qs = widen(q[s], dtype)
        for h in range(Hq):
            g = h // G
            o, w = attend(qs[h], K[:, g, :], V[:, g, :], sc)
            out[s, h] = o
            if return_weights:
                weights[(s, h)] = w
    return (out, weights) if return_weights else out


def prefill_chunk(q, pool_k, pool_v, block_tables, query_start_loc, context_lens, scale, dtype,
                  rows=None, k_value=None, v_value=None):
    """Causal attention of each request's query chunk against its paged context.

    Request r owns query rows query_start_loc[r] .. query_start_loc[r+1]-1 (n_r of
    them); they are the last n_r tokens of its ctx_r-token context, so query i
    sits at position ctx_r - n_r + i and sees keys 0 .. that position.
    ``rows`` optionally restricts the work to some query rows (others stay zero).
    ``k_value`` / ``v_value`` as for ``decode``.
    Returns float64 [total_q, Hq, D].
    """
    Tq, Hq, D = q.shape
    Hkv = pool_k.shape[2]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    kf, vf = _value_fns(dtype, k_value, v_value)
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    want = None if rows is None else set(int(r) for r in rows)
    R = len(context_lens)
    for r in range(R):
        lo, hi = int(query_start_loc[r]), int(query_start_loc[r + 1])
        n_r = hi - lo
        ctx = int(context_lens[r])
        if n_r == 0:
            continue
        K = kf(gather(pool_k, block_tables[r], ctx))
        V = vf(gather(pool_v, block_tables[r], ctx))
        for i in range(n_r):
            row = lo + i
            if want is not None and row not in want:
                continue
            pos = ctx - n_r + i
            qrow = widen(q[row], dtype)
            for h in range(Hq):
                g = h // G
                o, _ = attend(qrow[h], K[: pos + 1, g, :], V[: pos + 1, g, :], sc)
                out[row, h] = o
    return out
