"""Seeded synthetic workloads for paged KV-cache attention.

Every workload is the input of one "step" of the serving loop the pages
describe (vLLM: from PagedAttention to Speculative Decoding, section 3.2/3.3;
zihan-zhang.net vLLM study, section 3.2): a pool of fixed 16-token KV blocks,
per-sequence block tables that map logical blocks to shuffled physical ones,
the history K/V already cached, and the new token(s) whose K/V the step
scatters into the pool through ``slot_mapping`` before attention runs.

Values are N(0, 1) drawn in float32 and, for bf16 workloads, rounded to bf16
(round to nearest even).  All tensors are returned as raw bit patterns
(``uint16`` for bf16, ``uint32`` for fp32) so that byte-exact comparisons stay
trivial.  Nothing here computes attention.

Seeds: lengths come from ``default_rng(396_000 + config_no)``; the values of
q, K and V from streams keyed by ``(396_000 + config_no, tensor tag, chunk)``
(see ``_draw``); the physical block permutation comes from a separate stream
``default_rng(396_100 + config_no + 1000 * layout_variant)``, so the same
values can be laid out under several permutations.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16

CONFIG_NAMES = {
    1: "tiny_f32",
    2: "llama3_8b_b64",
    3: "llama2_70b_b256",
    4: "shared_prefix_32x4",
    5: "long_mixed",
}

# Scales of fp8 (E4M3) pools for the bf16 workloads above: code c of the K
# pool stands for value(c) * FP8_K_SCALE.  N(0, 1) draws reach about 5.5 in
# magnitude over a few million values; these scales put 6 (K) and 5 (V) at
# the format's largest value 448, so typical values land among the normal
# codes and the rare draws beyond saturate.  Neither is a power of two, so
# the quantizing division rounds.
FP8_K_SCALE = np.float32(6.0 / 448.0)
FP8_V_SCALE = np.float32(5.0 / 448.0)
FP8_POISON = 0x7F  # NaN code that fills fp8 pool slots before any write

_CHUNK = 1 << 22  # elements per independent stream (bounds peak host memory)
_TAG_Q, _TAG_K, _TAG_V = 1, 2, 3


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even) and return the 16-bit patterns.

    Inputs are finite draws from N(0, 1); NaN handling is not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def poison_bits(dtype: str) -> int:
    """Bit pattern of the NaN that fills every pool slot before any write."""
    return 0x7FA5 if dtype == "bf16" else 0x7FA5A5A5


def raw_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.uint32


def elem_bytes(dtype: str) -> int:
    return 2 if dtype == "bf16" else 4


def _draw(seed: int, tag: int, shape, dtype: str) -> np.ndarray:
    """N(0, 1) values for one tensor.  Chunk ``c`` of the flattened tensor comes
    from its own stream ``SeedSequence([seed, tag, c])``, so the result does not
    depend on how many threads draw it."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=raw_dtype(dtype))

    def fill(lo):
        hi = min(n, lo + _CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence([seed, tag, lo // _CHUNK]))
        x = rng.standard_normal(size=hi - lo, dtype=np.float32)
        out[lo:hi] = bf16_bits_from_f32(x) if dtype == "bf16" else x.view(np.uint32)

    starts = range(0, n, _CHUNK)
    if n > 4 * _CHUNK:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, starts))
    else:
        for lo in starts:
            fill(lo)
    return out.reshape(shape)


@dataclass
class DecodeWorkload:
    """One decode step: history already cached, one new token per sequence."""

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    context_lens: np.ndarray  # int32 [S], counts the new token
    block_tables: np.ndarray  # int32 [S, MB], padded with -1
    q: np.ndarray  # raw [S, Hq, D]
    hist_k: np.ndarray  # raw [Th, Hkv, D]
    hist_v: np.ndarray
    hist_slots: np.ndarray  # int64 [Th]
    new_k: np.ndarray  # raw [S, Hkv, D] (the token at position ctx-1)
    new_v: np.ndarray
    new_slots: np.ndarray  # int64 [S]
    scale: np.float32
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def kv_bytes(self) -> int:
        """K and V bytes attention must read: every cached token once per kv head."""
        return int(self.context_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * elem_bytes(self.dtype)


@dataclass
class PrefillWorkload:
    """Chunked prefill: each request's last ``n_r`` tokens are the query chunk."""

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    context_lens: np.ndarray  # int32 [R], prior + chunk
    query_start_loc: np.ndarray  # int32 [R+1]
    block_tables: np.ndarray  # int32 [R, MB]
    q: np.ndarray  # raw [sum n_r, Hq, D]
    hist_k: np.ndarray  # prior tokens
    hist_v: np.ndarray
    hist_slots: np.ndarray
    new_k: np.ndarray  # chunk tokens, in query order
    new_v: np.ndarray
    new_slots: np.ndarray
    scale: np.float32
    extra: dict = field(default_factory=dict)

    @property
    def num_reqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def total_q_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_q_len(self) -> int:
        return int(np.diff(self.query_start_loc).max()) if self.num_reqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])


# ----------------------------------------------------------------------------
# block assignment


def _assign_blocks(owners, num_blocks, rng_layout):
    """Give each logical block (listed by owner key, in first-use order) a
    distinct physical id drawn from a seeded permutation of the pool."""
    perm = rng_layout.permutation(num_blocks).astype(np.int32)
    ids = {}
    for key in owners:
        if key not in ids:
            ids[key] = perm[len(ids)]
    return ids


def _slots_for(table_row, positions):
    pos = np.asarray(positions, dtype=np.int64)
    return table_row[pos // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + pos % BLOCK_SIZE


def _build_decode(name, dtype, ctx, Hq, Hkv, D, mb, vseed, rng_l, *, prompt_of=None,
                  prompt_len=0, pool_factor=1.25, num_blocks=None, share=True):
    """Shared builder.

    ``prompt_of[s]`` (optional) names the prompt whose first ``prompt_len``
    tokens sequence ``s`` shares; with ``share=False`` every sequence gets a
    private copy of those blocks holding the same values.
    """
    S = len(ctx)
    ctx = np.asarray(ctx, dtype=np.int32)
    nbs = [(int(c) + BLOCK_SIZE - 1) // BLOCK_SIZE for c in ctx]
    pblocks = prompt_len // BLOCK_SIZE
    # logical block owners in first-use order
    owners = []
    for s in range(S):
        for j in range(nbs[s]):
            if prompt_of is not None and j < pblocks and share:
                owners.append(("p", int(prompt_of[s]), j))
            else:
                owners.append(("s", s, j))
    need = len(set(owners))
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * need))
    ids = _assign_blocks(owners, num_blocks, rng_l)
    tables = np.full((S, mb), -1, dtype=np.int32)
    for s in range(S):
        for j in range(nbs[s]):
            if prompt_of is not None and j < pblocks and share:
                tables[s, j] = ids[("p", int(prompt_of[s]), j)]
            else:
                tables[s, j] = ids[("s", s, j)]

    scale = np.float32(1.0 / math.sqrt(D))
    q = _draw(vseed, _TAG_Q, (S, Hq, D), dtype)
    # K/V values in logical order: prompts first (if any), then each
    # sequence's own tokens.
    n_prompts = 0 if prompt_of is None else int(np.max(prompt_of)) + 1
    own_start = [prompt_len if prompt_of is not None else 0 for _ in range(S)]
    n_own = [int(ctx[s]) - own_start[s] for s in range(S)]
    tot = n_prompts * prompt_len + sum(n_own)
    k_all = _draw(vseed, _TAG_K, (tot, Hkv, D), dtype)
    v_all = _draw(vseed, _TAG_V, (tot, Hkv, D), dtype)

    hist_rows, hist_slots, new_rows, new_slots = [], [], [], []
    base = n_prompts * prompt_len
    own_base = []
    for s in range(S):
        own_base.append(base)
        base += n_own[s]
    # prompt tokens: written once when shared, once per sequence otherwise
    if prompt_of is not None:
        written = set()
        for s in range(S):
            p = int(prompt_of[s])
            if share and p in written:
                continue
            written.add(p)
            rows = np.arange(p * prompt_len, (p + 1) * prompt_len)
            hist_rows.append(rows)
            hist_slots.append(_slots_for(tables[s], np.arange(prompt_len)))
    for s in range(S):
        pos = np.arange(own_start[s], int(ctx[s]))
        rows = own_base[s] + np.arange(n_own[s])
        hist_rows.append(rows[:-1])
        hist_slots.append(_slots_for(tables[s], pos[:-1]))
        new_rows.append(rows[-1:])
        new_slots.append(_slots_for(tables[s], pos[-1:]))
    hist_rows = np.concatenate(hist_rows) if hist_rows else np.zeros(0, np.int64)
    new_rows = np.concatenate(new_rows)
    wl = DecodeWorkload(
        name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        num_blocks=num_blocks, context_lens=ctx, block_tables=tables, q=q,
        hist_k=k_all[hist_rows], hist_v=v_all[hist_rows],
        hist_slots=np.concatenate(hist_slots).astype(np.int64),
        new_k=k_all[new_rows], new_v=v_all[new_rows],
        new_slots=np.concatenate(new_slots).astype(np.int64), scale=scale,
        extra={"unique_blocks": need},
    )
    return wl


def make_tiny_decode(seed=7, ctx=(5, 17, 33, 64), Hq=4, Hkv=2, D=64, dtype="f32",
                     num_blocks=None, mb=None, layout_variant=0, name="tiny"):
    """Small decode workload with arbitrary shape, for tests."""
    rng_l = np.random.default_rng(seed + 100 + 1000 * layout_variant)
    nbs = [(c + BLOCK_SIZE - 1) // BLOCK_SIZE for c in ctx]
    if mb is None:
        mb = max(max(nbs), 1)
    return _build_decode(name, dtype, list(ctx), Hq, Hkv, D, mb, seed, rng_l,
                         num_blocks=num_blocks)


def make_decode(cfg, layout_variant=0, private_copies=False):
    """The decode part of one of the five benchmark configurations.

    cfg 1: 4 seqs, ctx {5,17,33,64}, 4q/2kv, d=64, fp32, 32-block pool.
    cfg 2: Llama-3.1-8B layer: 64 seqs, ctx ~ U[128, 4096], 32q/8kv, d=128, bf16.
    cfg 3: Llama-2-70B layer: 256 seqs, ctx 2048, 64q/8kv, d=128, bf16.
    cfg 4: 32 prompts x 4 samples sharing 2048-token prompts, tails U[1, 256].
    cfg 5: 8 seqs at ctx 32768 (the decode half of the mixed batch).
    """
    cfg_no = int(cfg)
    name = CONFIG_NAMES[cfg_no]
    vseed = 396_000 + cfg_no
    rng_v = np.random.default_rng(vseed)
    rng_l = np.random.default_rng(396_100 + cfg_no + 1000 * layout_variant)
    if cfg_no == 1:
        return _build_decode(name, "f32", [5, 17, 33, 64], 4, 2, 64, 4, vseed, rng_l,
                             num_blocks=32)
    if cfg_no == 2:
        ctx = rng_v.integers(128, 4097, size=64)
        return _build_decode(name, "bf16", ctx, 32, 8, 128, 256, vseed, rng_l)
    if cfg_no == 3:
        return _build_decode(name, "bf16", [2048] * 256, 64, 8, 128, 128, vseed, rng_l)
    if cfg_no == 4:
        tails = rng_v.integers(1, 257, size=128)
        ctx = 2048 + tails
        prompt_of = np.repeat(np.arange(32), 4)
        wl = _build_decode(name, "bf16", ctx, 32, 8, 128, 144, vseed, rng_l,
                           prompt_of=prompt_of, prompt_len=2048, share=not private_copies)
        wl.extra["prompt_of"] = prompt_of
        wl.extra["prompt_len"] = 2048
        return wl
    if cfg_no == 5:
        dec, _ = make_mixed(layout_variant, parts=("decode",))
        return dec
    raise ValueError(f"unknown config {cfg}")


def _build_prefill(name, dtype, prior, chunk, Hq, Hkv, D, mb, vseed, rng_l,
                   num_blocks=None, pool_factor=1.25, reserve=0):
    R = len(prior)
    ctx = np.asarray([p + c for p, c in zip(prior, chunk)], dtype=np.int32)
    nbs = [(int(c) + BLOCK_SIZE - 1) // BLOCK_SIZE for c in ctx]
    need = sum(nbs) + reserve
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * need))
    owners = [("r", r, j) for r in range(R) for j in range(nbs[r])]
    ids = _assign_blocks(owners, num_blocks, rng_l)
    tables = np.full((R, mb), -1, dtype=np.int32)
    for r in range(R):
        for j in range(nbs[r]):
            tables[r, j] = ids[("r", r, j)]
    qsl = np.zeros(R + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(chunk)
    scale = np.float32(1.0 / math.sqrt(D))
    q = _draw(vseed, _TAG_Q, (int(qsl[-1]), Hq, D), dtype)
    tot = int(ctx.sum())
    k_all = _draw(vseed, _TAG_K, (tot, Hkv, D), dtype)
    v_all = _draw(vseed, _TAG_V, (tot, Hkv, D), dtype)
    hist_rows, hist_slots, new_rows, new_slots = [], [], [], []
    base = 0
    for r in range(R):
        pos = np.arange(int(ctx[r]))
        rows = base + pos
        base += int(ctx[r])
        hist_rows.append(rows[: prior[r]])
        hist_slots.append(_slots_for(tables[r], pos[: prior[r]]))
        new_rows.append(rows[prior[r]:])
        new_slots.append(_slots_for(tables[r], pos[prior[r]:]))
    hist_rows = np.concatenate(hist_rows)
    new_rows = np.concatenate(new_rows)
    return PrefillWorkload(
        name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        num_blocks=num_blocks, context_lens=ctx, query_start_loc=qsl,
        block_tables=tables, q=q, hist_k=k_all[hist_rows], hist_v=v_all[hist_rows],
        hist_slots=np.concatenate(hist_slots).astype(np.int64),
        new_k=k_all[new_rows], new_v=v_all[new_rows],
        new_slots=np.concatenate(new_slots).astype(np.int64), scale=scale,
        extra={"unique_blocks": sum(nbs)},
    )


def make_tiny_prefill(seed=11, prior=(0, 5, 40), chunk=(7, 16, 33), Hq=4, Hkv=2, D=128,
                      dtype="bf16", mb=None, layout_variant=0, name="tiny_prefill"):
    rng_l = np.random.default_rng(seed + 100 + 1000 * layout_variant)
    nbs = [(p + c + BLOCK_SIZE - 1) // BLOCK_SIZE for p, c in zip(prior, chunk)]
    if mb is None:
        mb = max(nbs)
    return _build_prefill(name, dtype, list(prior), list(chunk), Hq, Hkv, D, mb, seed, rng_l)


def make_prefill(cfg=5, layout_variant=0):
    """The prefill half of config 5: 4 requests, 512-token causal chunks
    against 4096 prior paged tokens, 32q/8kv, d=128, bf16."""
    if int(cfg) != 5:
        raise ValueError("only config 5 has a prefill part")
    _, pre = make_mixed(layout_variant, parts=("prefill",))
    return pre


def make_mixed(layout_variant=0, parts=("decode", "prefill")):
    """Config 5: long-context decode and chunked prefill sharing one pool.

    The pool holds 1.25x the blocks both halves need; the decode half takes
    the first blocks of the shuffled pool, the prefill half the next ones.
    ``parts`` may name only one half (the other comes back as None); each
    half is drawn from its own streams, so it is the same either way.
    """
    cfg_no = 5
    vseed = 396_000 + cfg_no
    rng_l = np.random.default_rng(396_100 + cfg_no + 1000 * layout_variant)
    dec_need = 8 * (32768 // BLOCK_SIZE)
    pre_need = 4 * ((4096 + 512) // BLOCK_SIZE)
    num_blocks = int(math.ceil(1.25 * (dec_need + pre_need)))
    perm = rng_l.permutation(num_blocks).astype(np.int32)

    class _Fixed:
        """Hands out consecutive slices of one shared permutation."""

        def __init__(self, ids):
            self.ids = ids

        def permutation(self, n):  # noqa: ARG002 - size is fixed by the pool
            return self.ids

    dec = pre = None
    if "decode" in parts:
        dec = _build_decode(CONFIG_NAMES[5], "bf16", [32768] * 8, 32, 8, 128, 2048, vseed,
                            _Fixed(perm[:dec_need]), num_blocks=num_blocks)
    if "prefill" in parts:
        pre = _build_prefill(CONFIG_NAMES[5] + "_prefill", "bf16", [4096] * 4, [512] * 4, 32, 8,
                             128, 288, vseed + 50, _Fixed(perm[dec_need:]), num_blocks=num_blocks)
    return dec, pre


def make_tiny_shared(seed=21, n_prompts=2, samples=3, prompt_len=32, tails=(1, 5, 16, 17, 3, 30),
                     Hq=4, Hkv=2, D=64, dtype="f32", private_copies=False, layout_variant=0):
    """Small shared-prefix workload: ``samples`` sequences per prompt share the
    prompt's full blocks (``prompt_len`` must be a multiple of 16) and own
    private tails.  With ``private_copies`` every sequence holds its own copy of
    the prompt blocks, with identical values."""
    assert prompt_len % BLOCK_SIZE == 0
    S = n_prompts * samples
    tails = list(tails)[:S]
    ctx = [prompt_len + t for t in tails]
    prompt_of = np.repeat(np.arange(n_prompts), samples)
    nbs = [(c + BLOCK_SIZE - 1) // BLOCK_SIZE for c in ctx]
    rng_l = np.random.default_rng(seed + 100 + 1000 * layout_variant)
    wl = _build_decode("tiny_shared", dtype, ctx, Hq, Hkv, D, max(nbs), seed, rng_l,
                       prompt_of=prompt_of, prompt_len=prompt_len, share=not private_copies,
                       num_blocks=2 * S * max(nbs))
    wl.extra["prompt_of"] = prompt_of
    wl.extra["prompt_len"] = prompt_len
    return wl


@dataclass
class SpecVerifyWorkload:
    """One verification round of speculative decoding over a decode batch.

    Every sequence has its last token and k drafted tokens appended: their
    K/V go into the pool and the target's attention runs those k + 1
    positions as a prefill chunk (``attn``).  The sampler's inputs are fp32
    target distributions p [B, k+1, V], draft distributions q [B, k, V], the
    drafted tokens (drawn from q) and uniforms in [0, 1) [B, k+1].
    """

    attn: PrefillWorkload
    target_probs: np.ndarray
    draft_probs: np.ndarray
    draft_tokens: np.ndarray
    uniforms: np.ndarray


def _softmax32(logits: np.ndarray) -> np.ndarray:
    z = logits.astype(np.float64)
    z -= z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def make_spec_verify(batch=64, k=4, vocab=128256, Hq=32, Hkv=8, D=128, seed=396_400,
                     ctx_lo=128, ctx_hi=4096, logit_std=2.5, draft_noise=0.8):
    """A verification round on the Llama-3.1-8B-shaped decode batch: context
    before the round U[ctx_lo, ctx_hi) tokens, k drafts per sequence, the
    Llama-3 vocabulary size by default.  Target logits are N(0, logit_std);
    draft logits add N(0, draft_noise) to them, so drafts are accepted often
    but not always."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(ctx_lo, ctx_hi, size=batch).tolist()
    chunk = [k + 1] * batch
    mb = max((p + k + 1 + BLOCK_SIZE - 1) // BLOCK_SIZE for p in prior)
    attn = _build_prefill("spec_verify", "bf16", prior, chunk, Hq, Hkv, D, mb, seed,
                          np.random.default_rng(seed + 1))
    lp = rng.standard_normal((batch, k + 1, vocab), dtype=np.float32) * np.float32(logit_std)
    target = _softmax32(lp)
    lq = lp[:, :k] + rng.standard_normal((batch, k, vocab), dtype=np.float32) * np.float32(draft_noise)
    draft = _softmax32(lq)
    toks = np.zeros((batch, k), dtype=np.int32)
    for b in range(batch):
        for i in range(k):
            c = np.cumsum(draft[b, i].astype(np.float64))
            toks[b, i] = min(int(np.searchsorted(c, rng.random() * c[-1], side="right")), vocab - 1)
    u = rng.random((batch, k + 1), dtype=np.float32)
    return SpecVerifyWorkload(attn, target, draft, toks, u)
