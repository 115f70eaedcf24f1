"""CPU oracle for the verification step of speculative decoding.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline may import this module.  It shares no code with the HIP library.

What the pages fix (zihan-zhang.net vLLM study, 4.1.1; vLLM: from
PagedAttention to Speculative Decoding, 5.3-5.4):

* a cheap drafter proposes k tokens x_0..x_{k-1}, drawn from its
  distributions q_0..q_{k-1}; the target model scores all k + 1 positions in
  one forward pass, giving p_0..p_k;
* candidate x_i is accepted with probability min(1, p_i(x_i) / q_i(x_i)); the
  first rejection ends the round with one token drawn from the normalised
  positive part (p_i - q_i)_+;
* if all k are accepted, one more (bonus) token comes from p_k;
* the result has exactly the target's distribution, and with a per-token
  acceptance rate alpha a round yields (1 - alpha^(k+1)) / (1 - alpha) tokens
  on average.

Readings taken where the pages leave a step open:

* Randomness is an input: uniforms u_0..u_k in [0, 1) per request.  Candidate
  i is accepted iff u_i * q_i(x_i) <= p_i(x_i), the product and comparison
  exact (both factors are fp32, so the product is exact in fp64).  With u = 1
  this is the other page's deterministic rule, accept iff p(x) >= q(x).
* A draft token outside [0, vocab) is rejected.
* When drafts carry no distribution (draft_probs absent), q_i is one-hot at
  x_i, so acceptance happens with probability p_i(x_i).
* The final token is drawn by inverse CDF with u_k over integer weights:
  r_j = max(p_j - q_j, 0) evaluated in fp32 (a NaN counts as 0), weight
  w_j = floor(r_j * 2^32), W = sum of w_j, T = min(floor(u_k * W), W - 1)
  computed exactly, and the token is the smallest j whose running weight sum
  exceeds T.  Integer weights make the choice independent of summation order;
  they move each token's probability by at most 2^-32 / W of the normalised
  mass (the residual is normalised by W itself).  If the residual has no
  weight at all (W = 0), the token is drawn from p_i instead.

Everything is plain Python / NumPy with exact integer arithmetic.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

WEIGHT_ONE = 1 << 32


def accepts(p_x, q_x, u) -> np.ndarray:
    """Acceptance of a candidate with target probability p_x and draft
    probability q_x under uniform u: u * q_x <= p_x, exactly (fp32 inputs)."""
    p = np.asarray(p_x, dtype=np.float32).astype(np.float64)
    q = np.asarray(q_x, dtype=np.float32).astype(np.float64)
    uu = np.asarray(u, dtype=np.float32).astype(np.float64)
    return uu * q <= p


def weights(r32: np.ndarray) -> np.ndarray:
    """Integer weights floor(max(r, 0) * 2^32) of fp32 values (NaN -> 0)."""
    r = np.fmax(np.asarray(r32, dtype=np.float32), np.float32(0)).astype(np.float64)
    return np.floor(r * WEIGHT_ONE).astype(np.uint64)


def threshold(u, total: int) -> int:
    """T = floor(u * total) for an fp32 u, exact, kept inside [0, total - 1]
    (u <= 0 or NaN gives 0, u >= 1 gives total - 1)."""
    uf = float(np.float32(u))
    if not uf > 0:
        return 0
    return min(math.floor(Fraction(uf) * total), total - 1)


def sample_index(w: np.ndarray, u) -> int:
    """Smallest j whose running weight sum exceeds threshold(u, sum w); -1 if
    the weights are all zero."""
    cum = np.cumsum(w.astype(np.uint64), dtype=np.uint64)
    total = int(cum[-1]) if cum.size else 0
    if total == 0:
        return -1
    t = threshold(u, total)
    return int(np.searchsorted(cum, np.uint64(t), side="right"))


def residual(p_row: np.ndarray, q_row) -> np.ndarray:
    """(p - q)_+ in fp32, the distribution a rejection resamples from."""
    p = np.asarray(p_row, dtype=np.float32)
    q = np.asarray(q_row, dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        return np.fmax(p - q, np.float32(0))


def verify_request(target_probs, draft_probs, draft_tokens, uniforms):
    """One request's round: returns the emitted tokens (accepted drafts, then
    the resampled or bonus token).

    target_probs [k+1, V], draft_probs [k, V] or None (one-hot drafts),
    draft_tokens [k], uniforms [k+1], all fp32 / int32.
    """
    k = len(draft_tokens)
    V = target_probs.shape[1]
    out = []
    for i in range(k):
        x = int(draft_tokens[i])
        if 0 <= x < V:
            q_row = draft_probs[i] if draft_probs is not None else np.eye(1, V, x, dtype=np.float32)[0]
            ok = bool(accepts(target_probs[i, x], q_row[x], uniforms[i]))
        else:
            ok = False
        if ok:
            out.append(x)
            continue
        if 0 <= x < V:
            r = residual(target_probs[i], q_row)
        else:
            r = residual(target_probs[i], np.zeros(V, dtype=np.float32))
        j = sample_index(weights(r), uniforms[k])
        if j < 0:  # no residual weight: draw from p_i
            j = sample_index(weights(target_probs[i]), uniforms[k])
        out.append(j)
        return out
    out.append(sample_index(weights(target_probs[k]), uniforms[k]))
    return out


def rejection_sample(target_probs, draft_probs, draft_tokens, uniforms):
    """Every request of a batch.  Returns (out_tokens [B, k+1] padded with -1,
    num_tokens [B])."""
    B, k1, V = target_probs.shape
    out = np.full((B, k1), -1, dtype=np.int32)
    n = np.zeros(B, dtype=np.int32)
    for b in range(B):
        toks = verify_request(target_probs[b], None if draft_probs is None else draft_probs[b],
                              draft_tokens[b], uniforms[b])
        out[b, : len(toks)] = toks
        n[b] = len(toks)
    return out, n
