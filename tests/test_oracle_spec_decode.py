"""Pins for the speculative-decoding verification oracle.

Sources of truth, none of them the oracle itself:
* the tokens-per-round figure the pages print (tests/golden/), reached by
  simulation with drafts accepted at a known rate;
* the pages' central claim that verification leaves the target distribution
  unchanged: the distribution of the first emitted token, enumerated over a
  grid of uniforms, equals p_0;
* the other page's deterministic rule (accept iff p(x) >= q(x)) as the u = 1
  case;
* brute-force inverse-CDF sampling with exact fractions;
* special cases: all accepted (bonus from p_k), an out-of-range draft, a
  residual without weight.
The last tests plant mistakes and check that a pin fails.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.spec_decode as sd


def _golden(name):
    rows = []
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([float(x) for x in line.split()])
    return rows


def _dist(rng, V, sharp=1.0):
    x = rng.gamma(sharp, size=V).astype(np.float64)
    return (x / x.sum()).astype(np.float32)


# ----------------------------------------------------------------------------
# the printed tokens-per-round figure


def _mean_tokens(alpha, k, rounds, seed):
    """One-hot drafts whose token has target probability alpha: every
    candidate is accepted with probability alpha."""
    rng = np.random.default_rng(seed)
    V = 6
    tp = np.zeros((k + 1, V), dtype=np.float32)
    tp[:, 0] = alpha
    tp[:, 1:] = (1 - alpha) / (V - 1)
    toks = np.zeros(k, dtype=np.int32)
    total = 0
    u = rng.random((rounds, k + 1), dtype=np.float32)
    for r in range(rounds):
        total += len(sd.verify_request(tp, None, toks, u[r]))
    return total / rounds


def test_tokens_per_round_printed_on_pages():
    for alpha, k, lo, hi in _golden("spec_tokens_per_round.txt"):
        m = _mean_tokens(np.float32(alpha), int(k), 40_000, seed=1)
        assert lo <= m <= hi, m
        # and the closed form the same passage states (std of one round < 1.6)
        exact = (1 - alpha ** (k + 1)) / (1 - alpha)
        assert abs(m - exact) < 4 * 1.6 / np.sqrt(40_000), (m, exact)


def test_tokens_per_round_other_rates():
    for alpha, k in ((0.5, 2), (0.9, 6)):
        m = _mean_tokens(np.float32(alpha), k, 20_000, seed=2)
        exact = (1 - alpha ** (k + 1)) / (1 - alpha)
        assert abs(m - exact) < 4 * 2.5 / np.sqrt(20_000), (alpha, k, m, exact)


# ----------------------------------------------------------------------------
# the target distribution is preserved


def _first_token_distribution(p, q, M):
    """P(first emitted token = j) for k = 1, the draft x drawn from q, u_0 and
    u_1 on an M-point midpoint grid each; computed with the oracle's own
    accept and sample steps, vectorised over the grid."""
    V = len(p)
    grid = ((np.arange(M) + 0.5) / M).astype(np.float32)
    out = np.zeros(V)
    for x in range(V):
        acc = sd.accepts(p[x], q[x], grid).mean()
        w = sd.weights(sd.residual(p, q))
        picks = np.array([sd.sample_index(w, u) for u in grid])
        res = np.bincount(picks, minlength=V) / M
        out += float(q[x]) * (acc * np.eye(V)[x] + (1 - acc) * res)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_first_token_follows_target_distribution(seed):
    rng = np.random.default_rng(seed)
    V = 7
    p, q = _dist(rng, V, 0.7), _dist(rng, V, 0.7)
    got = _first_token_distribution(p, q, 2048)
    assert np.allclose(got, p.astype(np.float64), atol=3e-3), (got, p)


def test_whole_round_by_enumeration_k1():
    """verify_request itself over a coarse grid of (x, u0, u1)."""
    rng = np.random.default_rng(9)
    V, M = 5, 96
    p0, p1, q0 = _dist(rng, V), _dist(rng, V), _dist(rng, V)
    tp = np.stack([p0, p1])
    grid = ((np.arange(M) + 0.5) / M).astype(np.float32)
    freq = np.zeros(V)
    for x in range(V):
        for u0 in grid:
            for u1 in grid:
                t = sd.verify_request(tp, q0[None, :], np.array([x], dtype=np.int32),
                                      np.array([u0, u1], dtype=np.float32))
                freq[t[0]] += float(q0[x]) / (M * M)
    assert np.allclose(freq, p0, atol=2.5e-2), (freq, p0)


# ----------------------------------------------------------------------------
# rules and special cases


def test_u_one_is_the_deterministic_rule():
    rng = np.random.default_rng(4)
    for _ in range(200):
        V = 9
        p, q = _dist(rng, V), _dist(rng, V)
        x = int(rng.integers(V))
        t = sd.verify_request(np.stack([p, p]), q[None, :], np.array([x], dtype=np.int32),
                              np.array([1.0, 0.5], dtype=np.float32))
        assert (t[0] == x and len(t) == 2) == bool(p[x] >= q[x])


def test_all_accepted_gives_bonus_from_last_target():
    k, V = 3, 8
    tp = np.zeros((k + 1, V), dtype=np.float32)
    tp[:k, 2] = 1.0
    tp[k, 5] = 1.0
    t = sd.verify_request(tp, None, np.array([2, 2, 2], dtype=np.int32),
                          np.array([0.3, 0.9, 0.99, 0.4], dtype=np.float32))
    assert t == [2, 2, 2, 5]


def test_rejection_resamples_from_positive_residual():
    # p = (0.5, 0.5, 0), q = (0.1, 0.9, 0): residual (0.4, 0, 0) -> token 0
    p = np.array([0.5, 0.5, 0.0], dtype=np.float32)
    q = np.array([0.1, 0.9, 0.0], dtype=np.float32)
    t = sd.verify_request(np.stack([p, p]), q[None, :], np.array([1], dtype=np.int32),
                          np.array([0.99, 0.7], dtype=np.float32))
    assert t == [0]
    # u_0 = 0.5: 0.5 * 0.9 = 0.45 <= 0.5 accepts
    t = sd.verify_request(np.stack([p, p]), q[None, :], np.array([1], dtype=np.int32),
                          np.array([0.5, 0.7], dtype=np.float32))
    assert t == [1, 1]


def test_out_of_range_draft_is_rejected():
    p = np.array([0.25, 0.75], dtype=np.float32)
    for x in (-1, 2, 1000):
        t = sd.verify_request(np.stack([p, p]), None, np.array([x], dtype=np.int32),
                              np.array([0.0, 0.1], dtype=np.float32))
        assert t == [0]  # resampled from p itself (q is zero there): 0.1 * W lands in token 0


def test_zero_residual_falls_back_to_target():
    p = np.array([0.2, 0.8], dtype=np.float32)
    # q = p everywhere but u * q(x) > p(x) is impossible ... force a rejection
    # with an out-of-contract q(x) > p(x) at x and q >= p elsewhere
    q = np.array([0.9, 0.8], dtype=np.float32)
    t = sd.verify_request(np.stack([p, p]), q[None, :], np.array([0], dtype=np.int32),
                          np.array([0.9, 0.5], dtype=np.float32))
    assert t == [1]  # residual all zero -> drawn from p: 0.5 * W falls in token 1


def test_sample_index_matches_exact_inverse_cdf():
    rng = np.random.default_rng(5)
    for _ in range(300):
        V = int(rng.integers(1, 40))
        r = rng.random(V).astype(np.float32) * (rng.random(V) < 0.7)
        u = np.float32(rng.random())
        w = sd.weights(r)
        W = sum(int(x) for x in w)
        got = sd.sample_index(w, u)
        if W == 0:
            assert got == -1
            continue
        t = min(int(Fraction(float(u)) * W), W - 1)
        acc, want = 0, None
        for j in range(V):
            acc += int(w[j])
            if acc > t:
                want = j
                break
        assert got == want


def test_weights_and_threshold_are_exact():
    assert int(sd.weights(np.array([1.0], dtype=np.float32))[0]) == 1 << 32
    assert int(sd.weights(np.array([2.0 ** -33], dtype=np.float32))[0]) == 0
    assert int(sd.weights(np.array([np.nan, -1.0], dtype=np.float32)).sum()) == 0
    assert sd.threshold(np.float32(0.5), 7) == 3
    assert sd.threshold(np.float32(1.0), 7) == 6
    big = (1 << 49) + 12345
    u = np.float32(0.999999940395355224609375)  # largest fp32 below 1
    assert sd.threshold(u, big) == (big * ((1 << 24) - 1)) >> 24


def test_batch_layout_and_padding():
    rng = np.random.default_rng(6)
    B, k, V = 5, 4, 11
    tp = np.stack([np.stack([_dist(rng, V) for _ in range(k + 1)]) for _ in range(B)])
    dp = np.stack([np.stack([_dist(rng, V) for _ in range(k)]) for _ in range(B)])
    toks = rng.integers(0, V, size=(B, k)).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    out, n = sd.rejection_sample(tp, dp, toks, u)
    for b in range(B):
        t = sd.verify_request(tp[b], dp[b], toks[b], u[b])
        assert n[b] == len(t) and list(out[b, : n[b]]) == t
        assert (out[b, n[b]:] == -1).all()


# ----------------------------------------------------------------------------
# planted mistakes


def test_planted_reversed_residual_is_caught(monkeypatch):
    orig = sd.residual
    monkeypatch.setattr(sd, "residual", lambda p, q: orig(q, p))
    with pytest.raises(AssertionError):
        test_first_token_follows_target_distribution(0)


def test_planted_inverted_ratio_is_caught(monkeypatch):
    orig = sd.accepts
    monkeypatch.setattr(sd, "accepts", lambda p, q, u: orig(q, p, u))
    with pytest.raises(AssertionError):
        test_tokens_per_round_printed_on_pages()


def test_planted_missing_bonus_is_caught(monkeypatch):
    orig = sd.verify_request

    def no_bonus(tp, dp, toks, u):
        t = orig(tp, dp, toks, u)
        return t[:-1] if len(t) == len(toks) + 1 else t

    monkeypatch.setattr(sd, "verify_request", no_bonus)
    with pytest.raises(AssertionError):
        test_tokens_per_round_printed_on_pages()
