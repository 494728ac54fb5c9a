"""Pins for the oracle's probability-based acceptance (CPU only).

Checked against closed forms of the softmax (uniform rows, one raised logit,
probabilities summing to one), the limiting cases of both rules (threshold 0
accepts every checked node, a threshold of 1 none; soft matching with the
draft probability equal to the target's accepts for every u < 1, u = 0
accepts every positive probability), the greedy scan it shares its path rule
with (replaying greedy matches as acceptance bits reproduces the pinned
greedy acceptance), brute force over root paths, and the acceptance rate of
soft matching over many seeded uniforms (a binomial bound).
"""

import numpy as np
import pytest

import oracle
from masked_verification_attention_amd import workloads as wl


def test_uniform_row_and_one_raised_logit():
    V = 1000
    row = np.zeros(V, dtype=np.float32)
    assert abs(oracle.target_prob(row, "f32", 17) - 1.0 / V) < 1e-15
    a, c = 3.0, 0.5
    row = np.full(V, c, dtype=np.float32)
    row[42] = a
    pa = np.exp(a) / (np.exp(a) + (V - 1) * np.exp(c))
    assert abs(oracle.target_prob(row, "f32", 42) - pa) < 1e-15
    assert abs(oracle.target_prob(row, "f32", 7) - np.exp(c) / (np.exp(a) + (V - 1) * np.exp(c))) < 1e-15


def test_probabilities_sum_to_one_bf16():
    rng = np.random.default_rng(12)
    row = wl.f32_to_bf16_bits(rng.standard_normal(300).astype(np.float32) * 4)
    total = sum(oracle.target_prob(row, "bf16", i) for i in range(300))
    assert abs(total - 1.0) < 1e-12
    # order follows the logits
    z = oracle.as_f64(row, "bf16")
    i, j = int(np.argmax(z)), int(np.argmin(z))
    assert oracle.target_prob(row, "bf16", i) > oracle.target_prob(row, "bf16", j)


def chain_case(rng, B, T, V):
    logits = rng.standard_normal((B, T, V)).astype(np.float32)
    draft = rng.integers(0, V, size=(B, T)).astype(np.int32)
    parent = np.tile(np.arange(-1, T - 1, dtype=np.int32), (B, 1))
    return logits, draft, parent


def test_threshold_limits():
    rng = np.random.default_rng(1)
    B, T, V = 3, 6, 50
    logits, draft, parent = chain_case(rng, B, T, V)
    n = np.full(B, T, dtype=np.int32)
    _, p, ok, A, path, _ = oracle.prob_accept(logits, "f32", n, draft, parent, None, 8, oracle.MODE_THRESHOLD, 0.0)
    assert ok.all() and (A == T).all()
    _, _, ok, A, _, bonus = oracle.prob_accept(logits, "f32", n, draft, parent, None, 8, oracle.MODE_THRESHOLD, 1.0)
    assert not ok.any() and (A == 0).all() and (bonus == -1).all()
    # a threshold between two adjacent distinct probabilities splits exactly there
    s = np.unique(p)
    t = float(0.5 * (s[len(s) // 2 - 1] + s[len(s) // 2]))
    _, _, ok, _, _, _ = oracle.prob_accept(logits, "f32", n, draft, parent, None, 8, oracle.MODE_THRESHOLD, t)
    np.testing.assert_array_equal(ok, p > t)
    assert 0 < ok.sum() < ok.size
    # a threshold equal to a probability does not accept it (strict comparison)
    _, _, ok, _, _, _ = oracle.prob_accept(logits, "f32", n, draft, parent, None, 8, oracle.MODE_THRESHOLD,
                                           float(s[0]))
    assert not ok[p == s[0]].any() and ok[p > s[0]].all()


def test_soft_limits():
    rng = np.random.default_rng(2)
    B, T, V = 3, 6, 40
    logits, draft, parent = chain_case(rng, B, T, V)
    n = np.full(B, T, dtype=np.int32)
    p = oracle.node_probs(logits, "f32", n, draft, None)
    u = rng.random((B, T)) * 0.999
    _, _, ok, A, _, _ = oracle.prob_accept(logits, "f32", n, draft, parent, None, 8, oracle.MODE_SOFT,
                                           draft_prob=p.astype(np.float32), uniform=u)
    assert ok.all() and (A == T).all()                     # p_d = p_t: min(1, 1) = 1 > u
    _, _, ok, _, _, _ = oracle.prob_accept(logits, "f32", n, draft, parent, None, 8, oracle.MODE_SOFT,
                                           draft_prob=np.ones((B, T)), uniform=np.zeros((B, T)))
    assert ok.all()                                        # u = 0 accepts any p > 0
    _, _, ok, A, _, _ = oracle.prob_accept(logits, "f32", n, draft, parent, None, 8, oracle.MODE_SOFT,
                                           draft_prob=np.zeros((B, T)), uniform=u)
    assert ok.all()                                        # a draft that never proposes x: accept if p_t > 0
    # the decision is the real-valued u < p_t / p_d: just below and just above the ratio
    r = p / 0.5
    below = np.minimum(r * (1 - 1e-9), 0.999999)
    _, _, ok, _, _, _ = oracle.prob_accept(logits, "f32", n, draft, parent, None, 8, oracle.MODE_SOFT,
                                           draft_prob=np.full((B, T), 0.5), uniform=below)
    assert ok.all()
    _, _, ok, _, _, _ = oracle.prob_accept(logits, "f32", n, draft, parent, None, 8, oracle.MODE_SOFT,
                                           draft_prob=np.full((B, T), 0.5), uniform=r * (1 + 1e-9))
    assert not ok.any()


@pytest.mark.parametrize("seed", range(60))
def test_greedy_bits_replay_the_greedy_acceptance(seed):
    # acceptance bits equal to greedy matches reproduce the pinned greedy scan with rows
    rng = np.random.default_rng(300 + seed)
    T = int(rng.integers(1, 30))
    par = np.full(T, -1, dtype=np.int32)
    for v in range(1, T):
        par[v] = int(rng.integers(-1, v))
    greedy = rng.integers(0, 3, size=T).astype(np.int32)
    draft = rng.integers(0, 3, size=T).astype(np.int32)
    vrow = np.array([v if rng.random() < 0.8 else int(rng.integers(-1, T)) for v in range(T)], dtype=np.int32)
    ok = np.array([vrow[v] == -1 or (0 <= vrow[v] < T and draft[v] == greedy[vrow[v]]) for v in range(T)])
    md = int(rng.integers(1, 8))
    A, path, last = oracle.scan_accepted(ok, par, T, md)
    A2, path2, last2, _ = oracle.accept_request_rows(draft, par, vrow, greedy, T, md)
    assert A == A2 and last == last2
    np.testing.assert_array_equal(path, path2)


def test_scan_brute_force():
    rng = np.random.default_rng(9)
    for _ in range(200):
        T = int(rng.integers(1, 12))
        par = np.full(T, -1, dtype=np.int32)
        for v in range(1, T):
            par[v] = int(rng.integers(-1, v))
        ok = rng.random(T) < 0.7
        md = int(rng.integers(1, 6))
        best = []
        for v in range(T):
            chain, u = [], v
            while u >= 0:
                chain.append(u)
                u = int(par[u])
            chain.reverse()
            if len(chain) <= md and all(ok[c] for c in chain):
                if len(chain) > len(best) or (len(chain) == len(best) and chain < best):
                    best = chain
        A, path, _ = oracle.scan_accepted(ok, par, T, md)
        assert A == len(best) and list(path[:A]) == best


def test_soft_acceptance_rate_matches_probability():
    # one node, p_d = 1: accepted iff u < p_t, so over N seeded uniforms the rate is p_t
    rng = np.random.default_rng(4)
    V = 20
    row = rng.standard_normal(V).astype(np.float32)
    x = int(np.argsort(row)[-3])
    pt = oracle.target_prob(row, "f32", x)
    N = 20000
    u = rng.random(N)
    hits = sum(oracle.decide(pt, oracle.MODE_SOFT, draft_p=1.0, u=float(ui)) for ui in u)
    sd = np.sqrt(N * pt * (1 - pt))
    assert abs(hits - N * pt) < 5 * sd
