"""Pins for the oracle's next tree draft (CPU only).

Checked against what the Speculative Streaming page and plain definitions fix
independently of the oracle: the tree sizes the page prints (15 and 40
nodes), the complete k-ary tree of the generator (built by a heap formula,
not level by level), the enumeration of every root-to-leaf token path as the
Cartesian product of the streams' lists, top-1 = the pinned greedy token,
top-k order and exclusion properties on random rows with forced ties, a
brute-force check on tiny vocabularies, and the choice of the last accepted
node's stream rows.
"""

import itertools
import os

import numpy as np
import pytest

import oracle
from masked_verification_attention_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def printed_sizes():
    for line in open(os.path.join(GOLDEN, "ss_tree_sizes.txt")):
        if line.strip() and not line.startswith("#"):
            yield tuple(int(x) for x in line.split())


def test_printed_tree_sizes():
    for k, gamma, size in printed_sizes():
        topk = np.arange(gamma * k, dtype=np.int32).reshape(gamma, k)
        tok, par = oracle.draft_tree(topk, 99)
        assert len(tok) == len(par) == size


@pytest.mark.parametrize("k,gamma", [(1, 1), (1, 5), (2, 3), (3, 3), (4, 2), (2, 6), (8, 1), (3, 0)])
def test_tree_shape_equals_complete_kary_tree(k, gamma):
    rng = np.random.default_rng(k * 10 + gamma)
    topk = rng.integers(0, 1000, size=(gamma, k)).astype(np.int32)
    tok, par = oracle.draft_tree(topk, 7)
    np.testing.assert_array_equal(par, wl.kary_tree(k, gamma))
    assert tok[0] == 7 and par[0] == -1
    # every root-to-leaf path reads one token per stream: all k^gamma combinations, once each
    leaves = [v for v in range(len(par)) if v not in set(par.tolist())] if gamma else [0]
    paths = []
    for v in leaves:
        seq = []
        while v > 0:
            seq.append(int(tok[v]))
            v = int(par[v])
        paths.append(tuple(reversed(seq)))
    expected = list(itertools.product(*[list(topk[j]) for j in range(gamma)]))
    assert sorted(paths) == sorted(tuple(int(t) for t in p) for p in expected)
    # a node at depth g carries a token of stream g
    for v in range(1, len(par)):
        g, u = 0, v
        while u > 0:
            u, g = int(par[u]), g + 1
        assert tok[v] in topk[g - 1]


def test_top1_is_the_greedy_token():
    x = wl.generate(wl.CONFIGS["c2_la_7b"], B=2, L=(8, 8))
    lg = x["logits"]
    greedy = oracle.greedy_tokens(lg, "bf16")
    for b in range(lg.shape[0]):
        for t in range(lg.shape[1]):
            assert oracle.topk_tokens(lg[b, t], "bf16", 1)[0] == greedy[b, t]


@pytest.mark.parametrize("seed", range(30))
def test_topk_order_and_exclusion(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(8, 3000))
    k = int(rng.integers(1, 9))
    row = rng.standard_normal(V).astype(np.float32)
    # forced ties: copy some values, including the maximum, to other positions
    for _ in range(int(rng.integers(0, 6))):
        row[rng.integers(0, V)] = row[rng.integers(0, V)]
    row[rng.integers(0, V)] = row.max()
    bits = wl.f32_to_bf16_bits(row)                  # bf16 rounding makes more ties
    for data, dt in ((row, "f32"), (bits, "bf16")):
        vals = oracle.as_f64(data, dt)
        got = oracle.topk_tokens(data, dt, k)
        assert len(set(got.tolist())) == k
        for a, c in zip(got[:-1], got[1:]):          # best first, equal values in index order
            assert vals[a] > vals[c] or (vals[a] == vals[c] and a < c)
        rest = np.setdiff1d(np.arange(V), got)
        kth = vals[got[-1]]
        assert (vals[rest] <= kth).all()
        assert all(i > got[-1] for i in rest if vals[i] == kth)


def test_topk_brute_force_tiny():
    rng = np.random.default_rng(3)
    for _ in range(200):
        V = int(rng.integers(1, 7))
        k = int(rng.integers(1, V + 1))
        row = rng.integers(-2, 3, size=V).astype(np.float32)   # many ties
        best = None
        for combo in itertools.permutations(range(V), k):
            ok = True
            for a, c in zip(combo[:-1], combo[1:]):
                if not (row[a] > row[c] or (row[a] == row[c] and a < c)):
                    ok = False
            others = [i for i in range(V) if i not in combo]
            if ok and all(row[i] < row[combo[-1]] or (row[i] == row[combo[-1]] and i > combo[-1])
                          for i in others):
                assert best is None
                best = combo
        assert best is not None
        assert tuple(oracle.topk_tokens(row, "f32", k)) == best


def test_topk_nan_and_infinities_brute_force():
    """NaN ranks after every number (-inf included), lowest index first among NaNs;
    -0 ties with +0.  Checked against the full ordering of every element by
    (is NaN, larger value first, lower index first), written element by element."""
    rng = np.random.default_rng(5)
    choices = np.array([np.nan, -np.inf, np.inf, 0.0, -0.0, 1.0, -1.0], dtype=np.float32)
    for _ in range(300):
        V = int(rng.integers(1, 9))
        k = int(rng.integers(1, V + 1))
        row = choices[rng.integers(0, len(choices), size=V)]

        def before(a, c):
            na, nc = bool(np.isnan(row[a])), bool(np.isnan(row[c]))
            if na != nc:
                return nc                      # a number before a NaN
            if not na and row[a] != row[c]:
                return bool(row[a] > row[c])
            return a < c
        order = list(range(V))
        for i in range(V):                     # selection sort by the rule above
            m = i
            for c in range(i + 1, V):
                if before(order[c], order[m]):
                    m = c
            order[i], order[m] = order[m], order[i]
        assert list(oracle.topk_tokens(row, "f32", k)) == order[:k]


def test_next_draft_reads_last_accepted_node_streams():
    # request 0: path 0 -> 2 -> 5, so node 5's stream rows; request 1: nothing accepted;
    # request 2: last node outside the tree
    gamma, k, n, V = 2, 2, 7, 50
    R = n * (1 + gamma)
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((3, R, V)).astype(np.float32)
    for j in (1, 2):
        row = oracle.msa_row(n, gamma, 5, j)
        assert row == n + 5 * gamma + j - 1
        lg[0, row, [10 * j, 10 * j + 1]] = [50.0, 40.0]
    path = np.array([[0, 2, 5, -1], [-1, -1, -1, -1], [0, 9, -1, -1]], dtype=np.int32)
    topk, tok, par, n_out = oracle.next_draft(lg, "f32", np.array([n, n, n]), np.array([3, 0, 2]), path,
                                               np.array([123, 5, 6]), gamma, k)
    assert n_out.tolist() == [7, 0, 0]
    np.testing.assert_array_equal(topk[0], [[10, 11], [20, 21]])
    np.testing.assert_array_equal(tok[0], [123, 10, 11, 20, 21, 20, 21])
    np.testing.assert_array_equal(par[0], [-1, 0, 0, 1, 1, 2, 2])
    assert (tok[1:] == -1).all() and (par[1:] == -1).all() and (topk[1:] == -1).all()
