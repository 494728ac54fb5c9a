"""Pins for the oracle's visibility masks (CPU only).

The oracle's mask is checked against what the pages fix independently of it:
the 7x7 mask drawn on the Lookahead Attention page, the block formula of its
section 3.1, the tree sizes printed on the Speculative Streaming page, the
ancestor closure computed a different way (boolean matrix powers), and
ConFu's rule that only contemplate rows see the soft prompt.
"""

import os

import numpy as np
import pytest

import oracle
from masked_verification_attention_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_matrix(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.array(rows)


def la_full_parents(n, k):
    """Originals as a chain, every lookahead row hanging off the last original."""
    return np.array(list(range(-1, n - 1)) + [n - 1] * k, dtype=np.int32)


def test_la_mask_matches_drawn_example_after_reading():
    drawn = _read_matrix("la_drawn_mask_n4_k3.txt")
    assert drawn.shape == (7, 7)
    n, k = 4, 3
    expected = drawn.T.copy()
    expected[:n, :n] = np.tril(np.ones((n, n), dtype=int))
    M = oracle.block_visibility(la_full_parents(n, k), n + k, n + k)
    np.testing.assert_array_equal(M.astype(int), expected)
    # The pinned matrix, written out (rows = queries).
    pinned = ["1000000", "1100000", "1110000", "1111000", "1111100", "1111010", "1111001"]
    assert ["".join(str(x) for x in row) for row in M.astype(int)] == pinned


@pytest.mark.parametrize("n,k", [(4, 3), (5, 1), (8, 8), (128, 4)])
def test_la_mask_equals_block_formula(n, k):
    # Section 3.1: [[M_causal, 1_{n x k}], [0_{k x n}, M_lookahead]] in key x query
    # layout, M_causal causal over the originals, M_lookahead diagonal.
    kq = np.zeros((n + k, n + k), dtype=bool)
    kq[:n, :n] = np.triu(np.ones((n, n), dtype=bool))   # key i visible to query j iff i <= j
    kq[:n, n:] = True
    kq[n:, :n] = False
    kq[n:, n:] = np.eye(k, dtype=bool)
    M = oracle.block_visibility(la_full_parents(n, k), n + k, n + k)
    np.testing.assert_array_equal(M, kq.T)


def test_la_cache_form_is_diagonal():
    # Originals already in the cache: each lookahead row sees only itself in the block.
    k = 8
    M = oracle.block_visibility(np.full(k, -1, np.int32), k, k)
    np.testing.assert_array_equal(M, np.eye(k, dtype=bool))
    D = oracle.dense_visibility(np.full(k, -1, np.int32), None, k, 0, 100)
    assert D[:, :100].all()


def full_tree_parents(k, gamma):
    """Flattened full k-ary tree with its root at row 0, level by level."""
    parents = [-1]
    level = [0]
    for _ in range(gamma):
        nxt = []
        for p in level:
            for _ in range(k):
                parents.append(p)
                nxt.append(len(parents) - 1)
        level = nxt
    return np.array(parents, dtype=np.int32)


def _depths(parent):
    d = np.zeros(len(parent), dtype=int)
    for v, p in enumerate(parent):
        d[v] = 0 if p < 0 else d[p] + 1
    return d


def test_tree_sizes_and_popcounts_match_printed_sizes():
    sizes = _read_matrix("ss_tree_sizes.txt")
    for k, gamma, size in sizes:
        par = full_tree_parents(k, gamma)
        assert len(par) == size == 1 + sum(k ** g for g in range(1, gamma + 1))
        M = oracle.block_visibility(par, size, size)
        depth = _depths(par)              # root at depth 0
        # each node sees the path from the root to itself: depth + 1 block keys
        np.testing.assert_array_equal(M.sum(axis=1), depth + 1)
        assert M.sum() == sum(k ** g * (g + 1) for g in range(gamma + 1))


def _closure_by_matrix_powers(parent):
    n = len(parent)
    A = np.zeros((n, n), dtype=np.int64)
    for v, p in enumerate(parent):
        if p >= 0:
            A[v, p] = 1
    R = np.eye(n, dtype=np.int64)
    P = np.eye(n, dtype=np.int64)
    for _ in range(n):
        P = np.minimum(P @ A, 1)
        R = np.maximum(R, P)
    return R.astype(bool)


@pytest.mark.parametrize("seed", range(6))
def test_tree_mask_is_reflexive_ancestor_closure(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    par = wl.random_forest(rng, 30, 6)
    M = oracle.block_visibility(par, 30, 30)
    np.testing.assert_array_equal(M, _closure_by_matrix_powers(par))
    # no node sees a node of another branch: visible keys are exactly the path
    for r in range(30):
        path = {r} | set(oracle.ancestor_rows(par, r))
        assert set(np.nonzero(M[r])[0]) == path


def test_tree_node_sees_parent_but_not_other_branches():
    par = full_tree_parents(2, 3)
    M = oracle.block_visibility(par, len(par), len(par))
    depth = _depths(par)
    for r in range(len(par)):
        for c in range(len(par)):
            if depth[c] == depth[r] - 1:
                assert M[r, c] == (c == par[r])


def test_confu_soft_and_contemplate_rules():
    cfg = wl.CONFIGS["c3_confu_8b"]
    x = wl.generate(cfg, B=2, L=(32, 32), with_logits=False)
    T = cfg.T
    for b in range(2):
        D = oracle.dense_visibility(x["attn_parent"][b], x["sp_flag"][b], cfg.Tq, cfg.S, 32)
        soft, prefix, blk = D[:, :cfg.S], D[:, cfg.S:cfg.S + 32], D[:, cfg.S + 32:]
        assert soft.any(axis=1).sum() == T                   # 2T rows, T of them contemplate
        assert not soft[:T].any() and soft[T:].all()
        assert prefix.all()
        assert not blk[:T, T:].any()                          # nodes never see contemplate rows
        for v in range(T):
            path = {v} | set(oracle.ancestor_rows(x["attn_parent"][b], v))
            assert set(np.nonzero(blk[T + v])[0]) == path | {T + v}


def test_padded_rows_see_nothing_and_bits_pack_lsb_first():
    par = np.array([-1, 0, 1, -1, 3, -1], dtype=np.int32)
    sp = np.array([0, 0, 1, 1, 1, 1], dtype=np.uint8)
    bits, sp_bits = oracle.build_mask(par[None], sp[None], np.array([4]))
    M = oracle.block_visibility(par, 4, 6)
    assert not M[4:].any()
    for r in range(6):
        for c in range(6):
            assert bool((int(bits[0, r, c // 32]) >> (c % 32)) & 1) == M[r, c]
    assert int(sp_bits[0, 0]) == 0b001100
    # 40-row tree spans two words
    par40 = full_tree_parents(3, 3)
    bits40, _ = oracle.build_mask(par40[None], None, np.array([40]))
    assert bits40.shape == (1, 40, 2)
    assert int(bits40[0, 39, 1]) >> 7 & 1 == 1 and int(bits40[0, 39, 0]) & 1 == 1


def test_non_topological_parent_rejected():
    with pytest.raises(ValueError):
        oracle.block_visibility(np.array([1, -1], dtype=np.int32), 2, 2)
