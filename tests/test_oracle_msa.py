"""Pins for the oracle's multi-stream (MSA) rows (CPU only).

Checked against what the Speculative Streaming page fixes independently of
the oracle: a mask worked by hand from Equations 1, 2 and 4, the tree and
batch sizes the page prints (1 + sum k^g nodes, (1 + gamma) rows per node),
the reduction to the plain tree rule when there are no speculative streams,
row-by-row key counts, a second construction (streams as chains hanging off
their node, run through the already pinned parent-array rule), and the
attention of one stream computed over the literal concatenation of
Equation 2's keys by torch's scaled-dot-product attention in float64.
"""

import os

import numpy as np
import pytest
import torch

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


def random_tree(rng, n):
    """Random topological tree: node 0 is the root, node v's parent uniform over [0, v)."""
    par = np.full(n, -1, dtype=np.int32)
    for v in range(1, n):
        par[v] = int(rng.integers(0, v))
    return par


def depth_of(par, v):
    d = 0
    while par[v] >= 0:
        v = par[v]
        d += 1
    return d


def test_hand_worked_mask_gamma2():
    expected = _read_matrix("ss_msa_mask_gamma2.txt")
    M = oracle.msa_block_visibility(np.array([-1, 0, 0]), 3, 2, 9)
    np.testing.assert_array_equal(M.astype(int), expected)


def test_printed_tree_and_batch_sizes():
    # golden: (k, gamma, tree size) as printed on the page; MSA rows = (1 + gamma) x tree size
    for line in open(os.path.join(GOLDEN, "ss_tree_sizes.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, gamma, size = (int(x) for x in line.split())
        tree = wl.kary_tree(k, gamma)
        assert len(tree) == size
        _, _, n_q = oracle.build_msa_mask(tree[None, :], np.array([size]), gamma, (1 + gamma) * size)
        assert int(n_q[0]) == (1 + gamma) * size
    assert wl.CONFIGS["c6_msa_1b"].Tq == 160 and wl.CONFIGS["c6_msa_1b"].T == 40


def test_no_streams_is_the_tree_rule():
    rng = np.random.default_rng(5)
    for _ in range(50):
        n = int(rng.integers(1, 40))
        par = random_tree(rng, n)
        np.testing.assert_array_equal(oracle.msa_block_visibility(par, n, 0, n),
                                      oracle.block_visibility(par, n, n))


@pytest.mark.parametrize("seed", range(20))
def test_key_counts_and_exclusions(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 30))
    gamma = int(rng.integers(0, 6))
    Tq = n * (1 + gamma) + int(rng.integers(0, 5))
    par = random_tree(rng, n)
    M = oracle.msa_block_visibility(par, n, gamma, Tq)
    main = np.zeros(Tq, dtype=bool)
    main[:n] = True
    for v in range(n):
        dv = depth_of(par, v)
        for j in range(gamma + 1):
            r = oracle.msa_row(n, gamma, v, j)
            assert M[r, r]
            assert M[r].sum() == dv + 1 + j
            assert M[r, main].sum() == dv + 1          # the main-stream path only
            if j == 0:
                assert not M[r, ~main].any()           # main streams never see a speculative row
            else:
                own = [oracle.msa_row(n, gamma, v, i) for i in range(1, gamma + 1)]
                others = np.ones(Tq, dtype=bool)
                others[:n] = False
                others[own] = False
                assert not M[r, others].any()          # no other node's streams
    assert not M[n * (1 + gamma):].any()               # padding rows see nothing
    assert sorted({oracle.msa_row(n, gamma, v, j) for v in range(n) for j in range(gamma + 1)}) == \
        list(range(n * (1 + gamma)))                   # the layout is a bijection onto the valid rows


def streams_as_chains(par, n, gamma, Tq):
    """Second construction: stream 1 hangs off its node's main row, stream j off stream j-1."""
    ap = np.full(Tq, -1, dtype=np.int32)
    ap[:n] = par[:n]
    for v in range(n):
        for j in range(1, gamma + 1):
            ap[n + v * gamma + j - 1] = v if j == 1 else n + v * gamma + j - 2
    return ap


@pytest.mark.parametrize("seed", range(30))
def test_equals_streams_as_parent_chains(seed):
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(1, 25))
    gamma = int(rng.integers(0, 7))
    Tq = n * (1 + gamma)
    par = random_tree(rng, n)
    ap = streams_as_chains(par, n, gamma, Tq)
    np.testing.assert_array_equal(oracle.msa_block_visibility(par, n, gamma, Tq),
                                  oracle.block_visibility(ap, Tq, Tq))


def test_stream_attention_is_equation_2_concatenation():
    # one request, the 3-node tree, gamma = 2: every row's output equals softmax attention
    # over [prefix | main history on its path | own streams <= j], gathered literally
    rng = np.random.default_rng(7)
    n, gamma, L, H, D = 3, 2, 5, 2, 8
    Tq = n * (1 + gamma)
    par = np.array([-1, 0, 0])
    q = rng.standard_normal((1, Tq, H, D)).astype(np.float32)
    kc = rng.standard_normal((1, L, H, D)).astype(np.float32)
    vc = rng.standard_normal((1, L, H, D)).astype(np.float32)
    kb = rng.standard_normal((1, Tq, H, D)).astype(np.float32)
    vb = rng.standard_normal((1, Tq, H, D)).astype(np.float32)
    vis = oracle.msa_block_visibility(par, n, gamma, Tq)[None]
    out, _ = oracle.verify_attention(q, kc, vc, np.array([L]), kb, vb, None, None, None, None,
                                     np.array([Tq]), "f32", block_vis=vis)
    for v in range(n):
        path = oracle.tree_path(par, v)[::-1]
        for j in range(gamma + 1):
            r = oracle.msa_row(n, gamma, v, j)
            keys = [("c", l) for l in range(L)] + [("b", u) for u in path] + \
                   [("b", n + v * gamma + i - 1) for i in range(1, j + 1)]
            K = np.stack([kc[0, i] if s == "c" else kb[0, i] for s, i in keys]).astype(np.float64)
            Vv = np.stack([vc[0, i] if s == "c" else vb[0, i] for s, i in keys]).astype(np.float64)
            for h in range(H):
                ref = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(q[0, r, h].astype(np.float64))[None, None, None],
                    torch.from_numpy(K[:, h])[None, None], torch.from_numpy(Vv[:, h])[None, None])
                np.testing.assert_allclose(out[0, r, h], ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)
