"""Pins for the oracle's argmax, acceptance scan and KV commit (CPU only).

Argmax is checked by a pure-Python first-maximum loop on constructed ties;
the acceptance scan by brute-force enumeration of root-to-leaf paths in
depth-first order (Speculative Streaming, the verification step) and by the
chain closed form (Lookahead Attention section 2.4: the longest consistent
prefix); the commit by its invariants.
"""

import itertools

import numpy as np
import pytest

import oracle
from masked_verification_attention_amd import workloads as wl


def first_max_loop(row):
    best, idx = None, -1
    for i, x in enumerate(row):
        if best is None or x > best:
            best, idx = x, i
    return idx


def test_argmax_first_max_on_ties_and_signed_zero():
    rows = np.array([
        [0.0, -0.0, -1.0, 0.0],
        [-0.0, 0.0, -2.0, -3.0],
        [1.0, 3.0, 3.0, 2.0],
        [-5.0, -4.0, -4.0, -4.5],
        [7.0, 7.0, 7.0, 7.0],
    ], dtype=np.float32)
    got = oracle.greedy_tokens(rows[None], "f32")[0]
    assert list(got) == [first_max_loop(r) for r in rows] == [0, 0, 1, 1, 0]
    bits = wl.f32_to_bf16_bits(rows)
    assert list(oracle.greedy_tokens(bits[None], "bf16")[0]) == [0, 0, 1, 1, 0]


def test_argmax_random_bf16_rows_with_natural_ties():
    rng = np.random.Generator(np.random.PCG64(3))
    x = wl.f32_to_bf16_bits(rng.standard_normal((64, 32000), dtype=np.float32))
    got = oracle.greedy_tokens(x[None], "bf16")[0]
    vals = oracle.bf16_bits_to_f64(x)
    assert list(got) == [first_max_loop(list(r)) for r in vals]
    # ties at the maximum do occur in bf16 rows of this width
    assert any((r == r.max()).sum() > 1 for r in vals)


def brute_force_accept(parent, ok, max_depth):
    """Enumerate root-to-leaf paths depth-first (children in index order)."""
    n = len(parent)
    children = {u: [v for v in range(n) if parent[v] == u] for u in [-1] + list(range(n))}
    best = (0, [])

    def walk(u, path):
        nonlocal best
        kids = children[u]
        if not kids:
            run = 0
            for node in path:
                if ok[node] and run < max_depth:
                    run += 1
                else:
                    break
            if run > best[0]:
                best = (run, path[:run])
            return
        for c in kids:
            walk(c, path + [c])

    walk(-1, [])
    return best


@pytest.mark.parametrize("seed", range(200))
def test_accept_matches_brute_force_on_small_trees(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(rng.integers(1, 9))
    parent = wl.random_forest(rng, n, int(rng.integers(1, 5)))
    greedy = rng.integers(0, 3, n).astype(np.int32)
    draft = rng.integers(0, 3, n).astype(np.int32)
    max_depth = int(rng.integers(1, 6))
    A, path = oracle.accept_request(draft, parent, greedy, n, max_depth)
    bA, bpath = brute_force_accept(parent, draft == greedy, max_depth)
    assert A == bA
    assert list(path[:A]) == bpath
    assert (path[A:] == -1).all()
    # path follows parent links from the root
    for d in range(A):
        assert parent[path[d]] == (-1 if d == 0 else path[d - 1])


@pytest.mark.parametrize("seed", range(50))
def test_chain_closed_form_leading_run(seed):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    k = int(rng.integers(1, 12))
    parent = np.arange(-1, k - 1, dtype=np.int32)
    ok = rng.random(k) < 0.7
    greedy = np.zeros(k, np.int32)
    draft = np.where(ok, 0, 1).astype(np.int32)
    A, path = oracle.accept_request(draft, parent, greedy, k, k)
    run = next((i for i, o in enumerate(ok) if not o), k)
    assert A == run
    assert list(path[:A]) == list(range(run))


def test_accept_properties():
    parent = np.array([-1, -1, 0, 0, 1, 2, 4], dtype=np.int32)
    n = len(parent)
    greedy = np.zeros(n, np.int32)
    # nothing matches at depth 1 -> A = 0 even if deeper nodes match
    draft = np.array([1, 1, 0, 0, 0, 0, 0], np.int32)
    A, path = oracle.accept_request(draft, parent, greedy, n, 8)
    assert A == 0 and (path == -1).all()
    # everything matches -> A = tree depth; DFS-first among the two depth-3 leaves (5 via 0,2 and 6 via 1,4)
    A, path = oracle.accept_request(np.zeros(n, np.int32), parent, greedy, n, 8)
    assert A == 3 and list(path[:3]) == [0, 2, 5]
    # the cap: nodes deeper than max_depth are never accepted
    A, path = oracle.accept_request(np.zeros(n, np.int32), parent, greedy, n, 2)
    assert A == 2 and list(path) == [0, 2]
    # n_nodes restricts the scan
    A, _ = oracle.accept_request(np.zeros(n, np.int32), parent, greedy, 2, 8)
    assert A == 1


def test_relabelling_keeps_length_and_maps_unique_path():
    rng = np.random.Generator(np.random.PCG64(11))
    for _ in range(30):
        n = 10
        parent = wl.random_forest(rng, n, 4)
        ok = rng.random(n) < 0.6
        A, path = oracle.accept_request(np.where(ok, 0, 1), parent, np.zeros(n, np.int32), n, 8)
        # a different topological numbering: reverse the sibling order under every node
        order = []

        def visit(u):
            kids = [v for v in range(n) if parent[v] == u]
            for c in reversed(kids):
                order.append(c)
                visit(c)
        visit(-1)
        new_of = {old: i for i, old in enumerate(order)}
        par2 = np.array([-1 if parent[o] < 0 else new_of[parent[o]] for o in order], np.int32)
        ok2 = ok[order]
        A2, path2 = oracle.accept_request(np.where(ok2, 0, 1), par2, np.zeros(n, np.int32), n, 8)
        assert A2 == A


def test_commit_invariants():
    rng = np.random.Generator(np.random.PCG64(5))
    B, lmax, Hkv, D, Tq = 3, 12, 2, 4, 5
    kc = rng.standard_normal((B, lmax, Hkv, D)).astype(np.float32)
    vc = rng.standard_normal((B, lmax, Hkv, D)).astype(np.float32)
    kb = rng.standard_normal((B, Tq, Hkv, D)).astype(np.float32)
    vb = rng.standard_normal((B, Tq, Hkv, D)).astype(np.float32)
    L = np.array([4, 0, 10], np.int32)
    A = np.array([3, 0, 4], np.int32)
    path = np.array([[0, 2, 4, -1], [-1, -1, -1, -1], [1, 3, 0, 2]], np.int32)
    k2, v2, L2 = oracle.commit_kv(kc, vc, L, kb, vb, A, path)
    assert list(L2) == [7, 0, 12]          # request 2 hits the capacity after 2 rows
    for b in range(B):
        written = L2[b] - L[b]
        for s in range(lmax):
            if L[b] <= s < L[b] + written:
                d = s - L[b]
                assert np.array_equal(k2[b, s], kb[b, path[b, d]])
                assert np.array_equal(v2[b, s], vb[b, path[b, d]])
            else:
                assert np.array_equal(k2[b, s], kc[b, s]) and np.array_equal(v2[b, s], vc[b, s])
