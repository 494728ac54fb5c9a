"""GPU parity of spec_argmax_accept_rows (explicit verification rows, an
explicit root, the correction token) against the fp64 oracle: bit-exact
argmax, accepted lengths, paths and correction tokens."""

import sys

import numpy as np
import pytest
import torch

import oracle
from masked_verification_attention_amd import binding as bd
from masked_verification_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_rows(logits, dtype, n_nodes, draft, parent, verify_row, max_depth):
    B, T, V = logits.shape
    if dtype == "bf16":
        lg = torch.from_numpy(logits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        lg = torch.from_numpy(logits).cuda()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    out = torch.empty(B, T, dtype=torch.int32, device="cuda")
    ln = torch.empty(B, dtype=torch.int32, device="cuda")
    pth = torch.empty(B, max_depth, dtype=torch.int32, device="cuda")
    bonus = torch.empty(B, dtype=torch.int32, device="cuda")
    vr = None if verify_row is None else dev(verify_row)
    bd.spec_argmax_accept_rows(lg, bd.SPEC_F32 if dtype == "f32" else bd.SPEC_BF16, B, T, V, dev(n_nodes),
                               dev(draft), dev(parent), vr, max_depth, out, ln, pth, bonus)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ln.cpu().numpy(), pth.cpu().numpy(), bonus.cpu().numpy()


def check(logits, dtype, n_nodes, draft, parent, verify_row, max_depth):
    got = run_rows(logits, dtype, n_nodes, draft, parent, verify_row, max_depth)
    g, A, path, _, bonus = oracle.argmax_accept_rows(logits, dtype, n_nodes, draft, parent, verify_row, max_depth)
    g = g.copy()
    for b in range(len(n_nodes)):
        g[b, int(n_nodes[b]):] = -1   # rows past n_nodes are not computed
    np.testing.assert_array_equal(got[0], g)
    np.testing.assert_array_equal(got[1], A)
    np.testing.assert_array_equal(got[2], path)
    np.testing.assert_array_equal(got[3], bonus)
    return A


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_random_rows_small_trees(dtype):
    rng = np.random.Generator(np.random.PCG64(41))
    B, T, V = 24, 20, 37
    x = rng.integers(-3, 4, (B, T, V)).astype(np.float32)   # many ties at the maximum
    logits = x if dtype == "f32" else wl.f32_to_bf16_bits(x)
    greedy = oracle.greedy_tokens(logits, dtype)
    parent = np.stack([wl.random_forest(rng, T, int(rng.integers(1, 8))) for _ in range(B)])
    n_nodes = rng.integers(0, T + 1, B).astype(np.int32)
    verify_row = rng.choice(np.array([-1, -2, T, T + 9] + list(range(T))), size=(B, T)).astype(np.int32)
    # half the drafts copy the greedy token of their verification row
    draft = rng.integers(0, V, (B, T)).astype(np.int32)
    for b in range(B):
        for v in range(T):
            u = verify_row[b, v]
            if 0 <= u < T and rng.random() < 0.6:
                draft[b, v] = greedy[b, u]
    A = check(logits, dtype, n_nodes, draft, parent, verify_row, 8)
    say(f"    accepted lengths {A.tolist()}")
    assert A.max() > 1


def test_null_rows_is_same_position_acceptance():
    cfg = wl.CONFIGS["c3_confu_8b"]
    x = wl.generate(cfg, B=4, L=(8, 8))
    got = run_rows(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"], x["acc_parent"], None, 6)
    g, A, path = oracle.argmax_accept(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                      x["acc_parent"], 6)
    np.testing.assert_array_equal(got[1], A)
    np.testing.assert_array_equal(got[2], path)
    for b in range(len(A)):
        assert got[3][b] == (g[b, path[b, A[b] - 1]] if A[b] else -1)


def test_real_model_layout_full_vocabulary():
    """Explicit root (node 0, accepted unchecked), every other node verified by
    its parent's row, distinct tokens among siblings, and the target's greedy
    token planted at each parent row (the maximum of a bf16 N(0,1) row is far
    below the planted value) on one child w.p. 0.8: the Llama-3 vocabulary,
    30 drafted nodes plus the root per request."""
    rng = np.random.Generator(np.random.PCG64(1234))
    B, T, V = 8, 31, 128256
    logits32 = rng.standard_normal((B, T, V), dtype=np.float32)
    parent = np.full((B, T), -1, np.int32)
    draft = np.zeros((B, T), np.int32)
    for b in range(B):
        depth = np.zeros(T, np.int64)
        for v in range(1, T):
            cand = [u for u in range(v) if depth[u] < 6]
            parent[b, v] = cand[int(rng.integers(0, len(cand)))]
            depth[v] = depth[parent[b, v]] + 1
        for u in range(T):
            kids = [c for c in range(T) if parent[b, c] == u]
            toks = rng.choice(V, size=len(kids), replace=False)
            for c, t in zip(kids, toks):
                draft[b, c] = t
            if kids and rng.random() < 0.8:
                logits32[b, u, draft[b, kids[int(rng.integers(0, len(kids)))]]] = wl.PLANTED_LOGIT
        draft[b, 0] = int(rng.integers(0, V))   # the root's token: the previous correction token
    logits = wl.f32_to_bf16_bits(logits32)
    verify_row = np.where(parent < 0, -1, parent).astype(np.int32)
    A = check(logits, "bf16", np.full(B, T, np.int32), draft, parent, verify_row, 7)
    say(f"    accepted lengths (root included) {A.tolist()}")
    assert (A >= 1).all() and A.max() > 2


def test_rows_edge_cases():
    rng = np.random.Generator(np.random.PCG64(7))
    B, T, V = 4, 6, 11
    logits = rng.standard_normal((B, T, V)).astype(np.float32)
    parent = np.tile(np.array([-1, 0, 1, 2, 3, 4], np.int32), (B, 1))
    draft = np.zeros((B, T), np.int32)
    # request 0: no nodes; 1: every node unchecked (A = min(depth, max_depth));
    # 2: rows below -1 or past n_nodes (no match); 3: a single unchecked root
    n_nodes = np.array([0, 6, 6, 1], np.int32)
    verify_row = np.array([[0] * 6, [-1] * 6, [-1, -5, 6, 7, 100, -2], [-1, 0, 0, 0, 0, 0]], np.int32)
    A = check(logits, "f32", n_nodes, draft, parent, verify_row, 4)
    assert A.tolist() == [0, 4, 1, 1]
