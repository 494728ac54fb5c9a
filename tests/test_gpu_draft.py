"""GPU parity of the next tree draft (spec_draft_tree) against the oracle.

Bit-exact: each stream's top-k tokens (order included, ties to the lower
token), the flattened tree's tokens and parents, and the node counts, for
bf16 and float32 logits, rows that start misaligned, forced ties, k from 1 to
8, no streams, and requests that get no draft.
"""

import sys
import zlib

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


CASES = [
    # (id, B, n nodes, gamma, k, V, dtype)
    ("bf16_c6", 4, 40, 3, 3, 50272, "bf16"),
    ("bf16_llama_vocab", 3, 15, 3, 2, 128256, "bf16"),
    ("bf16_misaligned", 3, 7, 2, 8, 1003, "bf16"),
    ("f32_misaligned", 3, 7, 2, 5, 1003, "f32"),
    ("greedy_chain", 2, 5, 6, 1, 32000, "bf16"),
    ("no_streams", 2, 9, 0, 4, 500, "bf16"),
    ("k_equals_v", 2, 4, 1, 8, 8, "f32"),
    ("one_stream_k8", 2, 31, 1, 8, 50272, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_draft_tree_parity(case):
    cid, B, n, gamma, k, V, dt = case
    rng = np.random.default_rng(zlib.crc32(cid.encode()))
    R = n * (1 + gamma) + 3
    max_depth = 6
    raw = rng.standard_normal((B, R, V)).astype(np.float32)
    # forced ties: repeat each row's largest values at other positions
    for b in range(B):
        for r in range(R):
            top = np.argsort(-raw[b, r])[:3]
            for t in top:
                raw[b, r, rng.integers(0, V)] = raw[b, r, t]
    data = wl.f32_to_bf16_bits(raw) if dt == "bf16" else raw
    n_nodes = np.full(B, n, dtype=np.int32)
    acc_len = rng.integers(1, max_depth + 1, size=B).astype(np.int32)
    acc_path = rng.integers(0, n, size=(B, max_depth)).astype(np.int32)
    root = rng.integers(0, V, size=B).astype(np.int32)
    if B > 2:
        acc_len[1] = 0                     # no accepted node: no draft
        acc_path[2, acc_len[2] - 1] = n    # last node outside the tree: no draft
    N = 1 + sum(k ** g for g in range(1, gamma + 1))
    dev = dict(dtype=torch.int32, device="cuda")
    lg = (torch.from_numpy(data.view(np.int16)).view(torch.bfloat16) if dt == "bf16"
          else torch.from_numpy(data)).cuda()
    t = {name: torch.from_numpy(a).cuda() for name, a in
         dict(n=n_nodes, len=acc_len, path=acc_path, root=root).items()}
    topk = torch.full((B, max(gamma, 1), k), -9, **dev)
    tok = torch.full((B, N), -9, **dev)
    par = torch.full((B, N), -9, **dev)
    n_out = torch.full((B,), -9, **dev)
    say(f"[gpu] draft {cid}: B={B} R={R} V={V} gamma={gamma} k={k}")
    bd.spec_draft_tree(lg, bd.SPEC_BF16 if dt == "bf16" else bd.SPEC_F32, B, R, V, t["n"], t["len"], t["path"],
                       max_depth, t["root"], gamma, k, topk, tok, par, n_out)
    torch.cuda.synchronize()
    r_topk, r_tok, r_par, r_n = oracle.next_draft(data, dt, n_nodes, acc_len, acc_path, root, gamma, k)
    if gamma:
        np.testing.assert_array_equal(topk.cpu().numpy(), r_topk)
    np.testing.assert_array_equal(tok.cpu().numpy(), r_tok)
    np.testing.assert_array_equal(par.cpu().numpy(), r_par)
    np.testing.assert_array_equal(n_out.cpu().numpy(), r_n)
    say(f"    draft nodes {r_n.tolist()}")


def test_rows_too_small_for_the_streams():
    # n * (1 + gamma) > R: the streams of the new root are not in the block
    B, n, gamma, k, V, R = 2, 10, 3, 2, 300, 30
    lg = torch.randn(B, R, V, device="cuda").to(torch.bfloat16)
    dev = dict(dtype=torch.int32, device="cuda")
    topk = torch.zeros(B, gamma, k, **dev)
    tok = torch.zeros(B, 15, **dev)
    par = torch.zeros(B, 15, **dev)
    n_out = torch.full((B,), 5, **dev)
    bd.spec_draft_tree(lg, bd.SPEC_BF16, B, R, V, torch.full((B,), n, **dev), torch.ones(B, **dev),
                       torch.zeros(B, 4, **dev), 4, torch.zeros(B, **dev), gamma, k, topk, tok, par, n_out)
    torch.cuda.synchronize()
    assert (n_out == 0).all() and (topk == -1).all() and (tok == -1).all() and (par == -1).all()


def _special_rows(V, rng):
    """Rows that exercise every path of the top-k: flat rows and long runs of equal
    values (more candidates than are ranked directly, and exactly at that limit),
    rows with fewer numbers than k (NaN places), infinities and signed zeros."""
    def normal():
        return rng.standard_normal(V).astype(np.float32)
    pats = [("flat", np.zeros(V, np.float32))]
    for cnt in (255, 256, 257, 300):
        a = normal()
        a[rng.choice(V, cnt, replace=False)] = a.max() + 1.0
        pats.append((f"{cnt}_ties_at_max", a))
    a = np.full(V, np.nan, np.float32)
    a[[5, 77]] = [1.0, -np.inf]
    pats.append(("two_numbers", a))
    pats.append(("all_nan", np.full(V, np.nan, np.float32)))
    a = np.full(V, -np.inf, np.float32)
    a[rng.choice(V, 3, replace=False)] = np.nan
    pats.append(("neg_inf_and_nan", a))
    a = normal()
    a[[9, 3]] = np.inf
    a[rng.choice(V, 50, replace=False)] = np.nan
    pats.append(("pos_inf_and_nan", a))
    a = np.where(rng.random(V) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    a[rng.choice(V, 20, replace=False)] = -1.0
    pats.append(("signed_zeros", a))
    return pats


def _to_bf16_bits(a):
    bits = wl.f32_to_bf16_bits(np.nan_to_num(a, nan=0.0, posinf=0.0, neginf=0.0))
    bits = np.where(np.isnan(a), np.uint16(0x7fc0), bits)
    bits = np.where(np.isposinf(a), np.uint16(0x7f80), bits)
    bits = np.where(np.isneginf(a), np.uint16(0xff80), bits)
    return bits.astype(np.uint16)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("k", [5, 8])
def test_draft_special_rows(dt, k):
    """Bit-exact top-k on crafted rows; request b's stream rows all hold pattern b."""
    rng = np.random.default_rng(17 + k)
    V, n, gamma, max_depth = 4099, 4, 2, 4
    pats = _special_rows(V, rng)
    B = len(pats)
    R = n * (1 + gamma)
    raw = np.ascontiguousarray(np.stack([np.broadcast_to(p, (R, V)) for _, p in pats]), dtype=np.float32)
    data = _to_bf16_bits(raw) if dt == "bf16" else raw
    n_nodes = np.full(B, n, dtype=np.int32)
    acc_len = np.ones(B, dtype=np.int32)
    acc_path = np.zeros((B, max_depth), dtype=np.int32)
    acc_path[:, 0] = rng.integers(0, n, size=B)
    root = np.arange(B, dtype=np.int32)
    N = 1 + sum(k ** g for g in range(1, gamma + 1))
    dev = dict(dtype=torch.int32, device="cuda")
    lg = (torch.from_numpy(data.view(np.int16)).view(torch.bfloat16) if dt == "bf16"
          else torch.from_numpy(data)).cuda()
    t = {name: torch.from_numpy(a).cuda() for name, a in
         dict(n=n_nodes, len=acc_len, path=acc_path, root=root).items()}
    topk = torch.full((B, gamma, k), -9, **dev)
    tok = torch.full((B, N), -9, **dev)
    par = torch.full((B, N), -9, **dev)
    n_out = torch.full((B,), -9, **dev)
    say(f"[gpu] draft special rows {dt} k={k}: {[p for p, _ in pats]}")
    bd.spec_draft_tree(lg, bd.SPEC_BF16 if dt == "bf16" else bd.SPEC_F32, B, R, V, t["n"], t["len"], t["path"],
                       max_depth, t["root"], gamma, k, topk, tok, par, n_out)
    torch.cuda.synchronize()
    r_topk, r_tok, r_par, r_n = oracle.next_draft(data, dt, n_nodes, acc_len, acc_path, root, gamma, k)
    got = topk.cpu().numpy()
    for b, (name, _) in enumerate(pats):
        np.testing.assert_array_equal(got[b], r_topk[b], err_msg=name)
    np.testing.assert_array_equal(tok.cpu().numpy(), r_tok)
    np.testing.assert_array_equal(par.cpu().numpy(), r_par)
    np.testing.assert_array_equal(n_out.cpu().numpy(), r_n)


def test_binding_refuses_strided_views():
    # the C ABI takes base pointers of dense arrays: a strided view is refused
    lg = torch.zeros(2, 12, 64, dtype=torch.float32, device="cuda").transpose(1, 2)
    dev = dict(dtype=torch.int32, device="cuda")
    z = torch.zeros(2, **dev)
    with pytest.raises(ValueError, match="contiguous"):
        bd.spec_draft_tree(lg, bd.SPEC_F32, 2, 12, 64, z, z, torch.zeros(2, 4, **dev), 4, z, 2, 2,
                           torch.zeros(2, 2, 2, **dev), torch.zeros(2, 7, **dev), torch.zeros(2, 7, **dev), z)
