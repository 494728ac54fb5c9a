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
