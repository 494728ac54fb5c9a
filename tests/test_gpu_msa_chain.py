"""Three chained multi-stream verification steps on the GPU, against the oracle.

Each step runs spec_build_msa_mask -> spec_verify_attn ->
spec_argmax_accept_commit (in place) -> spec_draft_tree, and the next step's
tree, draft tokens and node counts are the previous step's draft outputs,
moved device to device with no host decision in between.  The oracle runs the
same loop on its own state (cache, lengths, tree).  Fresh queries, block K/V
and logits are drawn per step on the host (with planted maxima on the
oracle's drafted tokens, so that paths are accepted) and given to both sides.
Bars: masks, acceptance, committed cache, lengths and drafts bit-exact;
attention within the bf16 bar.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from masked_verification_attention_amd import workloads as wl
from masked_verification_attention_amd.step import VerifyStep, to_device

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_three_chained_msa_steps():
    cfg = wl.CONFIGS["c6_msa_1b"].with_(gamma=3, branch=2, T=15, name="c6_chain")
    B = 2
    x = wl.generate(cfg, B=B, L=(60, 120))
    st = VerifyStep(cfg, x)
    rng = np.random.default_rng(77)
    Tq, T, V = cfg.Tq, cfg.T, cfg.V
    planted = wl.f32_to_bf16_bits(np.array([8.0], np.float32))[0]
    # oracle state
    kc, vc = x["k_cache"].copy(), x["v_cache"].copy()
    L = x["cache_len"].copy()
    tree = x["tree_parent"].copy()
    tok = x["draft_tok"][:, :T].copy()
    n_nodes = x["n_nodes"].copy()
    logits = x["logits"]
    q, kb, vb = x["q"], x["k_blk"], x["v_blk"]
    for step in range(3):
        say(f"[gpu] chained step {step}: nodes {n_nodes.tolist()}, lengths {L.tolist()}")
        st.build_mask()
        st.attention()
        st.accept_commit(in_place=True)
        st.draft()
        torch.cuda.synchronize()
        # oracle step
        bits, _, nq = oracle.build_msa_mask(tree, n_nodes, cfg.gamma, Tq)
        np.testing.assert_array_equal(st.mask_bits.cpu().numpy().view(np.uint32), bits)
        np.testing.assert_array_equal(st.n_q.cpu().numpy(), nq)
        vis = np.stack([oracle.msa_block_visibility(tree[b], int(n_nodes[b]), cfg.gamma, Tq) for b in range(B)])
        xin = dict(q=q, k_cache=kc, v_cache=vc, cache_len=L, k_blk=kb, v_blk=vb, n_q=nq)
        ref, _ = oracle.verify_attention(q, kc, vc, L, kb, vb, None, None, None, None, nq, cfg.dtype, block_vis=vis)
        out = st.out.cpu().numpy().astype(np.float64)
        for b in range(B):
            err = np.abs(out[b, :nq[b]] - ref[b, :nq[b]]).max()
            assert err <= 1e-2, (step, b, err)
        acc_parent = np.full((B, Tq), -1, np.int32)
        acc_parent[:, :T] = tree
        draft = np.zeros((B, Tq), np.int32)
        draft[:, :T] = tok
        _, A, path, _, bonus = oracle.argmax_accept_rows(logits, cfg.logits_dtype, n_nodes, draft, acc_parent,
                                                         acc_parent, st.max_depth)
        np.testing.assert_array_equal(st.out_len.cpu().numpy(), A)
        np.testing.assert_array_equal(st.out_path.cpu().numpy(), path)
        np.testing.assert_array_equal(st.out_bonus.cpu().numpy(), bonus)
        kc, vc, L = oracle.commit_kv(kc, vc, L, kb, vb, A, path)
        np.testing.assert_array_equal(st.cache_len.cpu().numpy(), L)
        k_host, v_host = st.cache_host()
        np.testing.assert_array_equal(k_host, kc)
        np.testing.assert_array_equal(v_host, vc)
        topk, ntok, npar, nn = oracle.next_draft(logits, cfg.logits_dtype, n_nodes, A, path, bonus, cfg.gamma,
                                                 cfg.branch)
        np.testing.assert_array_equal(st.next_tok.cpu().numpy(), ntok)
        np.testing.assert_array_equal(st.next_parent.cpu().numpy(), npar)
        np.testing.assert_array_equal(st.next_n.cpu().numpy(), nn)
        say(f"    accepted {A.tolist()}, correction {bonus.tolist()}, next draft nodes {nn.tolist()}")
        assert (A >= 1).all()                            # the explicit root is always accepted
        # next step: the draft becomes the tree (device to device on the GPU side)
        st.tree_parent.copy_(st.next_parent)
        st.acc_parent[:, :T].copy_(st.next_parent)
        st.draft_tok[:, :T].copy_(st.next_tok)
        st.n_nodes.copy_(st.next_n)
        tree, tok, n_nodes = npar, ntok, nn
        # fresh rows for the new block; plant each drafted node's token in its parent's row
        q = wl.f32_to_bf16_bits(rng.standard_normal(q.shape).astype(np.float32))
        kb = wl.f32_to_bf16_bits(rng.standard_normal(kb.shape).astype(np.float32))
        vb = wl.f32_to_bf16_bits(rng.standard_normal(vb.shape).astype(np.float32))
        logits = wl.f32_to_bf16_bits(rng.standard_normal(logits.shape).astype(np.float32))
        for b in range(B):
            for v in range(1, int(n_nodes[b])):
                if rng.random() < 0.7:
                    logits[b, tree[b, v], tok[b, v]] = planted
        st.q.copy_(to_device(q, "bf16", st.device))
        st.k_blk.copy_(to_device(kb, "bf16", st.device))
        st.v_blk.copy_(to_device(vb, "bf16", st.device))
        st.logits.copy_(to_device(logits, "bf16", st.device))
