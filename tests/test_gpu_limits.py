"""The library's stated limits, through the C ABI against the fp64 oracle: the
largest soft prompt (SPEC_MAX_SOFT rows, eight soft tiles), the largest key
split (64 ranges), and acceptance capped at the longest path (SPEC_MAX_DEPTH)
on a chain whose every draft matches, with the commit of that many rows."""

import sys

import numpy as np
import pytest
import torch

import oracle
from masked_verification_attention_amd import binding as bd
from masked_verification_attention_amd import workloads as wl
from masked_verification_attention_amd.step import VerifyStep, to_host_bits

pytestmark = pytest.mark.gpu

BF16_ATOL = 1e-2
BF16_REL_L2 = 5e-3
LSE_ATOL = 2e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_against_oracle(st, x, cfg, what):
    torch.cuda.synchronize()
    got, got_lse = st.out.cpu().numpy(), st.lse.cpu().numpy()
    ref, ref_lse = oracle.verify_attention(x["q"], x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"],
                                           x["v_blk"], x["k_soft"] if cfg.S else None,
                                           x["v_soft"] if cfg.S else None, x["attn_parent"], x["sp_flag"],
                                           x["n_q"], cfg.dtype)
    worst = num = den = 0.0
    for b in range(got.shape[0]):
        nq = int(x["n_q"][b])
        assert (got[b, nq:] == 0).all() and np.isneginf(got_lse[b, nq:]).all(), f"{what}: padding rows"
        g, e = got[b, :nq].astype(np.float64), ref[b, :nq]
        assert np.isfinite(g).all(), what
        worst = max(worst, float(np.abs(g - e).max()) if nq else 0.0)
        num += float(((g - e) ** 2).sum())
        den += float((e ** 2).sum())
        np.testing.assert_allclose(got_lse[b, :nq], ref_lse[b, :nq], rtol=0, atol=LSE_ATOL)
    rel = (num / den) ** 0.5 if den else 0.0
    say(f"    {what}: max-abs {worst:.3e}, rel-L2 {rel:.3e}")
    assert worst <= BF16_ATOL and rel <= BF16_REL_L2, what


@pytest.mark.parametrize("layout", ["bhld", "blhd"])
def test_largest_soft_prompt(layout):
    cfg = wl.CONFIGS["c3_confu_8b"].with_(S=bd.SPEC_MAX_SOFT, name="c3_soft256")
    say(f"[gpu] limits: {bd.SPEC_MAX_SOFT} soft rows, {layout}")
    x = wl.generate(cfg, B=2, L=(300, 420), with_logits=False)
    assert x["sp_flag"].any() and not x["sp_flag"].all()
    for fused in (False, True):
        st = VerifyStep(cfg, x, layout=layout)
        if fused:
            st.attention_tree()
        else:
            st.build_mask()
            st.attention()
        check_against_oracle(st, x, cfg, f"S={cfg.S} {layout} {'fused' if fused else 'two calls'}")


def test_largest_key_split():
    cfg = wl.CONFIGS["c3_confu_8b"]
    say("[gpu] limits: 64 key ranges")
    x = wl.generate(cfg, B=2, L=(2100, 2400), with_logits=False)
    st = VerifyStep(cfg, x, kv_splits=64)
    assert st.ws_bytes > 0
    st.build_mask()
    st.attention()
    check_against_oracle(st, x, cfg, "kv_splits=64")


def test_longest_accepted_path_and_its_commit():
    depth = bd.SPEC_MAX_DEPTH
    cfg = wl.CONFIGS["c2_la_7b"].with_(T=depth + 4, accept_p=1.0, name="c2_chain20")
    say(f"[gpu] limits: a {cfg.T}-node chain, every draft the greedy token, max_depth {depth}")
    x = wl.generate(cfg, B=3, L=(100, 200))
    st = VerifyStep(cfg, x, max_depth=depth)
    st.accept_commit()
    torch.cuda.synchronize()
    greedy, A, path = oracle.argmax_accept(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                           x["acc_parent"], depth)
    assert (A == depth).all(), A    # the chain is longer than the cap and every draft matches
    np.testing.assert_array_equal(st.argmax.cpu().numpy(), greedy)
    np.testing.assert_array_equal(st.out_len.cpu().numpy(), A)
    np.testing.assert_array_equal(st.out_path.cpu().numpy(), path)
    kc, vc, L2 = oracle.commit_kv(x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"], x["v_blk"], A, path)
    np.testing.assert_array_equal(st.cache_len_out.cpu().numpy(), L2)
    np.testing.assert_array_equal(to_host_bits(st.k_cache), kc)
    np.testing.assert_array_equal(to_host_bits(st.v_cache), vc)
