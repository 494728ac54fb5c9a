"""spec_verify_attn_noalloc (no workspace argument, library-held scratch) against
spec_verify_attn with a caller workspace, through the C ABI: bitwise-equal
outputs and log-sum-exps on two calls in a row, the second with a smaller input,
with forced key splits so that the scratch really carries the partials.  Also
checked once against the fp64 oracle."""

import sys

import numpy as np
import pytest
import torch

import oracle
from masked_verification_attention_amd import binding as bd
from masked_verification_attention_amd import workloads as wl
from masked_verification_attention_amd.step import VerifyStep

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def both(st):
    """Outputs of the workspace entry point and of the no-alloc one on the same inputs."""
    st.build_mask()
    st.attention()
    out_ws, lse_ws = st.out.clone(), st.lse.clone()
    out_na = torch.full_like(st.out, float("nan"))
    lse_na = torch.full_like(st.lse, float("nan"))
    bd.spec_verify_attn_noalloc(st.desc, st.q, st.k_cache, st.v_cache, st.cache_len, st.k_blk, st.v_blk,
                                st.k_soft, st.v_soft, st.mask_bits, st.sp_bits, st.n_q, out_na, lse_na)
    torch.cuda.synchronize()
    return out_ws.cpu().numpy(), lse_ws.cpu().numpy(), out_na.cpu().numpy(), lse_na.cpu().numpy()


CALLS = [
    # (id, config, generate overrides, kv_splits): the second call is smaller than the first
    ("c3_b3_split4", "c3_confu_8b", {"B": 3, "L": (700, 1300)}, 4),
    ("c3_b1_split2", "c3_confu_8b", {"B": 1, "L": (90, 90)}, 2),
]


def test_noalloc_matches_workspace_entry_point_twice():
    sizes = []
    for cid, name, over, splits in CALLS:
        cfg = wl.CONFIGS[name]
        x = wl.generate(cfg, **over, with_logits=False)
        st = VerifyStep(cfg, x, kv_splits=splits)
        assert 0 < st.ws_bytes <= bd.SPEC_NOALLOC_SCRATCH_BYTES
        sizes.append(st.ws_bytes)
        say(f"[gpu] noalloc {cid}: partials {st.ws_bytes} B")
        out_ws, lse_ws, out_na, lse_na = both(st)
        np.testing.assert_array_equal(out_na.view(np.uint32), out_ws.view(np.uint32))
        np.testing.assert_array_equal(lse_na.view(np.uint32), lse_ws.view(np.uint32))
        if cid == CALLS[0][0]:
            ref, _ = oracle.verify_attention(x["q"], x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"],
                                             x["v_blk"], x["k_soft"], x["v_soft"], x["attn_parent"], x["sp_flag"],
                                             x["n_q"], cfg.dtype)
            err = float(np.abs(out_na.astype(np.float64) - ref).max())
            say(f"    max-abs vs oracle {err:.2e}")
            assert err <= 1e-2
    assert sizes[1] < sizes[0]


def test_noalloc_without_split():
    cfg = wl.CONFIGS["c3_confu_8b"]
    x = wl.generate(cfg, B=2, L=(300, 300), with_logits=False)
    st = VerifyStep(cfg, x, kv_splits=1)
    assert st.ws_bytes == 0
    out_ws, lse_ws, out_na, lse_na = both(st)
    np.testing.assert_array_equal(out_na.view(np.uint32), out_ws.view(np.uint32))
    np.testing.assert_array_equal(lse_na.view(np.uint32), lse_ws.view(np.uint32))
