"""bf16 attention output (spec_attn_desc.out_dtype = SPEC_BF16) through the C ABI:
on the same inputs, every value is bitwise the float32 output of the same entry
point rounded to nearest even, and the log-sum-exps are bitwise equal, for
spec_verify_attn (one key range, forced key splits through the combine kernel,
the transposed-tile V layout, 64- and 128-row workgroups, ragged row counts with
zero padding rows, an empty prefix), spec_verify_attn_tree, spec_verify_attn_msa
and spec_verify_attn_noalloc, at small sizes and at the full 16-request size
with 4096-key prefixes.  A VerifyStep built with a bf16 output runs the whole
pass and writes the same values."""

import sys

import numpy as np
import pytest
import torch

from masked_verification_attention_amd import binding as bd
from masked_verification_attention_amd import workloads as wl
from masked_verification_attention_amd.step import VerifyStep

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_desc(desc):
    d = bd.AttnDesc.from_buffer_copy(desc)
    d.out_dtype = bd.SPEC_BF16
    return d


def call(entry, st, desc, out, lse):
    """One attention call of ``entry`` on the inputs of ``st`` into (out, lse)."""
    if entry == "attn":
        bd.spec_verify_attn(desc, st.q, st.k_cache, st.v_cache, st.cache_len, st.k_blk, st.v_blk, st.k_soft,
                            st.v_soft, st.mask_bits, st.sp_bits, st.n_q, out, lse, st.workspace, st.ws_bytes)
    elif entry == "noalloc":
        bd.spec_verify_attn_noalloc(desc, st.q, st.k_cache, st.v_cache, st.cache_len, st.k_blk, st.v_blk,
                                    st.k_soft, st.v_soft, st.mask_bits, st.sp_bits, st.n_q, out, lse)
    elif entry == "tree":
        bd.spec_verify_attn_tree(desc, st.q, st.k_cache, st.v_cache, st.cache_len, st.k_blk, st.v_blk,
                                 st.k_soft, st.v_soft, st.attn_parent, st.sp_flag, st.n_q, out, lse,
                                 st.workspace, st.ws_bytes)
    elif entry == "msa":
        bd.spec_verify_attn_msa(desc, st.q, st.k_cache, st.v_cache, st.cache_len, st.k_blk, st.v_blk,
                                st.k_soft, st.v_soft, st.tree_parent, st.n_nodes, st.tree_parent.shape[1],
                                st.cfg.gamma, out, lse, st.workspace, st.ws_bytes)
    else:
        raise ValueError(entry)


def f32_and_bf16(entry, st):
    """(fp32 out, fp32 lse, bf16 out, bf16-call lse) of one entry point, as torch CPU tensors."""
    dev = st.out.device
    if entry != "tree" and entry != "msa":
        st.build_mask()
    o32 = torch.full(tuple(st.out.shape), float("nan"), dtype=torch.float32, device=dev)
    l32 = torch.full(tuple(st.lse.shape), float("nan"), dtype=torch.float32, device=dev)
    o16 = torch.full(tuple(st.out.shape), float("nan"), dtype=torch.bfloat16, device=dev)
    l16 = torch.full(tuple(st.lse.shape), float("nan"), dtype=torch.float32, device=dev)
    d16 = bf16_desc(st.desc)
    assert bd.spec_verify_attn_workspace(d16) == st.ws_bytes
    call(entry, st, st.desc, o32, l32)
    call(entry, st, d16, o16, l16)
    torch.cuda.synchronize()
    return o32.cpu(), l32.cpu(), o16.cpu(), l16.cpu()


def assert_rounded(o32, l32, o16, l16, what):
    want = o32.to(torch.bfloat16)    # round to nearest even
    same = want.view(torch.int16) == o16.view(torch.int16)
    assert bool(same.all()), f"{what}: {int((~same).sum())} of {same.numel()} bf16 values differ"
    assert bool((l32.view(torch.int32) == l16.view(torch.int32)).all()), f"{what}: lse differs"
    assert bool(torch.isfinite(o16.float()).all()), f"{what}: a non-finite output"


CASES = [
    # (id, config, generate overrides, kv_splits, layout, entry)
    ("c3_one_range", "c3_confu_8b", {"B": 2, "L": (300, 333)}, 0, "bhld", "attn"),
    ("c3_split3_combine", "c3_confu_8b", {"B": 2, "L": (700, 900)}, 3, "bhld", "attn"),
    ("c3_vt", "c3_confu_8b", {"B": 2, "L": (300, 333)}, 0, "bhld_vt", "attn"),
    ("c3_blhd_tree", "c3_confu_8b", {"B": 2, "L": (200, 400)}, 0, "blhd", "tree"),
    ("c3_empty_prefix", "c3_confu_8b", {"B": 2, "L": (0, 0)}, 0, "bhld", "attn"),
    ("c2_ragged_nq", "c2_la_7b", {"B": 3, "L": (64, 200), "n_q": np.array([8, 5, 1])}, 0, "bhld", "attn"),
    ("c2_ragged_nq_split2", "c2_la_7b", {"B": 3, "L": (64, 200), "n_q": np.array([8, 0, 3])}, 2, "blhd", "attn"),
    ("c4_noalloc_split2", "c4_tree_3b", {"B": 2, "L": (300, 700)}, 2, "bhld", "noalloc"),
    ("c5_rows1024", "c5_stream_70b", {"B": 1, "L": (500, 500)}, 0, "bhld", "attn"),
    ("c6_msa_d64", "c6_msa_1b", {"B": 2, "L": (100, 300)}, 0, "bhld", "msa"),
    ("c6_msa_d64_split2", "c6_msa_1b", {"B": 2, "L": (600, 700)}, 2, "bhld_vt", "msa"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bf16_out_is_rounded_f32_out(case):
    cid, name, over, splits, layout, entry = case
    cfg = wl.CONFIGS[name]
    say(f"[gpu] bf16 out {cid}: {entry}, {layout}, kv_splits {splits}")
    x = wl.generate(cfg, **over, with_logits=False)
    st = VerifyStep(cfg, x, kv_splits=splits, layout=layout)
    o32, l32, o16, l16 = f32_and_bf16(entry, st)
    assert_rounded(o32, l32, o16, l16, cid)
    if entry != "msa":     # padding rows are zero (msa rows come from the node count)
        for b in range(st.B):
            nq = int(x["n_q"][b])
            assert bool((o16[b, nq:].float() == 0).all()), f"{cid}: padding rows of request {b}"   # +-0


def test_bf16_out_full_size_headline():
    cfg = wl.CONFIGS["c3_confu_8b"]
    say("[gpu] bf16 out c3 full size: attn and tree, bhld_vt")
    x = wl.generate(cfg, with_logits=False)
    st = VerifyStep(cfg, x, layout="bhld_vt")
    for entry in ("attn", "tree"):
        o32, l32, o16, l16 = f32_and_bf16(entry, st)
        assert_rounded(o32, l32, o16, l16, f"c3 full {entry}")


def test_step_with_bf16_out_runs_the_pass():
    cfg = wl.CONFIGS["c3_confu_8b"]
    say("[gpu] bf16 out: VerifyStep(out_dtype='bf16').run() against the fp32 step")
    x = wl.generate(cfg, B=2, L=(500, 600))
    s32 = VerifyStep(cfg, x, layout="bhld")
    s16 = VerifyStep(cfg, x, layout="bhld", out_dtype="bf16")
    assert s16.out.dtype == torch.bfloat16
    s32.run()
    s16.run()
    torch.cuda.synchronize()
    assert_rounded(s32.out.cpu(), s32.lse.cpu(), s16.out.cpu(), s16.lse.cpu(), "step")
    for name in ("out_len", "out_path", "cache_len_out"):
        assert torch.equal(getattr(s32, name).cpu(), getattr(s16, name).cpu()), name


def test_bf16_out_of_fp32_inputs_is_refused():
    cfg = wl.CONFIGS["c1_tiny_la"]
    x = wl.generate(cfg, with_logits=False)
    st = VerifyStep(cfg, x, out_dtype="bf16")
    st.build_mask()
    with pytest.raises(bd.SpecError) as e:
        st.attention()
    assert e.value.status == bd.SPEC_EUNSUPPORTED
