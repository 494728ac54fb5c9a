"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

Bars: bit-exact for the mask bits, the argmax, the accepted lengths and
paths, and the KV commit; attention within max-abs 1e-2 for bf16 inputs
(1e-5 for fp32) plus a relative-L2 gate, and bitwise invariance of a row's
output under changes of keys it cannot see.
"""

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
F32_ATOL = 1e-5
LSE_ATOL = 2e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_attention(x, cfg, **kw):
    return oracle.verify_attention(x["q"], x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"], x["v_blk"],
                                   x["k_soft"] if cfg.S else None, x["v_soft"] if cfg.S else None,
                                   x["attn_parent"], x["sp_flag"], x["n_q"], cfg.dtype, **kw)


def compare_attention(got, got_lse, ref, ref_lse, cfg, x, rows=None, requests=None, atol=None):
    Bn, Tq = x["q"].shape[:2]
    reqs = range(Bn) if requests is None else requests
    worst, num, den = 0.0, 0.0, 0.0
    for b in reqs:
        nq = int(x["n_q"][b])
        rr = range(Tq) if rows is None else rows
        for r in rr:
            if r >= nq:
                assert (got[b, r] == 0).all(), f"padded row {b},{r} not zero"
                assert np.isneginf(got_lse[b, r]).all()
                continue
            g, e = got[b, r].astype(np.float64), ref[b, r]
            assert np.isfinite(g).all(), f"non-finite output at {b},{r}"
            worst = max(worst, float(np.abs(g - e).max()))
            num += float(((g - e) ** 2).sum())
            den += float((e ** 2).sum())
            np.testing.assert_allclose(got_lse[b, r], ref_lse[b, r], rtol=0, atol=LSE_ATOL)
    rel = (num / den) ** 0.5 if den else 0.0
    say(f"    attention {cfg.name}: max-abs {worst:.3e}, rel-L2 {rel:.3e}")
    if cfg.dtype == "bf16":
        assert worst <= (BF16_ATOL if atol is None else atol)
        assert rel <= BF16_REL_L2
    else:
        assert worst <= F32_ATOL
    return worst, rel


SMALL_CASES = [
    # (id, config, overrides for generate, kv_splits)
    ("c1_cache", "c1_tiny_la", {}, 0),
    ("c1_full", "c1_tiny_la_full", {}, 0),
    ("c1_split3", "c1_tiny_la", {}, 3),
    ("c1_empty_prefix", "c1_tiny_la", {"L": (0, 0)}, 0),
    ("c2_small", "c2_la_7b", {"B": 2, "L": (100, 300)}, 0),
    ("c2_ragged_nq", "c2_la_7b", {"B": 3, "L": (64, 200), "n_q": np.array([8, 5, 1])}, 2),
    ("c3_small", "c3_confu_8b", {"B": 2, "L": (300, 300)}, 0),
    ("c3_split3", "c3_confu_8b", {"B": 2, "L": (333, 333)}, 3),
    ("c3_empty_prefix", "c3_confu_8b", {"B": 2, "L": (0, 0)}, 0),
    ("c4_small", "c4_tree_3b", {"B": 2, "L": (200, 333)}, 0),
    ("c5_small", "c5_stream_70b", {"B": 1, "L": (257, 257)}, 0),
    ("c5_small_split", "c5_stream_70b", {"B": 1, "L": (257, 257)}, 2),
    # long ragged prefixes (many steady-state steps), forced splits with ragged
    # prefixes, ragged block rows
    ("c3_long", "c3_confu_8b", {"B": 2, "L": (1500, 2047)}, 0),
    ("c4_split3_ragged", "c4_tree_3b", {"B": 2, "L": (500, 1500)}, 3),
    ("c3_ragged_nq", "c3_confu_8b", {"B": 3, "L": (700, 900), "n_q": np.array([60, 37, 1])}, 0),
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_mask_and_attention_small(case):
    cid, name, over, splits = case
    cfg = wl.CONFIGS[name]
    say(f"[gpu] {cid}: generate")
    x = wl.generate(cfg, **over, with_logits=False)
    st = VerifyStep(cfg, x, kv_splits=splits)
    say(f"[gpu] {cid}: build_mask + attention (ws {st.ws_bytes} B)")
    st.build_mask()
    st.attention()
    torch.cuda.synchronize()
    bits = st.mask_bits.cpu().numpy().view(np.uint32)
    sp = st.sp_bits.cpu().numpy().view(np.uint32)
    ref_bits, ref_sp = oracle.build_mask(x["attn_parent"], x["sp_flag"], x["n_q"])
    np.testing.assert_array_equal(bits, ref_bits)
    np.testing.assert_array_equal(sp, ref_sp)
    ref, ref_lse = oracle_attention(x, cfg)
    compare_attention(st.out.cpu().numpy(), st.lse.cpu().numpy(), ref, ref_lse, cfg, x)


BF16_SMALL = [c for c in SMALL_CASES if wl.CONFIGS[c[1]].dtype == "bf16"]


@pytest.mark.parametrize("case", BF16_SMALL, ids=[c[0] for c in BF16_SMALL])
def test_attention_small_transposed_v(case):
    # V in transposed 32-key tiles (SPEC_V_TILE32): ragged last tiles whose unused
    # slots hold NaN, split boundaries, empty prefixes, ragged block rows
    cid, name, over, splits = case
    cfg = wl.CONFIGS[name]
    x = wl.generate(cfg, **over, with_logits=False)
    st = VerifyStep(cfg, x, kv_splits=splits, layout="bhld_vt")
    say(f"[gpu] {cid} (transposed V): build_mask + attention (ws {st.ws_bytes} B)")
    st.build_mask()
    st.attention()
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(x, cfg)
    compare_attention(st.out.cpu().numpy(), st.lse.cpu().numpy(), ref, ref_lse, cfg, x)


def test_mid_size_block_two_group_kernel():
    # 15 nodes + 15 contemplate rows, GQA group 4: 120 rows per kv-head, the
    # largest block that still runs two wave groups of 64-row slices
    cfg = wl.CONFIGS["c3_confu_8b"].with_(T=15, name="c3_t15")
    x = wl.generate(cfg, B=2, L=(400, 613), with_logits=False)
    st = VerifyStep(cfg, x)
    st.build_mask()
    st.attention()
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(x, cfg)
    compare_attention(st.out.cpu().numpy(), st.lse.cpu().numpy(), ref, ref_lse, cfg, x)


@pytest.mark.parametrize("layout", ["blhd", "bhld_vt"])
def test_large_scores_rescale_often(layout):
    # queries scaled by 6: scores spread over tens of log2 units, so the running
    # max moves by more than the rescale threshold inside the steady-state steps
    cfg = wl.CONFIGS["c3_confu_8b"].with_(name="c3_q6")
    x = wl.generate(cfg, B=1, L=(2047, 2047), with_logits=False)
    qf = (x["q"].astype(np.uint32) << 16).view(np.float32) * np.float32(6.0)
    x["q"] = wl.f32_to_bf16_bits(qf)
    st = VerifyStep(cfg, x, layout=layout)
    st.build_mask()
    st.attention()
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(x, cfg)
    # Out of the workloads' distribution, so not their 1e-2 bar: the kernels round
    # the probabilities to bf16 (unit roundoff 2^-8) for the P*V product while
    # normalising by their fp32 sum, which bounds a row's error by 2^-8 times the
    # largest |v| it sees; peaky rows here are dominated by single V rows of
    # magnitude ~4, so that bound, not 1e-2, is the one that holds.
    vmax = max(np.abs(wl_values(x["v_cache"], cfg)).max(), np.abs(wl_values(x["v_blk"], cfg)).max(),
               np.abs(wl_values(x["v_soft"], cfg)).max())
    compare_attention(st.out.cpu().numpy(), st.lse.cpu().numpy(), ref, ref_lse, cfg, x, atol=2.0 ** -8 * vmax)


def wl_values(a, cfg):
    # stored inputs as float64 (bf16 bit patterns widened exactly), NaN canaries dropped
    v = (a.astype(np.uint32) << 16).view(np.float32) if cfg.dtype == "bf16" else a
    v = v.astype(np.float64)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("layout", ["blhd", "bhld_vt"])
def test_d64_bf16_mfma_path(layout):
    cfg = wl.CONFIGS["c3_confu_8b"].with_(D=64, name="c3_d64")
    x = wl.generate(cfg, B=2, L=(130, 161), with_logits=False)
    st = VerifyStep(cfg, x, layout=layout)
    st.build_mask()
    st.attention()
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(x, cfg)
    compare_attention(st.out.cpu().numpy(), st.lse.cpu().numpy(), ref, ref_lse, cfg, x)


@pytest.mark.parametrize("layout", ["blhd", "bhld_vt"])
def test_max_block_rows(layout):
    # Tq = 256 block rows (the limit), 64 chains of 4, GQA group 2
    cfg = wl.CONFIGS["c5_stream_70b"].with_(Hq=4, Hkv=2, T=256, chain_len=4, name="c5_tq256")
    x = wl.generate(cfg, B=1, L=(40, 40), with_logits=False)
    st = VerifyStep(cfg, x, layout=layout)
    st.build_mask()
    st.attention()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.mask_bits.cpu().numpy().view(np.uint32),
                                  oracle.build_mask(x["attn_parent"], x["sp_flag"], x["n_q"])[0])
    ref, ref_lse = oracle_attention(x, cfg)
    compare_attention(st.out.cpu().numpy(), st.lse.cpu().numpy(), ref, ref_lse, cfg, x)


def test_single_row_block():
    cfg = wl.CONFIGS["c2_la_7b"].with_(T=1, Hq=4, Hkv=4, name="c2_tq1")
    x = wl.generate(cfg, B=2, L=(50, 77), with_logits=False)
    st = VerifyStep(cfg, x)
    st.build_mask()
    st.attention()
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(x, cfg)
    compare_attention(st.out.cpu().numpy(), st.lse.cpu().numpy(), ref, ref_lse, cfg, x)


@pytest.mark.parametrize("layout", ["blhd", "bhld_vt"])
def test_invisible_keys_do_not_change_outputs_bitwise(layout):
    cfg = wl.CONFIGS["c3_confu_8b"]
    x = wl.generate(cfg, B=2, L=(200, 200), with_logits=False)
    st = VerifyStep(cfg, x, layout=layout)
    st.build_mask()
    st.attention()
    base = st.out.clone()
    T = cfg.T
    # node rows never see the soft prompt or the contemplate rows' K/V
    g = torch.Generator(device="cuda").manual_seed(5)
    st.k_blk[:, T:] = torch.randn(st.k_blk[:, T:].shape, generator=g, device="cuda").to(torch.bfloat16)
    st.v_blk[:, T:] = torch.randn(st.v_blk[:, T:].shape, generator=g, device="cuda").to(torch.bfloat16)
    st.k_soft.copy_(torch.randn(st.k_soft.shape, generator=g, device="cuda").to(torch.bfloat16))
    st.v_soft.copy_(torch.randn(st.v_soft.shape, generator=g, device="cuda").to(torch.bfloat16))
    # cache slots past the prefix: garbage of another kind (infinities in the V tile
    # that holds the prefix's last keys when V is tiled)
    if layout == "blhd":
        st.k_cache[:, 200:] = 1e4
        st.v_cache[:, 200:] = float("inf")
    else:
        from masked_verification_attention_amd.step import VT_POS_OF
        st.k_cache[:, :, 200:] = 1e4
        for k in range(200 % 32, 32):                     # tile [D/16][group][16][slot]
            g, e = divmod(VT_POS_OF[k], 8)
            st.v_cache[:, :, 200 // 32, :, g, :, e] = float("inf")
        st.v_cache[:, :, 200 // 32 + 1:] = 1e4
    st.attention()
    torch.cuda.synchronize()
    assert torch.equal(st.out[:, :T], base[:, :T])
    assert not torch.equal(st.out[:, T:], base[:, T:])


@pytest.mark.parametrize("layout", ["blhd", "bhld_vt"])
@pytest.mark.parametrize("name", ["c3_confu_8b", "c4_tree_3b"])
def test_truncated_block_leaves_earlier_rows_bitwise(name, layout):
    """Parents precede children, so cutting a request's block after row n' leaves
    what rows < n' see unchanged; their outputs must not move by a single bit
    although the rows sharing their waves and the block's tile count change."""
    cfg = wl.CONFIGS[name]
    x = wl.generate(cfg, B=3, L=(300, 500), with_logits=False)
    st = VerifyStep(cfg, x, layout=layout)
    st.build_mask()
    st.attention()
    torch.cuda.synchronize()
    base = st.out.clone()
    base_lse = st.lse.clone()
    full = x["n_q"].copy()
    cut = np.array([max(1, int(full[0]) // 2), 1, max(1, int(full[2]) - 33)], dtype=np.int32)
    say(f"{name}: n_q {full.tolist()} -> {cut.tolist()}")
    st.n_q.copy_(torch.from_numpy(cut))
    st.build_mask()
    st.attention()
    torch.cuda.synchronize()
    for b in range(3):
        n = int(cut[b])
        assert torch.equal(st.out[b, :n], base[b, :n]), (b, n)
        assert torch.equal(st.lse[b, :n], base_lse[b, :n]), (b, n)


@pytest.mark.parametrize("name", ["c1_tiny_la", "c2_la_7b", "c3_confu_8b", "c4_tree_3b", "c5_stream_70b"])
def test_argmax_accept_and_commit_small(name):
    cfg = wl.CONFIGS[name]
    say(f"[gpu] accept {name}")
    x = wl.generate(cfg, B=min(cfg.B, 4), L=(64, 96) if cfg.L[0] else None)
    st = VerifyStep(cfg, x)
    st.argmax_accept()
    st.commit()
    torch.cuda.synchronize()
    greedy, A, path = oracle.argmax_accept(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                           x["acc_parent"], st.max_depth)
    np.testing.assert_array_equal(st.argmax.cpu().numpy(), greedy)
    np.testing.assert_array_equal(st.out_len.cpu().numpy(), A)
    np.testing.assert_array_equal(st.out_path.cpu().numpy(), path)
    kc, vc, L2 = oracle.commit_kv(x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"], x["v_blk"], A, path)
    np.testing.assert_array_equal(st.cache_len_out.cpu().numpy(), L2)
    np.testing.assert_array_equal(to_host_bits(st.k_cache), kc)
    np.testing.assert_array_equal(to_host_bits(st.v_cache), vc)
    say(f"    accepted lengths {list(A)}")


def test_argmax_ties_and_signed_zero():
    # rows built so that the maximum repeats, including -0 / +0 ties and misaligned row starts
    rng = np.random.Generator(np.random.PCG64(9))
    B, T, V = 2, 6, 1003
    rows = rng.standard_normal((B, T, V)).astype(np.float32)
    rows[0, 0, [5, 17, 900]] = 9.0
    rows[0, 1, :] = -1.0
    rows[0, 1, [0, 1002]] = 0.0
    rows[0, 1, 3] = -0.0
    rows[0, 2, :] = 3.5
    rows[1, 0, [1001, 1002]] = 7.0
    rows[1, 1, :] = -0.0
    rows[1, 1, 600] = 0.0
    rows[1, 2, [2, 3]] = 6.0
    for dtype in ("f32", "bf16"):
        data = rows if dtype == "f32" else wl.f32_to_bf16_bits(rows)
        lg = torch.from_numpy(data.view(np.int16)).view(torch.bfloat16).cuda() if dtype == "bf16" \
            else torch.from_numpy(data).cuda()
        out = torch.empty(B, T, dtype=torch.int32, device="cuda")
        ln = torch.empty(B, dtype=torch.int32, device="cuda")
        pth = torch.empty(B, 4, dtype=torch.int32, device="cuda")
        nn = torch.tensor([T, T - 1], dtype=torch.int32, device="cuda")
        dr = torch.zeros(B, T, dtype=torch.int32, device="cuda")
        par = torch.tensor([[-1, 0, 1, 2, 3, 4]] * B, dtype=torch.int32, device="cuda")
        bd.spec_argmax_accept(lg, bd.SPEC_F32 if dtype == "f32" else bd.SPEC_BF16, B, T, V, nn, dr, par, 4,
                              out, ln, pth)
        torch.cuda.synchronize()
        ref = oracle.greedy_tokens(data, dtype)
        ref[1, T - 1] = -1
        np.testing.assert_array_equal(out.cpu().numpy(), ref)
        assert out[0, 0].item() == 5 and out[0, 1].item() == 0 and out[0, 2].item() == 0
        assert out[1, 1].item() == 0


def test_commit_in_place_alias():
    cfg = wl.CONFIGS["c3_confu_8b"]
    x = wl.generate(cfg, B=3, L=(50, 50))
    st = VerifyStep(cfg, x)
    st.argmax_accept()
    st.commit(in_place=True)
    torch.cuda.synchronize()
    _, A, path = oracle.argmax_accept(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                      x["acc_parent"], st.max_depth)
    _, _, L2 = oracle.commit_kv(x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"], x["v_blk"], A, path)
    np.testing.assert_array_equal(st.cache_len.cpu().numpy(), L2)


def test_commit_respects_capacity():
    cfg = wl.CONFIGS["c5_stream_70b"].with_(Hq=8, Hkv=2)
    x = wl.generate(cfg, B=2, L=(30, 30))
    st = VerifyStep(cfg, x)
    # every draft matches: accepted length = chain length 4; room for only 2 rows in request 1
    st.draft_tok.copy_(torch.from_numpy(oracle.greedy_tokens(x["logits"], cfg.logits_dtype)).cuda())
    lmax = st.lmax
    st.cache_len.copy_(torch.tensor([10, lmax - 2], dtype=torch.int32))
    st.argmax_accept()
    st.commit()
    torch.cuda.synchronize()
    assert list(st.out_len.cpu().numpy()) == [4, 4]
    assert list(st.cache_len_out.cpu().numpy()) == [14, lmax]
    path = st.out_path.cpu().numpy()
    kc, vc, L2 = oracle.commit_kv(x["k_cache"], x["v_cache"], np.array([10, lmax - 2], np.int32),
                                  x["k_blk"], x["v_blk"], np.array([4, 4], np.int32), path)
    np.testing.assert_array_equal(to_host_bits(st.k_cache), kc)
    np.testing.assert_array_equal(to_host_bits(st.v_cache), vc)


def test_full_step_chain_matches_oracle():
    cfg = wl.CONFIGS["c3_confu_8b"]
    x = wl.generate(cfg, B=3, L=(150, 150))
    st = VerifyStep(cfg, x)
    st.run()
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(x, cfg)
    compare_attention(st.out.cpu().numpy(), st.lse.cpu().numpy(), ref, ref_lse, cfg, x)
    greedy, A, path = oracle.argmax_accept(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                           x["acc_parent"], st.max_depth)
    np.testing.assert_array_equal(st.out_len.cpu().numpy(), A)
    np.testing.assert_array_equal(st.out_path.cpu().numpy(), path)


HEAD_MAJOR = [(n, "bhld") for n in ["c1_tiny_la", "c2_la_7b", "c3_confu_8b", "c4_tree_3b", "c5_stream_70b"]] + \
    [(n, "bhld_vt") for n in ["c2_la_7b", "c3_confu_8b", "c4_tree_3b", "c5_stream_70b"]]


@pytest.mark.parametrize("name,layout", HEAD_MAJOR, ids=[f"{n}-{l}" for n, l in HEAD_MAJOR])
def test_head_major_cache_layout(name, layout):
    # the cache may be [B, Hkv, lmax, D] (head-major) through the descriptor's strides, with V
    # row-major or in transposed 32-key tiles; the whole step, commit included
    cfg = wl.CONFIGS[name]
    x = wl.generate(cfg, B=min(cfg.B, 2), L=(70, 140) if cfg.L[0] else None)
    st = VerifyStep(cfg, x, layout=layout)
    st.run()
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(x, cfg)
    compare_attention(st.out.cpu().numpy(), st.lse.cpu().numpy(), ref, ref_lse, cfg, x)
    _, A, path = oracle.argmax_accept(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                      x["acc_parent"], st.max_depth)
    kc, vc, L2 = oracle.commit_kv(x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"], x["v_blk"], A, path)
    np.testing.assert_array_equal(st.cache_len_out.cpu().numpy(), L2)
    k_host, v_host = st.cache_host()
    np.testing.assert_array_equal(k_host, kc)
    np.testing.assert_array_equal(v_host, vc)


FULL_SAMPLES = {
    # name: (requests, rows) sampled for the oracle; rows include first/last and contemplate rows
    "c2_la_7b": ([0, 3, 7], [0, 3, 7]),
    "c3_confu_8b": ([0, 7, 15], [0, 1, 17, 29, 30, 45, 59]),
    "c4_tree_3b": ([0, 19, 31], [0, 31, 59, 60, 90, 119]),
    "c5_stream_70b": ([0, 15], [0, 3, 64, 127]),
}


FULL_CASES = [(n, "bhld_vt") for n in sorted(FULL_SAMPLES)] + [("c3_confu_8b", "bhld")]


@pytest.mark.parametrize("name,layout", FULL_CASES, ids=[f"{n}-{l}" for n, l in FULL_CASES])
def test_full_size_sampled(name, layout):
    """Whole workload at its full size in the benchmark's launch configuration
    (automatic split, head-major cache, V in transposed 32-key tiles; row-major V
    too for the headline workload); attention checked on sampled rows, the
    argmax / acceptance / commit checked everywhere."""
    cfg = wl.CONFIGS[name]
    reqs, rows = FULL_SAMPLES[name]
    say(f"[gpu] full-size {name} {layout}: generate")
    x = wl.generate(cfg)
    st = VerifyStep(cfg, x, layout=layout)
    say(f"[gpu] full-size {name}: run step (ws {st.ws_bytes} B)")
    st.run()
    if st.fused_mask:   # run() built the mask inside the attention launch; check the mask kernel too
        st.build_mask()
    torch.cuda.synchronize()
    bits, sp = oracle.build_mask(x["attn_parent"], x["sp_flag"], x["n_q"])
    np.testing.assert_array_equal(st.mask_bits.cpu().numpy().view(np.uint32), bits)
    np.testing.assert_array_equal(st.sp_bits.cpu().numpy().view(np.uint32), sp)
    say(f"[gpu] full-size {name}: oracle on sampled rows")
    ref, ref_lse = oracle_attention(x, cfg, requests=reqs, rows=rows)
    compare_attention(st.out.cpu().numpy(), st.lse.cpu().numpy(), ref, ref_lse, cfg, x, rows=rows, requests=reqs)
    out = st.out.cpu().numpy()
    assert np.isfinite(out).all()
    say(f"[gpu] full-size {name}: acceptance and commit")
    greedy, A, path = oracle.argmax_accept(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                           x["acc_parent"], st.max_depth)
    np.testing.assert_array_equal(st.argmax.cpu().numpy(), greedy)
    np.testing.assert_array_equal(st.out_len.cpu().numpy(), A)
    np.testing.assert_array_equal(st.out_path.cpu().numpy(), path)
    L = x["cache_len"]
    np.testing.assert_array_equal(st.cache_len_out.cpu().numpy(), L + A)
    k_host, v_host = st.cache_host()
    for b in range(cfg.B):
        for d in range(int(A[b])):
            np.testing.assert_array_equal(k_host[b, L[b] + d], x["k_blk"][b, path[b, d]])
            np.testing.assert_array_equal(v_host[b, L[b] + d], x["v_blk"][b, path[b, d]])
        np.testing.assert_array_equal(k_host[b, :L[b]], x["k_cache"][b, :L[b]])
    say(f"    accepted lengths {A.tolist()}")


@pytest.mark.parametrize("name", ["c1_tiny_la", "c2_la_7b", "c3_confu_8b", "c4_tree_3b", "c5_stream_70b",
                                  "c6_msa_1b"])
def test_fused_accept_commit_matches_oracle(name):
    # spec_argmax_accept_commit: the same results as acceptance then commit, in two launches
    cfg = wl.CONFIGS[name]
    say(f"[gpu] fused accept+commit {name}")
    x = wl.generate(cfg, B=min(cfg.B, 3), L=(40, 90) if cfg.L[0] else None)
    st = VerifyStep(cfg, x)
    # request 0 has room for one row only: the capacity rule applies in the fused form too
    st.cache_len.copy_(torch.tensor([st.lmax - 1] + [int(v) for v in x["cache_len"][1:]], dtype=torch.int32))
    st.accept_commit()
    torch.cuda.synchronize()
    L0 = np.array([st.lmax - 1] + list(x["cache_len"][1:]), dtype=np.int32)
    if cfg.structure == "msa_tree":
        B, T = x["acc_parent"].shape
        vrow = x["acc_parent"].copy()             # nodes first: a parent's node index is its main row
        _, A, path, _, bonus = oracle.argmax_accept_rows(x["logits"], cfg.logits_dtype, x["n_nodes"],
                                                         x["draft_tok"], x["acc_parent"], vrow, st.max_depth)
        np.testing.assert_array_equal(st.out_bonus.cpu().numpy(), bonus)
    else:
        _, A, path = oracle.argmax_accept(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                          x["acc_parent"], st.max_depth)
    np.testing.assert_array_equal(st.out_len.cpu().numpy(), A)
    np.testing.assert_array_equal(st.out_path.cpu().numpy(), path)
    greedy = np.argmax(oracle.as_f64(x["logits"], cfg.logits_dtype), axis=-1)
    got = st.argmax.cpu().numpy()
    for b in range(x["logits"].shape[0]):
        n = int(x["n_nodes"][b])
        np.testing.assert_array_equal(got[b, :n], greedy[b, :n])
        assert (got[b, n:] == -1).all()
    kc, vc, L2 = oracle.commit_kv(x["k_cache"], x["v_cache"], L0, x["k_blk"], x["v_blk"], A, path)
    np.testing.assert_array_equal(st.cache_len_out.cpu().numpy(), L2)
    k_host, v_host = st.cache_host()
    np.testing.assert_array_equal(k_host, kc)
    np.testing.assert_array_equal(v_host, vc)
    say(f"    accepted {A.tolist()}, new lengths {L2.tolist()}")


def _padded_cache(a, lmax):
    """A generator cache [B, lmax0, Hkv, D] widened to lmax slots of NaN canaries."""
    pad = lmax - a.shape[1]
    if pad == 0:
        return a
    fill = np.full((a.shape[0], pad) + a.shape[2:], 0x7FC0 if a.dtype == np.uint16 else np.nan, dtype=a.dtype)
    return np.concatenate([a, fill], axis=1)


@pytest.mark.parametrize("name", ["c2_la_7b", "c3_confu_8b", "c4_tree_3b", "c5_stream_70b", "c6_msa_1b"])
def test_fused_accept_commit_transposed_v(name):
    # the fused commit writes accepted V rows into transposed 32-key tiles, capacity rule included
    cfg = wl.CONFIGS[name]
    say(f"[gpu] fused accept+commit {name}, transposed V")
    x = wl.generate(cfg, B=min(cfg.B, 3), L=(40, 90))
    st = VerifyStep(cfg, x, layout="bhld_vt")
    L0 = np.array([st.lmax - 1] + [int(v) for v in x["cache_len"][1:]], dtype=np.int32)
    st.cache_len.copy_(torch.from_numpy(L0))
    st.accept_commit()
    torch.cuda.synchronize()
    if cfg.structure == "msa_tree":
        _, A, path, _, _ = oracle.argmax_accept_rows(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                                     x["acc_parent"], x["acc_parent"], st.max_depth)
    else:
        _, A, path = oracle.argmax_accept(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                          x["acc_parent"], st.max_depth)
    np.testing.assert_array_equal(st.out_len.cpu().numpy(), A)
    kc, vc, L2 = oracle.commit_kv(_padded_cache(x["k_cache"], st.lmax), _padded_cache(x["v_cache"], st.lmax), L0,
                                  x["k_blk"], x["v_blk"], A, path)
    np.testing.assert_array_equal(st.cache_len_out.cpu().numpy(), L2)
    k_host, v_host = st.cache_host(full=True)
    np.testing.assert_array_equal(k_host, kc)
    np.testing.assert_array_equal(v_host, vc)
    say(f"    accepted {A.tolist()}, new lengths {L2.tolist()}")
