"""Seeded sweep of random shapes through the whole step, against the oracle.

Each case draws a structure (tree + contemplate rows with a soft prompt,
causal chains, lookahead rows over the cache, multi-stream tree rows), GQA
group, head dimension, batch, ragged prefix range (empty prefixes included),
cache layout and split count, runs mask -> attention -> fused argmax /
acceptance / commit on the GPU, and compares every output with the oracle:
mask bits and acceptance bit-exact, attention within the bf16 bar (float32
workloads: 1e-5), committed cache bit-exact.
"""

import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from masked_verification_attention_amd import workloads as wl
from masked_verification_attention_amd.step import VerifyStep

pytestmark = pytest.mark.gpu

N_CASES = 24


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def draw_case(i):
    rng = np.random.default_rng(zlib.crc32(f"shape-{i}".encode()))
    structure = ["confu_tree", "stream_chains", "la_cache", "msa_tree"][i % 4]
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 8]))
    lo = int(rng.choice([0, 1, 17, 64, 100]))
    L = (lo, lo + int(rng.integers(0, 200)))
    kw = dict(name=f"rand{i}_{structure}", Hq=Hkv * G, Hkv=Hkv, D=D, L=L, seed=5000 + i)
    base = {"confu_tree": "c3_confu_8b", "stream_chains": "c5_stream_70b", "la_cache": "c2_la_7b",
            "msa_tree": "c6_msa_1b"}[structure]
    if structure == "confu_tree":
        kw.update(T=int(rng.integers(2, 61)), S=int(rng.choice([0, 3, 16, 33])), depth_cap=int(rng.integers(1, 8)))
    elif structure == "stream_chains":
        cl = int(rng.integers(1, 6))
        kw.update(chain_len=cl, T=cl * int(rng.integers(1, 200 // cl + 1)))
    elif structure == "la_cache":
        kw.update(T=int(rng.integers(1, 17)))
        if rng.random() < 0.3:
            kw.update(dtype="f32", logits_dtype="f32", D=64)
    else:
        gamma, branch = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        kw.update(gamma=gamma, branch=branch, T=sum(branch ** g for g in range(gamma + 1)))
    cfg = wl.CONFIGS[base].with_(**kw)
    if cfg.Tq > 256:
        cfg = cfg.with_(T=max(1, 256 // (1 + cfg.gamma)) if structure == "msa_tree" else 256)
    B = int(rng.integers(1, 4))
    layout = str(rng.choice(["blhd", "bhld", "bhld_vt"]))
    if layout == "bhld_vt" and cfg.dtype != "bf16":
        layout = "bhld"                                  # transposed V tiles are a bf16 layout
    splits = int(rng.choice([0, 0, 2, 5]))
    V = int(rng.choice([1003, 4096, 32000]))
    cfg = cfg.with_(V=V)
    fused = bool(rng.integers(0, 2)) and cfg.dtype == "bf16"
    return cfg, B, layout, splits, fused


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_step(i):
    cfg, B, layout, splits, fused = draw_case(i)
    if cfg.structure == "msa_tree" and cfg.Tq > 256:
        pytest.skip("block over 256 rows")
    say(f"[gpu] {cfg.name}: B={B} Hq/Hkv={cfg.Hq}/{cfg.Hkv} D={cfg.D} Tq={cfg.Tq} S={cfg.S} L={cfg.L} "
        f"{cfg.dtype} {layout} splits={splits} V={cfg.V} fused mask={fused}")
    x = wl.generate(cfg, B=B)
    st = VerifyStep(cfg, x, layout=layout, kv_splits=splits, fused_mask=fused)
    st.run()
    if fused:
        st.build_mask()   # the mask kernel is checked as well
    torch.cuda.synchronize()
    if cfg.structure == "msa_tree":
        bits, _, nq = oracle.build_msa_mask(x["tree_parent"], x["n_nodes"], cfg.gamma, cfg.Tq)
        np.testing.assert_array_equal(st.n_q.cpu().numpy(), nq)
        vis = np.stack([oracle.msa_block_visibility(x["tree_parent"][b], int(x["n_nodes"][b]), cfg.gamma, cfg.Tq)
                        for b in range(B)])
        ref, ref_lse = oracle.verify_attention(x["q"], x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"],
                                               x["v_blk"], None, None, None, None, x["n_q"], cfg.dtype,
                                               block_vis=vis)
        _, A, path, _, bonus = oracle.argmax_accept_rows(x["logits"], cfg.logits_dtype, x["n_nodes"],
                                                         x["draft_tok"], x["acc_parent"], x["acc_parent"],
                                                         st.max_depth)
        np.testing.assert_array_equal(st.out_bonus.cpu().numpy(), bonus)
    else:
        bits, sp = oracle.build_mask(x["attn_parent"], x["sp_flag"], x["n_q"])
        np.testing.assert_array_equal(st.sp_bits.cpu().numpy().view(np.uint32), sp)
        ref, ref_lse = oracle.verify_attention(x["q"], x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"],
                                               x["v_blk"], x["k_soft"] if cfg.S else None,
                                               x["v_soft"] if cfg.S else None, x["attn_parent"], x["sp_flag"],
                                               x["n_q"], cfg.dtype)
        _, A, path = oracle.argmax_accept(x["logits"], cfg.logits_dtype, x["n_nodes"], x["draft_tok"],
                                          x["acc_parent"], st.max_depth)
    np.testing.assert_array_equal(st.mask_bits.cpu().numpy().view(np.uint32), bits)
    out, lse = st.out.cpu().numpy(), st.lse.cpu().numpy()
    atol = 1e-2 if cfg.dtype == "bf16" else 1e-5
    worst = 0.0
    for b in range(B):
        nq = int(x["n_q"][b])
        assert (out[b, nq:] == 0).all() and np.isneginf(lse[b, nq:]).all()
        if nq:
            worst = max(worst, float(np.abs(out[b, :nq].astype(np.float64) - ref[b, :nq]).max()))
            np.testing.assert_allclose(lse[b, :nq], ref_lse[b, :nq], rtol=0, atol=2e-3)
    assert worst <= atol, worst
    np.testing.assert_array_equal(st.out_len.cpu().numpy(), A)
    np.testing.assert_array_equal(st.out_path.cpu().numpy(), path)
    kc, vc, L2 = oracle.commit_kv(x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"], x["v_blk"], A, path)
    np.testing.assert_array_equal(st.cache_len_out.cpu().numpy(), L2)
    k_host, v_host = st.cache_host()
    np.testing.assert_array_equal(k_host, kc)
    np.testing.assert_array_equal(v_host, vc)
    say(f"    max-abs {worst:.2e}, accepted {A.tolist()}")
