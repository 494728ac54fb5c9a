"""spec_verify_attn_tree (block mask built inside the attention launch from the
parent array) through the C ABI: bitwise equal to spec_build_mask followed by
spec_verify_attn on the same inputs, across workloads, cache layouts, forced key
splits, ragged row counts, soft-prompt flags and parent arrays up to a 256-row
chain; within the attention bars of the fp64 oracle for valid parent arrays; and
equal to the two-call path also on parent arrays with links that break the
precondition (where both kernels end a chain at its first such link)."""

import sys

import numpy as np
import pytest
import torch

import oracle
from masked_verification_attention_amd import binding as bd
from masked_verification_attention_amd import workloads as wl
from masked_verification_attention_amd.step import VerifyStep

pytestmark = pytest.mark.gpu

BF16_ATOL = 1e-2
BF16_REL_L2 = 5e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def fused_and_two_calls(st):
    """(out, lse) of the fused entry point and of the two calls, as host arrays."""
    st.out.fill_(float("nan"))
    st.lse.fill_(float("nan"))
    st.attention_tree()
    torch.cuda.synchronize()
    fo, fl = st.out.cpu().numpy().copy(), st.lse.cpu().numpy().copy()
    st.out.fill_(float("nan"))
    st.lse.fill_(float("nan"))
    st.build_mask()
    st.attention()
    torch.cuda.synchronize()
    return fo, fl, st.out.cpu().numpy(), st.lse.cpu().numpy()


def assert_bitwise(a, b, what):
    assert a.shape == b.shape
    same = (a.view(np.uint32) == b.view(np.uint32))
    assert same.all(), f"{what}: {int((~same).sum())} of {same.size} values differ"


def check_oracle(out, lse, x, cfg):
    ref, ref_lse = oracle.verify_attention(x["q"], x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"],
                                           x["v_blk"], x["k_soft"] if cfg.S else None,
                                           x["v_soft"] if cfg.S else None, x["attn_parent"], x["sp_flag"],
                                           x["n_q"], cfg.dtype)
    num = den = worst = 0.0
    for b in range(out.shape[0]):
        nq = int(x["n_q"][b])
        assert (out[b, nq:] == 0).all() and np.isneginf(lse[b, nq:]).all(), "padding rows"
        g, e = out[b, :nq].astype(np.float64), ref[b, :nq]
        assert np.isfinite(g).all()
        worst = max(worst, float(np.abs(g - e).max()) if nq else 0.0)
        num += float(((g - e) ** 2).sum())
        den += float((e ** 2).sum())
        np.testing.assert_allclose(lse[b, :nq], ref_lse[b, :nq], rtol=0, atol=2e-3)
    rel = (num / den) ** 0.5 if den else 0.0
    say(f"    vs oracle: max-abs {worst:.3e}, rel-L2 {rel:.3e}")
    assert worst <= BF16_ATOL and rel <= BF16_REL_L2


CASES = [
    # (id, config, generate overrides, kv_splits, layout)
    ("c2_small", "c2_la_7b", {"B": 2, "L": (100, 300)}, 0, "blhd"),
    ("c2_ragged_nq_split2", "c2_la_7b", {"B": 3, "L": (64, 200), "n_q": np.array([8, 5, 1])}, 2, "bhld"),
    ("c3_small", "c3_confu_8b", {"B": 2, "L": (300, 300)}, 0, "bhld"),
    ("c3_small_vt", "c3_confu_8b", {"B": 2, "L": (300, 333)}, 0, "bhld_vt"),
    ("c3_split3", "c3_confu_8b", {"B": 2, "L": (333, 333)}, 3, "bhld"),
    ("c3_empty_prefix", "c3_confu_8b", {"B": 2, "L": (0, 0)}, 0, "blhd"),
    ("c4_small", "c4_tree_3b", {"B": 2, "L": (200, 333)}, 0, "bhld"),
    ("c5_small", "c5_stream_70b", {"B": 1, "L": (257, 257)}, 0, "bhld"),
    ("c5_small_split", "c5_stream_70b", {"B": 1, "L": (257, 257)}, 2, "bhld_vt"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_tree_equals_two_calls(case):
    cid, name, over, splits, layout = case
    cfg = wl.CONFIGS[name]
    say(f"[gpu] attn_tree {cid}: {name} {over} splits={splits} {layout}")
    x = wl.generate(cfg, with_logits=False, **over)
    st = VerifyStep(cfg, x, kv_splits=splits, layout=layout)
    fo, fl, to, tl = fused_and_two_calls(st)
    assert_bitwise(fo, to, "out")
    assert_bitwise(fl, tl, "lse")
    check_oracle(fo, fl, x, cfg)


def random_parents(rng, Tq, broken=0.0):
    """A random forest over the block rows (parent[r] = -1 or an earlier row); with
    ``broken`` > 0 that fraction of links point at r or below -1 or past r."""
    par = np.full(Tq, -1, dtype=np.int32)
    for r in range(1, Tq):
        if rng.random() < 0.8:
            par[r] = rng.integers(max(0, r - 8), r) if rng.random() < 0.7 else rng.integers(0, r)
    if broken:
        for r in range(Tq):
            if rng.random() < broken:
                par[r] = int(rng.choice([r, r + 1 + rng.integers(0, 4), -2 - rng.integers(0, 3)]))
    return par


SHAPES = [
    # (id, config, overrides, Tq shape source)
    ("c3_tq60", "c3_confu_8b", {"B": 3, "L": (40, 200)}),
    ("c4_tq120", "c4_tree_3b", {"B": 2, "L": (100, 150)}),
    ("c5_tq128", "c5_stream_70b", {"B": 2, "L": (64, 96)}),
    ("tq256", "c5_tq256", {"B": 2, "L": (40, 70)}),
]


def shape_cfg(name):
    if name == "c5_tq256":
        return wl.CONFIGS["c5_stream_70b"].with_(Hq=4, Hkv=2, T=256, chain_len=4, name="c5_tq256")
    return wl.CONFIGS[name]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_tree_random_parent_arrays(shape, seed):
    sid, name, over = shape
    cfg = shape_cfg(name)
    rng = np.random.default_rng(1000 + 17 * seed + len(sid))
    x = wl.generate(cfg, with_logits=False, seed=cfg.seed + 31 * seed, **over)
    B, Tq = x["attn_parent"].shape
    for b in range(B):
        x["attn_parent"][b] = random_parents(rng, Tq)
    x["n_q"] = rng.integers(0, Tq + 1, size=B).astype(np.int32)
    x["n_q"][0] = Tq
    x["sp_flag"] = (rng.random((B, Tq)) < 0.4).astype(np.uint8)
    say(f"[gpu] attn_tree random parents {sid} seed {seed}: Tq={Tq} n_q={x['n_q'].tolist()} S={cfg.S}")
    st = VerifyStep(cfg, x, layout="bhld")
    fo, fl, to, tl = fused_and_two_calls(st)
    assert_bitwise(fo, to, "out")
    assert_bitwise(fl, tl, "lse")
    check_oracle(fo, fl, x, cfg)


def test_tree_deep_chain_and_no_flags():
    # a 256-row chain (every row sees all earlier rows: 8 rounds of pointer jumping), soft
    # prompt present but sp_flag NULL (no row sees it)
    cfg = shape_cfg("c5_tq256").with_(S=16)
    x = wl.generate(cfg, B=1, L=(33, 33), with_logits=False)
    x["attn_parent"][0] = np.arange(-1, 255, dtype=np.int32)
    x["sp_flag"][:] = 0
    st = VerifyStep(cfg, x, layout="bhld")
    st.sp_flag = None
    fo, fl, to, tl = fused_and_two_calls(st)
    assert_bitwise(fo, to, "out")
    assert_bitwise(fl, tl, "lse")
    check_oracle(fo, fl, x, cfg)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_broken_links_match_two_calls(seed):
    # links that break -1 <= parent[r] < r end a chain in both kernels; the oracle
    # rejects such arrays (its precondition), so only the two paths are compared
    cfg = wl.CONFIGS["c4_tree_3b"]
    rng = np.random.default_rng(77 + seed)
    x = wl.generate(cfg, B=2, L=(50, 90), with_logits=False, seed=cfg.seed + seed)
    Tq = x["attn_parent"].shape[1]
    for b in range(2):
        x["attn_parent"][b] = random_parents(rng, Tq, broken=0.15)
    st = VerifyStep(cfg, x, layout="bhld")
    fo, fl, to, tl = fused_and_two_calls(st)
    assert_bitwise(fo, to, "out")
    assert_bitwise(fl, tl, "lse")


def test_tree_full_size_headline():
    # the headline workload at full size in the benchmark's configuration
    cfg = wl.CONFIGS["c3_confu_8b"]
    say("[gpu] attn_tree full-size c3: generate")
    x = wl.generate(cfg, with_logits=False)
    st = VerifyStep(cfg, x, layout="bhld")
    say("[gpu] attn_tree full-size c3: fused and two-call runs")
    fo, fl, to, tl = fused_and_two_calls(st)
    assert_bitwise(fo, to, "out")
    assert_bitwise(fl, tl, "lse")


def test_tree_rejects_fp32_inputs():
    cfg = wl.CONFIGS["c1_tiny_la"]
    x = wl.generate(cfg, with_logits=False)
    st = VerifyStep(cfg, x, fused_mask=False)
    with pytest.raises(bd.SpecError) as e:
        st.attention_tree()
    assert e.value.status == bd.SPEC_EUNSUPPORTED


# ---- multi-stream rows: spec_verify_attn_msa against spec_build_msa_mask + spec_verify_attn

def msa_oracle_check(out, lse, x, cfg):
    vis = np.stack([oracle.msa_block_visibility(x["tree_parent"][b], int(x["n_nodes"][b]), cfg.gamma, cfg.Tq)
                    for b in range(out.shape[0])])
    ref, ref_lse = oracle.verify_attention(x["q"], x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"],
                                           x["v_blk"], None, None, None, None, x["n_q"], cfg.dtype, block_vis=vis)
    num = den = worst = 0.0
    for b in range(out.shape[0]):
        nq = int(x["n_q"][b])
        assert (out[b, nq:] == 0).all() and np.isneginf(lse[b, nq:]).all(), "padding rows"
        g, e = out[b, :nq].astype(np.float64), ref[b, :nq]
        assert np.isfinite(g).all()
        worst = max(worst, float(np.abs(g - e).max()) if nq else 0.0)
        num += float(((g - e) ** 2).sum())
        den += float((e ** 2).sum())
        np.testing.assert_allclose(lse[b, :nq], ref_lse[b, :nq], rtol=0, atol=2e-3)
    rel = (num / den) ** 0.5 if den else 0.0
    say(f"    vs oracle: max-abs {worst:.3e}, rel-L2 {rel:.3e}")
    assert worst <= BF16_ATOL and rel <= BF16_REL_L2


MSA_CASES = [
    # (id, config overrides, generate overrides, kv_splits, layout)
    ("c6_small", {}, {"B": 2, "L": (100, 300)}, 0, "bhld"),
    ("c6_pruned_split2", {}, {"B": 3, "L": (64, 200), "n_nodes": np.array([40, 13, 0])}, 2, "bhld"),
    ("c6_g4k2_vt", {"gamma": 4, "branch": 2, "T": 31}, {"B": 2, "L": (150, 260)}, 0, "bhld_vt"),
    ("c6_d128_gqa", {"Hq": 32, "Hkv": 8, "D": 128}, {"B": 2, "L": (200, 333)}, 0, "bhld"),
    ("c6_empty_prefix", {}, {"B": 2, "L": (0, 0)}, 0, "blhd"),
]


@pytest.mark.parametrize("case", MSA_CASES, ids=[c[0] for c in MSA_CASES])
def test_msa_fused_equals_two_calls(case):
    cid, cov, gov, splits, layout = case
    cfg = wl.CONFIGS["c6_msa_1b"].with_(name=cid, **cov)
    say(f"[gpu] attn_msa {cid}: {cov} {gov} splits={splits} {layout}")
    x = wl.generate(cfg, with_logits=False, **gov)
    st = VerifyStep(cfg, x, kv_splits=splits, layout=layout)
    fo, fl, to, tl = fused_and_two_calls(st)
    assert_bitwise(fo, to, "out")
    assert_bitwise(fl, tl, "lse")
    msa_oracle_check(fo, fl, x, cfg)


@pytest.mark.parametrize("gamma,branch", [(1, 100), (2, 6), (3, 3), (0, 1)])
def test_msa_fused_random_trees(gamma, branch):
    # random trees over the generator's node count (any earlier node as parent: deep
    # chains too) and ragged node counts
    T = sum(branch ** g for g in range(gamma + 1))
    cfg = wl.CONFIGS["c6_msa_1b"].with_(name=f"msa_g{gamma}_k{branch}", gamma=gamma, branch=branch, T=T)
    rng = np.random.default_rng(500 + 7 * gamma + branch)
    x = wl.generate(cfg, B=3, L=(30, 120), with_logits=False)
    N = x["tree_parent"].shape[1]
    for b in range(3):
        par = np.full(N, -1, dtype=np.int32)
        for v in range(1, N):
            par[v] = int(rng.integers(max(0, v - 3), v)) if rng.random() < 0.6 else int(rng.integers(0, v))
        x["tree_parent"][b] = par
    x["n_nodes"] = np.array([N, int(rng.integers(1, N + 1)), int(rng.integers(0, min(N, 4) + 1))], dtype=np.int32)
    x["n_q"] = (x["n_nodes"] * (1 + gamma)).astype(np.int32)
    say(f"[gpu] attn_msa random trees gamma={gamma}: N={N} Tq={cfg.Tq} n_nodes={x['n_nodes'].tolist()}")
    st = VerifyStep(cfg, x, layout="bhld")
    fo, fl, to, tl = fused_and_two_calls(st)
    assert_bitwise(fo, to, "out")
    assert_bitwise(fl, tl, "lse")
    msa_oracle_check(fo, fl, x, cfg)


def test_msa_fused_full_size():
    cfg = wl.CONFIGS["c6_msa_1b"]
    x = wl.generate(cfg, with_logits=False)
    st = VerifyStep(cfg, x, layout="bhld")
    fo, fl, to, tl = fused_and_two_calls(st)
    assert_bitwise(fo, to, "out")
    assert_bitwise(fl, tl, "lse")


@pytest.mark.parametrize("layout", ["bhld", "bhld_vt"])
def test_hidden_nonfinite_keys_never_reach_a_row(layout):
    """A key a row cannot see never reaches its output, whatever its K holds:
    NaN and infinities in the contemplate rows' and the soft prompt's K (with
    new finite V) leave the tree-node rows bitwise unchanged, and NaN in one
    leaf node's K leaves every row that does not see that node bitwise unchanged
    (rows that see it turn NaN, as the definition gives).  A hidden key's V must
    be finite: the P*V product multiplies it by a zero probability."""
    cfg = wl.CONFIGS["c3_confu_8b"]
    x = wl.generate(cfg, B=2, L=(200, 231), with_logits=False)
    T = cfg.T

    def run(st):
        st.attention_tree()
        torch.cuda.synchronize()
        return st.out.cpu().numpy().copy(), st.lse.cpu().numpy().copy()

    st = VerifyStep(cfg, x, layout=layout)
    base, base_lse = run(st)
    g = torch.Generator(device="cuda").manual_seed(11)
    st.k_blk[:, T:] = float("nan")
    st.v_blk[:, T:] = torch.randn(st.v_blk[:, T:].shape, generator=g, device="cuda").to(torch.bfloat16)
    st.k_soft.fill_(float("inf"))
    st.v_soft.copy_(torch.randn(st.v_soft.shape, generator=g, device="cuda").to(torch.bfloat16))
    out, lse = run(st)
    say(f"    {layout}: node rows finite after non-finite hidden K: {np.isfinite(out[:, :T]).all()}")
    assert_bitwise(out[:, :T], base[:, :T], "node rows' outputs")
    assert_bitwise(lse[:, :T], base_lse[:, :T], "node rows' lse")

    par = x["attn_parent"][0]
    nq = int(x["n_q"][0])
    Tq = par.shape[0]
    parents = {int(p) for p in par[:min(nq, T)]}                # links among the tree nodes
    j = max(r for r in range(1, min(nq, T)) if r not in parents)   # a leaf of the node tree
    M = oracle.block_visibility(par, nq, Tq)
    sees = M[:, j]
    st = VerifyStep(cfg, x, layout=layout)
    st.k_blk[0, j] = float("nan")
    out, lse = run(st)
    say(f"    {layout}: leaf {j} seen by rows {np.flatnonzero(sees).tolist()}")
    assert sees[j] and sees.sum() < nq
    assert_bitwise(out[0, ~sees], base[0, ~sees], "rows that do not see the leaf")
    assert_bitwise(lse[0, ~sees], base_lse[0, ~sees], "lse of rows that do not see the leaf")
    assert np.isnan(out[0, sees]).all()
    assert_bitwise(out[1], base[1], "the other request")


def test_longest_first_dealing_covers_every_row():
    """A grid of several rounds (32 requests x 8 kv-heads x 3 row chunks) with
    ragged prefixes takes the longest-first dealing of pairs over the XCDs:
    every valid row is written (NaN-filled output, all finite afterwards),
    padded rows are zero, and the longest, the shortest and two middle requests
    match the oracle."""
    cfg = wl.CONFIGS["c4_tree_3b"]
    x = wl.generate(cfg, L=(64, 1500), with_logits=False)
    assert x["q"].shape[0] * cfg.Hkv % 8 == 0
    st = VerifyStep(cfg, x, layout="bhld")
    st.out.fill_(float("nan"))
    st.lse.fill_(float("nan"))
    st.attention_tree()
    torch.cuda.synchronize()
    out, lse = st.out.cpu().numpy(), st.lse.cpu().numpy()
    for b in range(out.shape[0]):
        nq = int(x["n_q"][b])
        assert np.isfinite(out[b, :nq]).all() and np.isfinite(lse[b, :nq]).all(), f"request {b}"
        assert (out[b, nq:] == 0).all() and np.isneginf(lse[b, nq:]).all(), f"request {b} padding"
    order = np.argsort(-x["cache_len"], kind="stable")
    pick = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2]), int(order[len(order) // 3])})
    say(f"    prefixes {int(x['cache_len'].min())}..{int(x['cache_len'].max())}; oracle on requests {pick}")
    sub = {k: (v[pick] if isinstance(v, np.ndarray) and v.ndim >= 1 and v.shape[0] == out.shape[0] else v)
           for k, v in x.items()}
    check_oracle(out[pick], lse[pick], sub, cfg)
