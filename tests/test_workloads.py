"""Generator checks (CPU only): determinism, bf16 rounding, structure, canaries."""

import numpy as np
import pytest
import torch

import oracle
from masked_verification_attention_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.Generator(np.random.PCG64(0))
    x = np.concatenate([rng.standard_normal(100000, dtype=np.float32),
                        np.array([1.0, -0.0, 0.0, 3.0039062, 1.00390625, 1.01171875, 65504.0, 1e-30],
                                 dtype=np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_deterministic_per_seed():
    cfg = wl.CONFIGS["c3_confu_8b"]
    a = wl.generate(cfg, B=2, L=(64, 64))
    b = wl.generate(cfg, B=2, L=(64, 64))
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    c = wl.generate(cfg, seed=7, B=2, L=(64, 64))
    assert not np.array_equal(a["q"], c["q"])


@pytest.mark.parametrize("name", sorted(wl.CONFIGS))
def test_structure_and_canaries(name):
    cfg = wl.CONFIGS[name]
    lo, hi = cfg.L
    small_L = None if cfg.structure == "la_full" else (min(lo, 64), min(hi, 96))
    x = wl.generate(cfg, B=min(cfg.B, 3), L=small_L)
    Bn = x["q"].shape[0]
    assert x["q"].shape == (Bn, cfg.Tq, cfg.Hq, cfg.D)
    assert x["k_cache"].shape[1] == int(x["cache_len"].max()) + cfg.Tq
    for b in range(Bn):
        par = x["attn_parent"][b]
        assert all(-1 <= p < r for r, p in enumerate(par))
        ap = x["acc_parent"][b]
        assert all(-1 <= p < v for v, p in enumerate(ap))
        L = x["cache_len"][b]
        slots = x["k_cache"][b, L:]
        if cfg.dtype == "bf16":
            assert (slots == wl.BF16_NAN).all()
            assert (x["k_cache"][b, :L] != wl.BF16_NAN).all()
        else:
            assert np.isnan(slots).all() and np.isfinite(x["k_cache"][b, :L]).all()
    if cfg.structure == "confu_tree":
        d = np.zeros(cfg.T, int)
        for b in range(Bn):
            par = x["acc_parent"][b]
            for v, p in enumerate(par):
                d[v] = 1 if p < 0 else d[p] + 1
            assert d.max() <= cfg.depth_cap
            assert (x["sp_flag"][b, cfg.T:] == 1).all() and (x["sp_flag"][b, :cfg.T] == 0).all()
            assert list(x["attn_parent"][b, cfg.T:]) == list(range(cfg.T))


def test_planted_drafts_are_the_greedy_tokens():
    for name in ("c1_tiny_la", "c2_la_7b"):
        cfg = wl.CONFIGS[name]
        x = wl.generate(cfg, B=min(cfg.B, 2), L=(64, 64))
        greedy = oracle.greedy_tokens(x["logits"], cfg.logits_dtype)
        assert (greedy[x["planted"]] == x["draft_tok"][x["planted"]]).all()
        if cfg.exact_accepts is not None:
            assert (x["planted"].sum(axis=1) == cfg.exact_accepts).all()
