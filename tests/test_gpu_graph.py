"""The verification step captured in a HIP graph (torch's CUDAGraph around the
library's launches): the library allocates nothing and clears nothing with
memsets on this path, so every replay must reproduce the eager results.  Each
replay is checked, with eager work and synchronisation between replays."""

import sys

import pytest
import torch

from masked_verification_attention_amd import workloads as wl
from masked_verification_attention_amd.step import VerifyStep

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", ["c3_confu_8b", "c6_msa_1b"])
def test_graph_replays_match_eager(name):
    cfg = wl.CONFIGS[name]
    sts = [VerifyStep(cfg, wl.generate(cfg, B=2, seed=cfg.seed + 7 * j), layout="bhld") for j in range(2)]
    for s in sts:
        s.run()
    torch.cuda.synchronize()

    def outputs(s):
        outs = [s.out, s.lse, s.argmax, s.out_len, s.out_path, s.cache_len_out]
        if s.msa:
            outs += [s.out_bonus, s.next_tok, s.next_parent, s.next_n]
        return outs

    ref = [[t.clone() for t in outputs(s)] for s in sts]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in sts:
            s.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for s in sts:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s.run()
        graphs.append(g)
    torch.cuda.synchronize()
    say(f"[gpu] graph {name}: captured {len(graphs)} steps")
    for rep in range(3):
        for i, (s, g) in enumerate(zip(sts, graphs)):
            for t in outputs(s):
                t.fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            for a, b in zip(outputs(s), ref[i]):
                assert torch.equal(a, b), (rep, i)
            s.run()                                   # eager work between replays
            torch.cuda.synchronize()


def test_concurrent_streams_match_serial():
    """Two independent steps launched on two streams at once (the library keeps
    no state between calls) give the results they give one after the other."""
    cfg = wl.CONFIGS["c3_confu_8b"]
    sts = [VerifyStep(cfg, wl.generate(cfg, B=3, seed=cfg.seed + 11 * j), layout="bhld") for j in range(2)]
    for s in sts:
        s.run()
    torch.cuda.synchronize()
    ref = [[t.clone() for t in (s.out, s.lse, s.argmax, s.out_len, s.out_path, s.cache_len_out)] for s in sts]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(5):
        for s in sts:
            for t in (s.out, s.lse, s.argmax, s.out_len, s.out_path, s.cache_len_out):
                t.fill_(-7)
        torch.cuda.synchronize()
        for s, st in zip(sts, streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                s.run()
        torch.cuda.synchronize()
        for s, r in zip(sts, ref):
            for a, b in zip((s.out, s.lse, s.argmax, s.out_len, s.out_path, s.cache_len_out), r):
                assert torch.equal(a, b), rep
    say("[gpu] two streams: 5 concurrent rounds match the serial results")


@pytest.mark.parametrize("name,accept", [("c3_confu_8b", "greedy"), ("c3_confu_8b", "soft"),
                                         ("c6_msa_1b", "greedy")])
def test_prepared_calls_match_regular_calls(name, accept):
    # the benchmark's launch path (arguments converted once) against the regular binding calls
    import numpy as np
    cfg = wl.CONFIGS[name]
    x = wl.generate(cfg, B=2, seed=cfg.seed + 3)
    rng = np.random.default_rng(1)
    T = x["acc_parent"].shape[1]
    kw = dict(layout="bhld", accept=accept, threshold=1e-3,
              draft_prob=(rng.random((2, T)) * 0.02).astype(np.float32),
              uniform=rng.random((2, T)).astype(np.float32))
    a, b = VerifyStep(cfg, x, **kw), VerifyStep(cfg, x, **kw)
    a.run()
    stream = torch.cuda.current_stream()
    for calls in b.prepare(stream):
        for call in calls:
            call()
    torch.cuda.synchronize()
    names = ["out", "lse", "argmax", "out_len", "out_path", "cache_len_out", "mask_bits", "sp_bits"]
    if a.msa:
        names += ["out_bonus", "next_tok", "next_parent", "next_n"]
    if accept != "greedy":
        names += ["out_prob"]
    for n in names:
        assert torch.equal(getattr(a, n), getattr(b, n)), n
    ka, va = a.cache_host()
    kb, vb = b.cache_host()
    assert (ka == kb).all() and (va == vb).all()
