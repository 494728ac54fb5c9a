"""GPU parity of acceptance by probability (spec_prob_accept) against the oracle.

Bars: the greedy tokens bit-exact; each node's target probability within a
relative 2e-5 of the float64 softmax; the accepted lengths, paths and
correction tokens bit-exact against the oracle computed from the logits and
the draws alone (its decisions are the real-valued comparisons, in float64).
Thresholds and uniform draws are chosen a clear relative margin (1e-3, fifty
times the probability tolerance) away from every node's decision boundary,
so the float32 arithmetic of the kernel cannot flip a decision; a request
whose nodes sit inside the band anyway (the workload-driven cases, whose
inputs are not steered) is left out of the path comparison and counted, and
such requests must be rare.  Soft matching's acceptance rate over seeded
uniforms is checked against the target probability with a binomial bound.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from masked_verification_attention_amd import binding as bd
from masked_verification_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

P_RTOL = 2e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(a, dt=None):
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(logits, dt, n_nodes, draft, parent, vrow, max_depth, mode, threshold=0.0, dprob=None, unif=None):
    B, T, V = logits.shape
    dev = dict(device="cuda")
    am = torch.full((B, T), -9, dtype=torch.int32, **dev)
    prob = torch.full((B, T), -9.0, dtype=torch.float32, **dev)
    ln = torch.full((B,), -9, dtype=torch.int32, **dev)
    pth = torch.full((B, max_depth), -9, dtype=torch.int32, **dev)
    bonus = torch.full((B,), -9, dtype=torch.int32, **dev)
    bd.spec_prob_accept(upload(logits, dt), bd.SPEC_BF16 if dt == "bf16" else bd.SPEC_F32, B, T, V,
                        upload(n_nodes), upload(draft), upload(parent), None if vrow is None else upload(vrow),
                        max_depth, mode, threshold, None if dprob is None else upload(dprob.astype(np.float32)),
                        None if unif is None else upload(unif.astype(np.float32)), am, prob, ln, pth, bonus)
    torch.cuda.synchronize()
    return am.cpu().numpy(), prob.cpu().numpy(), ln.cpu().numpy(), pth.cpu().numpy(), bonus.cpu().numpy()


def random_case(rng, B, T, V, dt, rows):
    raw = rng.standard_normal((B, T, V)).astype(np.float32) * 2.0
    draft = rng.integers(0, V, size=(B, T)).astype(np.int32)
    # a third of the drafts are the row's best or second-best token: probabilities span the range
    for b in range(B):
        for t in range(T):
            r = rng.random()
            if r < 0.35:
                order = np.argsort(-raw[b, t])
                draft[b, t] = order[0] if r < 0.2 else order[1]
    parent = np.full((B, T), -1, dtype=np.int32)
    for b in range(B):
        for v in range(1, T):
            parent[b, v] = int(rng.integers(-1, v)) if rows == "same" else int(rng.integers(0, v))
    vrow = None
    if rows == "parent":
        # explicit root (node 0) and a parent's row verifying each child
        vrow = parent.copy()
        vrow[:, 0] = -1
        # the drafts are read against the parent's row: re-draw the strong ones there
        for b in range(B):
            for v in range(1, T):
                if rng.random() < 0.35:
                    draft[b, v] = int(np.argmax(raw[b, parent[b, v]]))
    data = wl.f32_to_bf16_bits(raw) if dt == "bf16" else raw
    n_nodes = rng.integers(max(1, T - 3), T + 1, size=B).astype(np.int32)
    return data, draft, parent, vrow, n_nodes


MARGIN = 1e-3     # relative distance of every steered decision from its boundary


def edge_of(mode, threshold, dprob, unif, b, v):
    """The value a node's probability is compared with."""
    if mode == oracle.MODE_THRESHOLD:
        return float(threshold)
    return float(unif[b, v]) * float(dprob[b, v])


def threshold_between(p):
    """A threshold strictly between two adjacent distinct probabilities near the middle,
    with at least MARGIN relative room on both sides."""
    s = np.unique(p[np.isfinite(p) & (p > 0)])
    order = sorted(range(1, len(s)), key=lambda i: abs(i - len(s) // 2))
    for i in order:
        lo, hi = s[i - 1], s[i]
        if hi > lo * (1 + 4 * MARGIN):
            return float(np.sqrt(lo * hi))
    return 0.5


def steer_uniforms(rng, p, dprob, n_nodes):
    """Uniform draws, re-drawn where u * p_d would fall within MARGIN of p."""
    unif = rng.random(p.shape).astype(np.float32)
    for b in range(p.shape[0]):
        for v in range(int(n_nodes[b])):
            while np.isfinite(p[b, v]) and abs(float(unif[b, v]) * float(dprob[b, v]) - p[b, v]) <= \
                    MARGIN * max(p[b, v], 1e-300):
                unif[b, v] = np.float32(rng.random())
    return unif


def check(case_id, data, dt, n_nodes, draft, parent, vrow, max_depth, mode, threshold=0.0, dprob=None, unif=None,
          steered=True):
    am, prob, ln, pth, bonus = run(data, dt, n_nodes, draft, parent, vrow, max_depth, mode, threshold, dprob, unif)
    greedy, p_ref, ok_ref, A_ref, path_ref, bonus_ref = oracle.prob_accept(
        data, dt, n_nodes, draft, parent, vrow, max_depth, mode, threshold, dprob, unif)
    B, T = draft.shape
    for b in range(B):
        n = int(n_nodes[b])
        np.testing.assert_array_equal(am[b, :n], greedy[b, :n])
        assert (am[b, n:] == -1).all() and np.isnan(prob[b, n:]).all()
        np.testing.assert_allclose(prob[b, :n], p_ref[b, :n], rtol=P_RTOL, atol=1e-30)
    # requests with a node whose probability lies within the band of its boundary
    near = []
    for b in range(B):
        for v in range(int(n_nodes[b])):
            # NaN rows, the unchecked root and the definitional zeros (a row or token out of
            # range: exactly 0 on both sides) decide nothing near a boundary
            if not np.isfinite(p_ref[b, v]) or p_ref[b, v] == 0.0 or (vrow is not None and vrow[b, v] == -1):
                continue
            edge = edge_of(mode, threshold, dprob, unif, b, v)
            if abs(p_ref[b, v] - edge) <= 2 * P_RTOL * max(abs(edge), p_ref[b, v], 1e-300):
                near.append(b)
                break
    if steered:
        assert not near, f"steered inputs left requests {near} at the boundary"
    else:
        assert len(near) <= max(1, B // 8), f"too many boundary requests: {near}"
    keep = [b for b in range(B) if b not in near]
    np.testing.assert_array_equal(ln[keep], A_ref[keep])
    np.testing.assert_array_equal(pth[keep], path_ref[keep])
    np.testing.assert_array_equal(bonus[keep], bonus_ref[keep])
    say(f"    {case_id}: accepted {ln.tolist()[:8]}, accepted nodes {int(ok_ref.sum())}, "
        f"boundary requests {len(near)}")


CASES = [
    # (id, B, T, V, dtype, rows)
    ("bf16_same_rows", 4, 30, 32000, "bf16", "same"),
    ("bf16_parent_rows_llama", 3, 31, 128256, "bf16", "parent"),
    ("f32_misaligned", 3, 12, 1003, "f32", "same"),
    ("bf16_misaligned_parent", 3, 20, 1001, "bf16", "parent"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("mode", [oracle.MODE_THRESHOLD, oracle.MODE_SOFT], ids=["threshold", "soft"])
def test_prob_accept_parity(case, mode):
    cid, B, T, V, dt, rows = case
    rng = np.random.default_rng(len(cid) * 100 + B * 10 + mode)
    say(f"[gpu] prob accept {cid} mode {mode}")
    data, draft, parent, vrow, n_nodes = random_case(rng, B, T, V, dt, rows)
    p = oracle.node_probs(data, dt, n_nodes, draft, vrow)
    if mode == oracle.MODE_THRESHOLD:
        check(cid, data, dt, n_nodes, draft, parent, vrow, 8, mode, threshold=threshold_between(p))
        check(cid + "/t0", data, dt, n_nodes, draft, parent, vrow, 8, mode, threshold=0.0, steered=False)
    else:
        dprob = rng.random((B, T)).astype(np.float32)
        dprob[:, ::7] = 0.0
        unif = steer_uniforms(rng, p, dprob, n_nodes)
        check(cid, data, dt, n_nodes, draft, parent, vrow, 8, mode, dprob=dprob, unif=unif)


def test_soft_acceptance_rate_on_device():
    # 4096 one-node requests over the same row: accepted iff u < p, so the rate is p
    rng = np.random.default_rng(21)
    B, V = 4096, 1000
    row = (rng.standard_normal(V) * 2).astype(np.float32)
    x = int(np.argsort(row)[-2])
    logits = np.broadcast_to(row, (B, 1, V)).copy()
    draft = np.full((B, 1), x, dtype=np.int32)
    parent = np.full((B, 1), -1, dtype=np.int32)
    n_nodes = np.ones(B, dtype=np.int32)
    unif = rng.random((B, 1)).astype(np.float32)
    _, prob, ln, _, _ = run(logits, "f32", n_nodes, draft, parent, None, 2, oracle.MODE_SOFT,
                            dprob=np.ones((B, 1), np.float32), unif=unif)
    pt = oracle.target_prob(row, "f32", x)
    hits = int(ln.sum())
    sd = np.sqrt(B * pt * (1 - pt))
    say(f"    soft rate: p = {pt:.4f}, accepted {hits} of {B}")
    assert abs(hits - B * pt) < 5 * sd
    assert (ln == (unif[:, 0] < prob[:, 0])).all()


def test_planted_workload_threshold():
    # the ConFu-shaped workload's planted drafts (logit 8 over standard normal rows of
    # 128256) carry probability ~0.01: a threshold of 1e-3 accepts them, 0.5 none
    cfg = wl.CONFIGS["c3_confu_8b"]
    x = wl.generate(cfg, B=4, L=(8, 8))
    for thr in (1e-3, 0.5):
        check(f"c3_planted/{thr}", x["logits"], "bf16", x["n_nodes"], x["draft_tok"], x["acc_parent"], None,
              cfg.max_depth, oracle.MODE_THRESHOLD, threshold=thr, steered=False)


@pytest.mark.parametrize("rule", ["threshold", "soft"])
def test_step_with_probability_acceptance(rule):
    # the whole step (mask, attention, probability acceptance, commit) as the benchmark runs it,
    # against the oracle computed from the logits and draws alone
    from masked_verification_attention_amd.step import VerifyStep
    cfg = wl.CONFIGS["c3_confu_8b"]
    x = wl.generate(cfg, B=3, L=(40, 80))
    rng = np.random.default_rng(5)
    mode = oracle.MODE_THRESHOLD if rule == "threshold" else oracle.MODE_SOFT
    dprob = (rng.random(x["acc_parent"].shape) * 0.02).astype(np.float32)
    p0 = oracle.node_probs(x["logits"], "bf16", x["n_nodes"], x["draft_tok"], None)
    unif = steer_uniforms(rng, p0, dprob, x["n_nodes"])
    st = VerifyStep(cfg, x, accept=rule, threshold=1e-3, draft_prob=dprob, uniform=unif)
    st.run()
    torch.cuda.synchronize()
    prob = st.out_prob.cpu().numpy().astype(np.float64)
    _, p_ref, ok_ref, A, path, _ = oracle.prob_accept(x["logits"], "bf16", x["n_nodes"], x["draft_tok"],
                                                      x["acc_parent"], None, st.max_depth, mode, 1e-3, dprob, unif)
    np.testing.assert_allclose(prob, p_ref, rtol=P_RTOL, atol=1e-30)
    # the threshold 1e-3 sits far from both the planted drafts (~1e-2) and the others (~1e-5)
    n = x["n_nodes"]
    for b in range(len(n)):
        for v in range(int(n[b])):
            edge = 1e-3 if mode == oracle.MODE_THRESHOLD else float(unif[b, v]) * float(dprob[b, v])
            assert abs(p_ref[b, v] - edge) > MARGIN * max(edge, p_ref[b, v]), (b, v)
    np.testing.assert_array_equal(st.out_len.cpu().numpy(), A)
    np.testing.assert_array_equal(st.out_path.cpu().numpy(), path)
    kc, vc, L2 = oracle.commit_kv(x["k_cache"], x["v_cache"], x["cache_len"], x["k_blk"], x["v_blk"], A, path)
    np.testing.assert_array_equal(st.cache_len_out.cpu().numpy(), L2)
    k_host, v_host = st.cache_host()
    np.testing.assert_array_equal(k_host, kc)
    np.testing.assert_array_equal(v_host, vc)
    say(f"    {rule}: accepted {A.tolist()} ({int(ok_ref.sum())} nodes pass)")


def _edge_rows(V, rng):
    """Rows for the NaN and infinity rules: NaN as the first entry of many 16-byte
    vectors, a row whose only numbers are -inf, a row of NaN only, a row of -inf
    only, +inf entries, ties across vectors, signed zeros."""
    rows = []
    a = rng.standard_normal(V).astype(np.float32)
    a[::8] = np.nan                                  # first entry of every bf16 vector
    a[::4] = np.where(np.arange(0, V, 4) % 8 == 0, np.nan, a[::4])
    rows.append(a)
    a = np.full(V, np.nan, np.float32)
    a[[7, 300]] = -np.inf
    rows.append(a)
    rows.append(np.full(V, np.nan, np.float32))
    rows.append(np.full(V, -np.inf, np.float32))
    a = rng.standard_normal(V).astype(np.float32)
    a[[1000, 17]] = np.inf
    rows.append(a)
    a = rng.standard_normal(V).astype(np.float32)
    a[rng.choice(V, 40, replace=False)] = a.max() + 1.0
    rows.append(a)
    a = np.where(rng.random(V) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    rows.append(a)
    rows.append(rng.standard_normal(V).astype(np.float32))
    return np.stack(rows)


def _bits(a):
    bits = wl.f32_to_bf16_bits(np.nan_to_num(a, nan=0.0, posinf=0.0, neginf=0.0))
    bits = np.where(np.isnan(a), np.uint16(0x7fc0), bits)
    bits = np.where(np.isposinf(a), np.uint16(0x7f80), bits)
    bits = np.where(np.isneginf(a), np.uint16(0xff80), bits)
    return bits.astype(np.uint16)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_greedy_token_and_probabilities_with_nan_and_infinities(dt):
    """Both argmax kernels follow the greedy rule on crafted rows (NaN after every
    number, first index on ties); the probability is NaN exactly where the
    oracle's is (a NaN entry, or a row without a finite maximum)."""
    rng = np.random.default_rng(23)
    V = 5003                                         # odd: rows start misaligned
    rows = _edge_rows(V, rng)
    T = rows.shape[0]
    raw = np.ascontiguousarray(rows[None], dtype=np.float32)       # B = 1
    data = _bits(raw) if dt == "bf16" else raw
    want = oracle.greedy_tokens(data, dt)
    n_nodes = np.array([T], dtype=np.int32)
    parent = np.arange(-1, T - 1, dtype=np.int32)[None]
    draft = want.copy().astype(np.int32)
    draft[0, 3] = 5                                  # a draft the -inf row's token is not
    say(f"[gpu] argmax / lse edge rows {dt}: V={V} rows={T}")
    # the greedy kernel (spec_argmax_accept)
    dev = dict(dtype=torch.int32, device="cuda")
    am = torch.full((1, T), -9, **dev)
    ln = torch.full((1,), -9, **dev)
    pth = torch.full((1, 8), -9, **dev)
    bd.spec_argmax_accept(upload(data, dt), bd.SPEC_BF16 if dt == "bf16" else bd.SPEC_F32, 1, T, V,
                          upload(n_nodes), upload(draft), upload(parent), 8, am, ln, pth)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(am.cpu().numpy(), want)
    # the greedy token + log-sum-exp kernel (spec_prob_accept)
    got_am, prob, _, _, _ = run(data, dt, n_nodes, draft, parent, None, 8, bd.SPEC_ACCEPT_THRESHOLD, 0.5)
    np.testing.assert_array_equal(got_am, want)
    ref_p = oracle.node_probs(data, dt, n_nodes, draft, None)
    np.testing.assert_array_equal(np.isnan(prob), np.isnan(ref_p))
    fin = ~np.isnan(ref_p)
    np.testing.assert_allclose(prob[fin], ref_p[fin], rtol=P_RTOL, atol=0)
