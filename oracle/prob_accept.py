"""Probability-based acceptance of a draft tree (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Two non-greedy acceptance rules the pages name beside hard matching:

* Lookahead Attention (its verification): a proposal is accepted when the
  target's probability of it exceeds a threshold; the output is the longest
  prefix of proposals that all pass.
* Speculative Streaming (the verification step, soft matching, after
  Leviathan et al.): a drafted token x is accepted with probability
  min(1, p_target(x) / p_draft(x)).  The random draw is an input here: with a
  uniform u in [0, 1) the node is accepted iff u < min(1, p_t / p_d), i.e.
  u * p_d < p_t (a draft probability of 0 accepts iff p_t > 0).

p_target(x) is the softmax of the verification row's logits at x (exact, in
float64).  Everything else is the verification step of the greedy rule: a
node counts only if every node on its root path is accepted, the longest
accepted path wins, depth-first-first among equals, the root of an explicit
tree (verification row -1) is accepted unchecked, a row outside the request's
nodes never accepts, and the correction token is the greedy token of the last
accepted node's row (this reading keeps the correction deterministic; the
pages' residual resampling needs the draft's whole distribution).

Both decisions are the real-valued comparisons the pages state, taken in
float64: p_t is the float64 softmax, and the inputs threshold, u and p_d are
widened exactly (they arrive as float32 or Python floats).
"""

import numpy as np

from .acceptance import greedy_tokens
from .bf16 import as_f64

MODE_THRESHOLD = 1
MODE_SOFT = 2


def target_prob(row: np.ndarray, dtype: str, x: int) -> float:
    """softmax(row)[x] in float64."""
    z = as_f64(np.asarray(row), dtype)
    with np.errstate(invalid="ignore", over="ignore"):   # NaN / infinite rows give NaN, as intended
        m = z.max()
        e = np.exp(z - m)
        return float(e[x] / e.sum())


def node_probs(logits, dtype: str, n_nodes, draft_tok, verify_row):
    """p [B, T] float64: the target probability of each node's draft at its verification row
    (1 for the unchecked root, 0 for a row or token out of range, NaN past n)."""
    B, T, V = logits.shape
    p = np.full((B, T), np.nan)
    for b in range(B):
        n = int(n_nodes[b])
        for v in range(n):
            u = v if verify_row is None else int(verify_row[b, v])
            x = int(draft_tok[b, v])
            if u == -1:
                p[b, v] = 1.0
            elif 0 <= u < n and 0 <= x < V:
                p[b, v] = target_prob(logits[b, u], dtype, x)
            else:
                p[b, v] = 0.0
    return p


def decide(p: float, mode: int, threshold: float = 0.0, draft_p: float = 1.0, u: float = 0.0) -> bool:
    """One node's acceptance from its target probability p (float64): the threshold
    rule p > threshold, or soft matching u < min(1, p / p_d), written u * p_d < p so
    that p_d = 0 needs no division (a NaN p accepts under neither rule)."""
    p = float(p)
    if mode == MODE_THRESHOLD:
        return p > float(threshold)
    if mode == MODE_SOFT:
        return float(u) * float(draft_p) < p
    raise ValueError(mode)


def scan_accepted(ok, acc_parent, n: int, max_depth: int):
    """(A, path [max_depth], last) from per-node acceptance bits: deepest node whose whole
    root path is accepted, the depth-first-first one among equals."""
    depth = np.zeros(n, dtype=np.int64)
    acc = np.zeros(n, dtype=bool)
    for v in range(n):
        p = int(acc_parent[v])
        if p >= v:
            raise ValueError("acceptance parents must precede their children")
        depth[v] = 1 if p < 0 else depth[p] + 1
        acc[v] = bool(ok[v]) and (p < 0 or acc[p]) and depth[v] <= max_depth
    path = np.full(max_depth, -1, dtype=np.int32)
    if not acc.any():
        return 0, path, -1
    A = int(depth[acc].max())
    best = None
    for v in range(n):
        if acc[v] and depth[v] == A:
            chain = []
            u = v
            while u >= 0:
                chain.append(u)
                u = int(acc_parent[u])
            chain.reverse()
            if best is None or chain < best:
                best = chain
    path[:A] = best
    return A, path, best[-1]


def prob_accept(logits, logits_dtype: str, n_nodes, draft_tok, acc_parent, verify_row, max_depth: int,
                mode: int, threshold: float = 0.0, draft_prob=None, uniform=None):
    """Batch form: (greedy [B, T], p [B, T], ok [B, T], out_len [B], out_path [B, max_depth],
    out_bonus [B]), everything computed here from the logits and the given draws."""
    B, T, V = logits.shape
    greedy = greedy_tokens(logits, logits_dtype)
    p = node_probs(logits, logits_dtype, n_nodes, draft_tok, verify_row)
    ok = np.zeros((B, T), dtype=bool)
    out_len = np.zeros(B, dtype=np.int32)
    out_path = np.full((B, max_depth), -1, dtype=np.int32)
    out_bonus = np.full(B, -1, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        for v in range(n):
            u = v if verify_row is None else int(verify_row[b, v])
            if u == -1:
                ok[b, v] = True
            elif 0 <= u < n:
                ok[b, v] = decide(p[b, v], mode, threshold,
                                  1.0 if draft_prob is None else draft_prob[b, v],
                                  0.0 if uniform is None else uniform[b, v])
        A, path, last = scan_accepted(ok[b], acc_parent[b], n, max_depth)
        out_len[b], out_path[b] = A, path
        if A > 0:
            out_bonus[b] = greedy[b, last]
    return greedy, p, ok, out_len, out_path, out_bonus
