"""Greedy acceptance of a draft tree (oracle side).

Definitions:

* Greedy target token of node v: the index of the largest logit of node v's
  row (hard matching in the verification step of Speculative Streaming; the
  check of predictions at the lookahead positions in Lookahead Attention
  section 2.3).  Row v verifies node v.  Ties go to the lowest index, and
  -0 equals +0.  NaN logits rank after every number (-inf included), so a
  row's greedy token is a NaN entry only when the row holds no number (then
  its first entry); this is the top-1 of the tree draft's top-k rule.
* Node v matches when its drafted token equals its greedy target token.  It
  is accepted when it matches and so does every node on its path from the
  root (a branch is followed until a rejection).  Its depth is the number of
  nodes on that path; nodes with parent -1 hang off the root and have depth 1.
  Nodes deeper than ``max_depth`` are never accepted (the caller's bound on
  the path length).
* The accepted length A is the largest depth of an accepted node (0 if none),
  i.e. the longest accepted path; for a chain it is the leading run of
  matches (Lookahead Attention section 2.4, longest consistent prefix).
* When several accepted nodes reach depth A, the path is the one a
  depth-first walk from the root meets first, visiting children in
  increasing index order; that is the path whose node-index sequence is
  lexicographically smallest.  ``path[d]`` is the node at depth d+1, and
  entries past A are -1.
"""

from typing import Tuple

import numpy as np

from .bf16 import as_f64


def greedy_tokens(logits: np.ndarray, logits_dtype: str) -> np.ndarray:
    """Per-row argmax over the vocabulary: the first index of the largest
    number, NaN ignored; a row of NaN only gives 0.  [..., V] -> [...] int32."""
    x = as_f64(logits, logits_dtype)
    nan = np.isnan(x)
    num = np.where(nan, -np.inf, x)
    top = num.max(axis=-1, keepdims=True)
    is_top = (num == top) & ~nan                      # numbers equal to the row's largest
    first_top = np.argmax(is_top, axis=-1)            # first True
    return np.where(is_top.any(axis=-1), first_top, 0).astype(np.int32)


def accept_request(draft_tok, acc_parent, greedy, n_nodes: int, max_depth: int):
    """Return (A, path[max_depth]) for one request."""
    n = int(n_nodes)
    depth = np.zeros(n, dtype=np.int64)
    acc = np.zeros(n, dtype=bool)
    for v in range(n):
        p = int(acc_parent[v])
        if p >= v:
            raise ValueError("acceptance parents must precede their children")
        ok = int(draft_tok[v]) == int(greedy[v])
        depth[v] = 1 if p < 0 else depth[p] + 1
        acc[v] = ok and (p < 0 or acc[p]) and depth[v] <= max_depth
    path = np.full(max_depth, -1, dtype=np.int32)
    if not acc.any():
        return 0, path
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
    return A, path


def argmax_accept(logits, logits_dtype: str, n_nodes, draft_tok, acc_parent,
                  max_depth: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Batch form: (greedy [B, T], out_len [B], out_path [B, max_depth]), all int32."""
    greedy = greedy_tokens(logits, logits_dtype)
    B = greedy.shape[0]
    out_len = np.zeros(B, dtype=np.int32)
    out_path = np.full((B, max_depth), -1, dtype=np.int32)
    for b in range(B):
        out_len[b], out_path[b] = accept_request(draft_tok[b], acc_parent[b], greedy[b],
                                                 int(n_nodes[b]), max_depth)
    return greedy, out_len, out_path


# ---------------------------------------------------------------------------
# Acceptance with explicit verification rows (real-model alignment).
#
# Speculative Streaming, "The verification step": the walk starts at the root,
# which is the previous step's correction token and is part of the block; the
# drafted token of a node is checked against the target's prediction at that
# position -- the output row of the position before it, i.e. its parent's row
# -- and the step advances by the accepted drafts plus one correction token
# drawn from the target's logits at the point where the walk stopped.  ConFu
# (overall framework) carries the future prediction of the last accepted token
# into the next round, which is the same node index.
#
# Definitions (a generalisation of the rules above):
#   * verify_row[v] = -1: node v is accepted without a check (the explicit,
#     pre-accepted root whose KV is committed with the path).
#   * verify_row[v] = u >= 0: node v matches when draft_tok[v] equals the
#     greedy token of row u; a row outside [0, n_nodes) never matches.
#   * acceptance, depth, max_depth, the accepted length A and the DFS-first
#     path are as for accept_request (depth counts the root when it is a node).
#   * last = path[A - 1] (-1 when A = 0); bonus = greedy[last], the correction
#     token, -1 when A = 0.
# verify_row = the identity reproduces accept_request.
# ---------------------------------------------------------------------------


def accept_request_rows(draft_tok, acc_parent, verify_row, greedy, n_nodes: int, max_depth: int):
    """Return (A, path[max_depth], last, bonus) for one request."""
    n = int(n_nodes)
    depth = np.zeros(n, dtype=np.int64)
    acc = np.zeros(n, dtype=bool)
    for v in range(n):
        p = int(acc_parent[v])
        if p >= v:
            raise ValueError("acceptance parents must precede their children")
        u = int(verify_row[v])
        if u == -1:
            ok = True
        elif 0 <= u < n:
            ok = int(draft_tok[v]) == int(greedy[u])
        else:
            ok = False
        depth[v] = 1 if p < 0 else depth[p] + 1
        acc[v] = ok and (p < 0 or acc[p]) and depth[v] <= max_depth
    path = np.full(max_depth, -1, dtype=np.int32)
    if not acc.any():
        return 0, path, -1, -1
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
    last = int(best[-1])
    return A, path, last, int(greedy[last])


def argmax_accept_rows(logits, logits_dtype: str, n_nodes, draft_tok, acc_parent, verify_row,
                       max_depth: int):
    """Batch form: (greedy [B, T], out_len [B], out_path [B, max_depth], out_last [B],
    out_bonus [B]), all int32.  verify_row None means row v verifies node v."""
    greedy = greedy_tokens(logits, logits_dtype)
    B, T = greedy.shape
    if verify_row is None:
        verify_row = np.broadcast_to(np.arange(T, dtype=np.int32), (B, T))
    out_len = np.zeros(B, dtype=np.int32)
    out_path = np.full((B, max_depth), -1, dtype=np.int32)
    out_last = np.full(B, -1, dtype=np.int32)
    out_bonus = np.full(B, -1, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        g = greedy[b].copy()
        g[n:] = -1   # rows past n_nodes carry no greedy token
        out_len[b], out_path[b], out_last[b], out_bonus[b] = accept_request_rows(
            draft_tok[b], acc_parent[b], verify_row[b], g, n, max_depth)
    return greedy, out_len, out_path, out_last, out_bonus
