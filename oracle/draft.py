"""The next tree draft from the speculative streams (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Speculative Streaming, tree draft construction and "parallel new draft
generation": the pass that verifies one draft also drafts the next one.  The
gamma speculative streams of the last accepted node (the new root) give one
logit row each; from stream j's row the top-k tokens are taken; the tokens of
stream j are the parents of the tokens of stream j + 1 and the tokens of
stream 1 hang off the correction token, which is the root.  Every node of
level j - 1 therefore receives stream j's k tokens as its children: a tree
of depth gamma, 1 + sum_{g=1..gamma} k^g nodes, flattened level by level.

Readings taken where the page leaves a step open:
* "top-k" is the k highest logits of the row, best first, equal logits in
  increasing token order (k = 1 is the greedy token).  NaN logits rank after
  every number, -inf included, in increasing token order.
* Within a level, nodes follow their parents' order and, under one parent,
  the rank of their token in the stream's top-k list.
* The streams' rows are those of the multi-stream layout (``msa.msa_row``) of
  the last node on the accepted path; a request with no accepted node, or
  whose last node or stream rows lie outside its block, gets no draft (zero
  nodes).
"""

from typing import List, Tuple

import numpy as np

from .bf16 import as_f64
from .msa import msa_row


def topk_tokens(row: np.ndarray, dtype: str, k: int) -> np.ndarray:
    """The k best token indices of one logit row, best first, ties to the lower index."""
    x = as_f64(np.asarray(row), dtype)
    nan = np.isnan(x)
    # sort keys, most significant last: numbers before NaN (-inf included), then
    # larger value first, then lower index first
    order = np.lexsort((np.arange(x.size), np.where(nan, 0.0, -x), nan))
    return order[:k].astype(np.int32)


def draft_tree(topk: np.ndarray, root_tok: int) -> Tuple[np.ndarray, np.ndarray]:
    """(tokens [N], parents [N]) of the tree draft from per-stream top-k lists [gamma, k].

    Built level by level as the page describes: the root is the correction
    token, and every node of the previous level gets stream j's tokens as its
    children.
    """
    gamma, k = topk.shape if topk.size else (0, 0)
    tokens: List[int] = [int(root_tok)]
    parents: List[int] = [-1]
    level = [0]
    for j in range(gamma):
        nxt = []
        for p in level:
            for i in range(k):
                tokens.append(int(topk[j, i]))
                parents.append(p)
                nxt.append(len(tokens) - 1)
        level = nxt
    return np.array(tokens, dtype=np.int32), np.array(parents, dtype=np.int32)


def next_draft(logits: np.ndarray, logits_dtype: str, n_nodes, acc_len, acc_path, root_tok,
               gamma: int, k: int):
    """Batch form: (topk [B, gamma, k], draft_tok [B, N], tree_parent [B, N], n_out [B]).

    logits [B, R, V] holds the multi-stream block's rows; the streams of the
    last accepted node of request b are read.  Requests without a draft have
    n_out = 0 and -1 everywhere.
    """
    B = logits.shape[0]
    N = 1 + sum(k ** g for g in range(1, gamma + 1))
    topk = np.full((B, gamma, k), -1, dtype=np.int32)
    tok = np.full((B, N), -1, dtype=np.int32)
    par = np.full((B, N), -1, dtype=np.int32)
    n_out = np.zeros(B, dtype=np.int32)
    for b in range(B):
        A = int(acc_len[b])
        if A < 1:
            continue
        last = int(acc_path[b][A - 1])
        n = int(n_nodes[b])
        if not 0 <= last < n or n * (1 + gamma) > logits.shape[1]:
            continue                                # no such node's streams in the block
        for j in range(1, gamma + 1):
            topk[b, j - 1] = topk_tokens(logits[b, msa_row(n, gamma, last, j)], logits_dtype, k)
        tok[b], par[b] = draft_tree(topk[b], int(root_tok[b]))
        n_out[b] = N
    return topk, tok, par, n_out
