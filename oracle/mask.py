"""Visibility of keys for the query rows of a speculative block (oracle side).

One parent array per request describes every mask the pages use.  Row r of
the speculative block has ``attn_parent[r]`` in {-1} and [0, r); -1 means the
row hangs directly off the already-cached prefix (the implicit root).

* Row r sees every cached prefix key.  The block keys it sees are itself and
  its ancestors through the parent links.  This is the tree rule of
  Speculative Streaming (tree draft, Equation 4): each node attends to the
  path from the root to itself and to no other branch.  The printed form of
  Equation 4 only admits the immediate parent stream; its prose (ancestors
  back to the root) is taken as the definition, with the node itself included
  as in causal attention (Equation 1 lets a position see itself).
* Lookahead Attention (section 3.1, M_LA = [M_causal, 1; 0, M_lookahead]):
  rows are queries.  With the n original tokens as a chain and every
  lookahead row's parent the last original, the ancestor rule yields exactly
  M_LA: originals see originals causally and never a lookahead row; a
  lookahead row sees all n originals and itself only (M_lookahead diagonal).
  With the originals already in the cache every lookahead row's parent is -1
  and the row sees prefix plus itself.
* ConFu (key design 1): a contemplate row's parent is the node it is attached
  to, so it sees that node's path, the node and itself.  The soft-prompt keys
  sit in the KV cache and only rows with ``sp_flag`` set (the contemplate
  rows) see them.
* Rows r >= n_q (batch padding, Lookahead Attention section 3.3) see nothing.
"""

from typing import List, Tuple

import numpy as np


def ancestor_rows(attn_parent_row: np.ndarray, r: int) -> List[int]:
    """Block rows strictly above r, walking parent links up to the prefix (nearest first)."""
    out = []
    p = int(attn_parent_row[r])
    while p >= 0:
        if p >= r or p in out:
            raise ValueError(f"parent array is not topological at row {r}")
        out.append(p)
        p = int(attn_parent_row[p])
    return out


def block_visibility(attn_parent_row: np.ndarray, n_q: int, Tq: int) -> np.ndarray:
    """Dense bool [Tq, Tq]: M[r, c] = row r may see block key c."""
    M = np.zeros((Tq, Tq), dtype=bool)
    for r in range(min(n_q, Tq)):
        M[r, r] = True
        for c in ancestor_rows(attn_parent_row, r):
            M[r, c] = True
    return M


def soft_visibility(sp_flag_row: np.ndarray, n_q: int, Tq: int) -> np.ndarray:
    """Bool [Tq]: row r sees the soft-prompt keys (contemplate rows only)."""
    s = np.zeros(Tq, dtype=bool)
    if sp_flag_row is not None:
        s[: min(n_q, Tq)] = np.asarray(sp_flag_row[: min(n_q, Tq)]) != 0
    return s


def dense_visibility(attn_parent_row, sp_flag_row, n_q: int, S: int, L: int,
                     block=None) -> np.ndarray:
    """Dense bool [Tq, S + L + Tq] over keys ordered [soft | prefix | block].

    ConFu places the soft prompt before the input in the cache dimension; the
    order of keys does not change the attention result.  ``block`` (bool
    [Tq, Tq]) replaces the parent-array rule for the block keys (the
    multi-stream rows of ``msa``).
    """
    Tq = len(attn_parent_row) if block is None else block.shape[0]
    M = np.zeros((Tq, S + L + Tq), dtype=bool)
    valid = np.arange(Tq) < n_q
    M[:, :S] = soft_visibility(sp_flag_row, n_q, Tq)[:, None] & (S > 0)
    M[:, S:S + L] = valid[:, None]
    M[:, S + L:] = block_visibility(attn_parent_row, n_q, Tq) if block is None else block
    return M


def pack_bits(M: np.ndarray) -> np.ndarray:
    """Bit-pack the last axis of a bool array into uint32 words, bit c%32 of word c//32."""
    M = np.asarray(M, dtype=bool)
    n = M.shape[-1]
    W = (n + 31) // 32
    out = np.zeros(M.shape[:-1] + (W,), dtype=np.uint32)
    for c in range(n):
        out[..., c // 32] |= (M[..., c].astype(np.uint32) << np.uint32(c % 32))
    return out


def build_mask(attn_parent: np.ndarray, sp_flag, n_q: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Packed masks for a batch: (mask_bits [B, Tq, W], sp_bits [B, W]) as uint32."""
    B, Tq = attn_parent.shape
    W = (Tq + 31) // 32
    mask_bits = np.zeros((B, Tq, W), dtype=np.uint32)
    sp_bits = np.zeros((B, W), dtype=np.uint32)
    for b in range(B):
        mask_bits[b] = pack_bits(block_visibility(attn_parent[b], int(n_q[b]), Tq))
        sp_row = None if sp_flag is None else sp_flag[b]
        sp_bits[b] = pack_bits(soft_visibility(sp_row, int(n_q[b]), Tq))
    return mask_bits, sp_bits
