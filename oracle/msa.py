"""Multi-stream (MSA) verification rows and their visibility (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Speculative Streaming replaces attention in its top layers with Multi-Stream
Attention: every position carries one main-stream query and gamma
speculative-stream queries, all sharing the key/value projections.  In the
verification pass every node of the flattened tree draft carries its main
stream and its gamma streams ("Batching with speculative streams": the MSA
batch is (1 + gamma) times the tree size).

Which block keys a row sees (read from the page's Equations 1 and 2 with the
tree-attention rule of Equation 4 as its prose states it):

* The main stream of node v (Equation 1, causal self-attention over the main
  stream) sees the main-stream rows of the nodes on the root-to-v path, v
  included: in a tree the main-stream history "up to t" is the node's path,
  never another branch (Equation 4's prose; the printed case only admits the
  immediate parent, and the prose, ancestors back to the root, is taken).
* Speculative stream j of node v (Equation 2) sees the same main-stream rows
  plus the speculative rows of v itself with stream index 1..j, and no
  speculative row of any other node (streams never attend across time steps).
* Every valid row also sees the whole cached prefix; no row sees a soft
  prompt (the page has none).

Row layout of the block (an interface convention the library states the same
way): for a request with n tree nodes, rows 0..n-1 are the main streams of
nodes 0..n-1 and row n + v*gamma + (j-1) is speculative stream j of node v;
the request has n*(1+gamma) valid rows, the rest are padding.  Tree nodes are
in topological order: tree_parent[v] in {-1} and [0, v), -1 = the root (the
previous step's correction token).
"""

from typing import List, Tuple

import numpy as np

from .mask import pack_bits


def msa_row(n: int, gamma: int, v: int, j: int) -> int:
    """Block row of stream j (0 = main) of node v, for a request with n nodes."""
    if not (0 <= v < n and 0 <= j <= gamma):
        raise ValueError("node or stream out of range")
    return v if j == 0 else n + v * gamma + (j - 1)


def tree_path(tree_parent_row: np.ndarray, v: int) -> List[int]:
    """Nodes on the root-to-v path, v included (nearest first)."""
    out = [v]
    p = int(tree_parent_row[v])
    while p >= 0:
        if p >= out[-1] or p in out:
            raise ValueError(f"tree is not topological at node {v}")
        out.append(p)
        p = int(tree_parent_row[p])
    return out


def msa_block_visibility(tree_parent_row: np.ndarray, n: int, gamma: int, Tq: int) -> np.ndarray:
    """Dense bool [Tq, Tq]: M[r, c] = block row r may see block key c (MSA rows)."""
    if n * (1 + gamma) > Tq:
        raise ValueError("block too small for n * (1 + gamma) rows")
    M = np.zeros((Tq, Tq), dtype=bool)
    for v in range(n):
        path = tree_path(tree_parent_row, v)
        for j in range(gamma + 1):
            r = msa_row(n, gamma, v, j)
            for u in path:                      # main-stream history (Equation 1 / 2, first part)
                M[r, msa_row(n, gamma, u, 0)] = True
            for i in range(1, j + 1):           # own node's streams 1..j (Equation 2, second part)
                M[r, msa_row(n, gamma, v, i)] = True
    return M


def build_msa_mask(tree_parent: np.ndarray, n_nodes: np.ndarray, gamma: int,
                   Tq: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Packed MSA masks for a batch: (mask_bits [B, Tq, W], sp_bits [B, W], n_q [B])."""
    B = tree_parent.shape[0]
    W = (Tq + 31) // 32
    mask_bits = np.zeros((B, Tq, W), dtype=np.uint32)
    sp_bits = np.zeros((B, W), dtype=np.uint32)
    n_q = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        mask_bits[b] = pack_bits(msa_block_visibility(tree_parent[b], n, gamma, Tq))
        n_q[b] = n * (1 + gamma)
    return mask_bits, sp_bits, n_q
