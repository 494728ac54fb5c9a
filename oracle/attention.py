"""Masked verification attention in float64 (oracle side).

Definition (Speculative Streaming, Equation 1 -- standard multi-head
attention): for a query row r and query head j, over the keys the row may
see, out = softmax(q k^T / sqrt(d)) v, and lse = m + ln(sum exp(s - m)) with
m the largest scaled score.  Query head j reads key/value head
floor(j * Hkv / Hq) (contiguous GQA groups).  Padded rows output zeros.

Keys of request b are ordered [soft prompt | cached prefix 0..L_b | block
rows 0..n_q_b) and the dense visibility matrix of ``mask.dense_visibility``
selects among them.  Cache slots at or past L_b and padded block rows hold
no data (the generators fill them with NaN), and no valid row can see them,
so they are left out of the key list before any arithmetic.
"""

from typing import Optional, Sequence, Tuple

import numpy as np

from .bf16 import as_f64
from .mask import dense_visibility


def verify_attention(q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft, v_soft,
                     attn_parent, sp_flag, n_q, dtype: str, scale: Optional[float] = None,
                     requests: Optional[Sequence[int]] = None,
                     rows: Optional[Sequence[int]] = None,
                     block_vis=None) -> Tuple[np.ndarray, np.ndarray]:
    """Return (out [B, Tq, Hq, D], lse [B, Tq, Hq]) in float64.

    ``requests`` / ``rows`` restrict the computation to a subset (entries
    not computed are NaN), for sampled checks of large workloads.
    ``block_vis`` (bool [B, Tq, Tq]) gives the block keys each row sees in
    place of ``attn_parent`` (multi-stream rows, ``msa.msa_block_visibility``).
    """
    B, Tq, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    S = 0 if k_soft is None else k_soft.shape[0]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((B, Tq, Hq, D), np.nan)
    lse = np.full((B, Tq, Hq), np.nan)
    soft_k = as_f64(k_soft, dtype) if S else np.zeros((0, Hkv, D))
    soft_v = as_f64(v_soft, dtype) if S else np.zeros((0, Hkv, D))
    for b in (range(B) if requests is None else requests):
        L = int(cache_len[b])
        nq = int(n_q[b])
        sp_row = None if sp_flag is None else sp_flag[b]
        M = dense_visibility(None if attn_parent is None else attn_parent[b], sp_row, nq, S, L,
                             None if block_vis is None else block_vis[b])   # [Tq, S+L+Tq]
        M = M[:, : S + L + nq]                                        # drop padded block keys
        K = np.concatenate([soft_k, as_f64(k_cache[b, :L], dtype), as_f64(k_blk[b, :nq], dtype)])
        V = np.concatenate([soft_v, as_f64(v_cache[b, :L], dtype), as_f64(v_blk[b, :nq], dtype)])
        row_list = range(Tq) if rows is None else rows
        for r in row_list:
            if r >= nq:
                out[b, r] = 0.0
                lse[b, r] = -np.inf
                continue
            vis = np.nonzero(M[r])[0]
            qr = as_f64(q[b, r], dtype)                               # [Hq, D]
            for h in range(Hkv):
                Kh = K[vis, h, :]
                Vh = V[vis, h, :]
                for j in range(Hq):
                    if (j * Hkv) // Hq != h:
                        continue
                    s = (Kh @ qr[j]) * scale
                    m = s.max()
                    w = np.exp(s - m)
                    l = w.sum()
                    out[b, r, j] = (w @ Vh) / l
                    lse[b, r, j] = m + np.log(l)
    return out, lse
