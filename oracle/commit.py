"""KV commit of the accepted path (oracle side).

Accepted tokens keep their key/value rows and everything else from the
speculative block is dropped: Lookahead Attention section 3.2 discards the
lookahead rows after the pass, and Speculative Streaming keeps the accepted
main-stream tokens while pruned or rejected entries are garbage-collected
after the step.  The accepted rows are appended in path order: the node at
depth d+1 goes to cache slot L + d.  Rows that would land at or past the
cache capacity are not written, and the new length counts only rows
written.  Every other cache slot is left untouched.  (The Lookahead caller
commits nothing; the operation itself is the same for every page.)
"""

import numpy as np


def commit_kv(k_cache, v_cache, cache_len, k_blk, v_blk, out_len, out_path):
    """Return (k_cache', v_cache', cache_len') as new arrays; inputs are not modified."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    B, lmax = kc.shape[0], kc.shape[1]
    new_len = np.array(cache_len, dtype=np.int32, copy=True)
    for b in range(B):
        L = int(cache_len[b])
        written = 0
        for d in range(int(out_len[b])):
            if L + d >= lmax:
                break
            row = int(out_path[b, d])
            kc[b, L + d] = k_blk[b, row]
            vc[b, L + d] = v_blk[b, row]
            written += 1
        new_len[b] = L + written
    return kc, vc, new_len
