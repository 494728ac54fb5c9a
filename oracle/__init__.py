"""Plain fp64 CPU oracle of the speculative verification step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(no kernels, headers, helpers, tables or pre/post-processing) and imports
nothing from it; both sides are fed by the seeded generators, which hold none
of the verification arithmetic.

Every function is the plain definition of what the pages describe, computed
the slow, obvious way (explicit dense masks, per-request loops, fp64):

* ``mask``       -- which keys each query row of the speculative block may see
                    (Lookahead Attention section 3.1; Speculative Streaming
                    Equation 4 and its prose; ConFu key design 1).
* ``attention``  -- softmax(q k^T / sqrt(d)) v over the visible keys
                    (Speculative Streaming Equation 1).
* ``acceptance`` -- per-node greedy target token (vocabulary argmax) and the
                    longest accepted root-to-node path found depth-first
                    (Speculative Streaming, the verification step;
                    Lookahead Attention section 2.4); also with explicit
                    verification rows, an explicit root and the correction
                    token (the same verification step and the tree draft
                    construction before it).
* ``commit``     -- keep the accepted nodes' K/V in the cache, drop the rest
                    (Lookahead Attention section 3.2; Speculative Streaming,
                    tree pruning and its lazy garbage collection).
* ``msa``        -- the multi-stream rows of a tree draft and what each sees
                    (Speculative Streaming, Equations 1, 2 and 4, and its
                    batching with speculative streams).
* ``prob_accept`` -- acceptance by the target's probability of each draft:
                    Lookahead Attention's threshold rule and Speculative
                    Streaming's soft matching with given uniforms.
* ``draft``      -- the next tree draft: per-stream top-k tokens of the last
                    accepted node's streams, linked stream to stream under the
                    correction token (Speculative Streaming, tree draft
                    construction and parallel new draft generation).

Pins: every function is checked by ``tests/test_oracle_*.py`` against things
other than itself -- the 7x7 mask drawn on the Lookahead Attention page (after
the reading that fixes its transposition), the tree sizes printed on the
Speculative Streaming page, closed forms, ``torch`` scaled-dot-product
attention in float64, brute-force enumeration and invariants.  No function
here is "parity unpinned".
"""

from .bf16 import bf16_bits_to_f64, as_f64
from .mask import (ancestor_rows, block_visibility, soft_visibility, dense_visibility,
                   pack_bits, build_mask)
from .attention import verify_attention
from .acceptance import greedy_tokens, accept_request, argmax_accept, accept_request_rows, argmax_accept_rows
from .commit import commit_kv
from .msa import msa_row, tree_path, msa_block_visibility, build_msa_mask
from .draft import topk_tokens, draft_tree, next_draft
from .prob_accept import (MODE_THRESHOLD, MODE_SOFT, target_prob, node_probs, decide, scan_accepted,
                          prob_accept)

__all__ = [
    "bf16_bits_to_f64", "as_f64",
    "ancestor_rows", "block_visibility", "soft_visibility", "dense_visibility",
    "pack_bits", "build_mask",
    "verify_attention",
    "greedy_tokens", "accept_request", "argmax_accept", "accept_request_rows", "argmax_accept_rows",
    "commit_kv",
    "msa_row", "tree_path", "msa_block_visibility", "build_msa_mask",
    "topk_tokens", "draft_tree", "next_draft",
    "MODE_THRESHOLD", "MODE_SOFT", "target_prob", "node_probs", "decide", "scan_accepted", "prob_accept",
]
