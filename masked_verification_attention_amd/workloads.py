"""Seeded synthetic inputs for the speculative verification step.

This module only draws inputs.  It holds none of the verification arithmetic:
no visibility mask, no attention, no argmax, no acceptance scan and no commit.
Both the HIP path (through the tests and the benchmark) and the CPU oracle are
fed from the arrays it returns, so the two sides always see identical bits.

Workload shapes follow the three pages this library implements:

* Lookahead Attention (LA), "Lookahead Attention: Self-Speculative
  Verification via Parallel Token Proposals", sections 2.1, 3.1 and 3.3:
  k lookahead rows that see the whole prefix plus themselves, padded to one
  k per batch.
* ConFu, "ConFu: Contemplate the Future for Better Speculative Sampling",
  key design 1: a draft tree of T nodes plus one contemplate token per node
  (2T query rows) and a learned soft prompt placed in the KV cache that only
  contemplate tokens may see (16 soft rows by default, limitations section).
* Speculative Streaming (SS), "Speculative Streaming: Fast LLM Inference
  without Auxiliary Models", tree draft and Equation 4: each node sees its
  ancestors; several candidate streams that are causal within themselves.
  Its multi-stream form ("msa_tree"): the tree draft of top-k tokens per
  speculative stream -- a complete k-ary tree of depth gamma, 1 + sum k^g
  nodes, flattened level by level -- with every node carrying its main stream
  and gamma speculative streams (Equation 2 and the batching paragraph).

Value recipe: float32 standard normal draws, rounded to bfloat16 with
round-to-nearest-even (bf16 tensors are returned as their uint16 bit
patterns); fp32 workloads keep the float32 draws.  Cache slots past a
request's length and the rows of padded queries are filled with NaN canaries,
so that any read of them poisons the result.

Greedy drafts: a node whose draft should match the target gets a planted
maximum -- the drafted token's logit is set to 8.0, which no bf16 standard
normal draw reaches in practice -- so the generator never has to compute an
argmax.  Other nodes get a uniformly random token, which may still equal the
row's argmax by chance; the oracle, not the coin, decides acceptance.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import numpy as np

# Planted logit value for a matching draft (exactly representable in bf16).
PLANTED_LOGIT = 8.0
# Bit patterns of the NaN canaries.
BF16_NAN = np.uint16(0x7FC0)
F32_NAN = np.float32(np.nan)


@dataclass(frozen=True)
class VerifyConfig:
    """One verification-step workload (one layer of attention, one LM-head output)."""

    name: str
    B: int                      # requests in the batch
    Hq: int                     # query heads
    Hkv: int                    # key/value heads (GQA groups of Hq // Hkv)
    D: int                      # head dimension
    dtype: str                  # "f32" or "bf16" for q, k, v, soft prompt
    L: Tuple[int, int]          # prefix length range, inclusive (lo == hi: fixed)
    S: int                      # soft-prompt KV rows (0 = none)
    structure: str              # "la_cache", "la_full", "confu_tree", "stream_chains", "msa_tree"
    T: int                      # acceptance nodes per request
    V: int                      # vocabulary size
    logits_dtype: str           # "f32" or "bf16"
    accept_p: float = 0.8       # per-node probability that the draft is the planted argmax
    exact_accepts: Optional[int] = None  # if set: exactly this many planted nodes (random subset)
    depth_cap: int = 6          # tree depth cap (confu_tree)
    chain_len: int = 4          # nodes per chain (stream_chains)
    n_lookahead: int = 0        # la_full: k lookahead rows after the n = L[0] originals
    gamma: int = 0              # msa_tree: speculative streams per node (tree depth)
    branch: int = 0             # msa_tree: tokens drawn per stream position (children per node)
    seed: int = 1000

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def Tq(self) -> int:
        """Query rows of the speculative block (attention rows per request)."""
        if self.structure == "confu_tree":
            return 2 * self.T
        if self.structure == "la_full":
            return self.L[0] + self.n_lookahead
        if self.structure == "msa_tree":
            return (1 + self.gamma) * self.T
        return self.T

    @property
    def max_depth(self) -> int:
        """Longest possible accepted path for this structure."""
        if self.structure == "confu_tree":
            return self.depth_cap
        if self.structure == "stream_chains":
            return self.chain_len
        if self.structure == "msa_tree":
            return self.gamma + 1          # the root (accepted unchecked) and gamma levels
        return self.T

    def with_(self, **kw) -> "VerifyConfig":
        return replace(self, **kw)


# The workloads (C1..C5 here, C6 below).  Values the workload descriptions
# leave open are readings: C3 accept probability 0.8, C4 soft rows 16 and
# depth cap 6, C5 as 32 fixed chains of 4.
CONFIGS: Dict[str, VerifyConfig] = {
    "c1_tiny_la": VerifyConfig(
        name="c1_tiny_la", B=1, Hq=2, Hkv=2, D=64, dtype="f32", L=(128, 128), S=0,
        structure="la_cache", T=4, V=1000, logits_dtype="f32", exact_accepts=3, seed=1000),
    "c2_la_7b": VerifyConfig(
        name="c2_la_7b", B=8, Hq=32, Hkv=32, D=128, dtype="bf16", L=(512, 2048), S=0,
        structure="la_cache", T=8, V=32000, logits_dtype="bf16", accept_p=0.85, seed=1001),
    "c3_confu_8b": VerifyConfig(
        name="c3_confu_8b", B=16, Hq=32, Hkv=8, D=128, dtype="bf16", L=(4096, 4096), S=16,
        structure="confu_tree", T=30, V=128256, logits_dtype="bf16", accept_p=0.8,
        depth_cap=6, seed=1002),
    "c4_tree_3b": VerifyConfig(
        name="c4_tree_3b", B=32, Hq=24, Hkv=8, D=128, dtype="bf16", L=(2048, 8192), S=16,
        structure="confu_tree", T=60, V=128256, logits_dtype="bf16", accept_p=0.8,
        depth_cap=6, seed=1003),
    "c5_stream_70b": VerifyConfig(
        name="c5_stream_70b", B=16, Hq=64, Hkv=8, D=128, dtype="bf16", L=(16384, 16384), S=0,
        structure="stream_chains", T=128, V=128256, logits_dtype="bf16", accept_p=0.75,
        chain_len=4, seed=1004),
}

# Speculative Streaming's multi-stream verification (the tree-draft ablation of
# its Figure 5: gamma = 3, k = 3 unpruned, 40 nodes, 160 MSA rows) on an
# OPT-1.3B-shaped layer (32 heads of 64, no GQA, 50272-token vocabulary); the
# prefix lengths are a reading (the page's tasks have prompts of a few hundred
# tokens).
CONFIGS["c6_msa_1b"] = VerifyConfig(
    name="c6_msa_1b", B=8, Hq=32, Hkv=32, D=64, dtype="bf16", L=(256, 1024), S=0,
    structure="msa_tree", T=40, V=50272, logits_dtype="bf16", accept_p=0.8,
    gamma=3, branch=3, seed=1006)

# The full form of the tiny LA workload: the n = 128 original tokens are part of
# the block as a causal chain and the k = 4 lookahead rows hang off the last one,
# so the block mask is exactly LA's [causal | 1; 0 | diagonal] layout.
CONFIGS["c1_tiny_la_full"] = CONFIGS["c1_tiny_la"].with_(
    name="c1_tiny_la_full", structure="la_full", n_lookahead=4, L=(128, 128))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Inputs must be finite (the draws are).  This is a storage conversion of the
    synthetic draws, not part of the verification arithmetic.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite floats are below 0x7F800000 in magnitude bits, so the sum cannot wrap
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def _values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _nan_fill(a: np.ndarray, dtype: str):
    return BF16_NAN if dtype == "bf16" else F32_NAN


def random_forest(rng: np.random.Generator, T: int, depth_cap: int) -> np.ndarray:
    """Random recursive forest under an implicit root (the last committed token).

    Node v's parent is uniform over {-1} and the earlier nodes whose depth is
    below the cap (a node with parent -1 has depth 1).  Parents always precede
    children, so the array is in topological order.
    """
    parent = np.full(T, -1, dtype=np.int32)
    depth = np.zeros(T, dtype=np.int32)
    for v in range(T):
        choices = [-1] + [u for u in range(v) if depth[u] < depth_cap]
        parent[v] = choices[int(rng.integers(0, len(choices)))]
        depth[v] = 1 if parent[v] < 0 else depth[parent[v]] + 1
    return parent


def chain_forest(n_chains: int, chain_len: int) -> np.ndarray:
    """n_chains independent chains of chain_len nodes, each causal within itself."""
    parent = np.empty(n_chains * chain_len, dtype=np.int32)
    for c in range(n_chains):
        for i in range(chain_len):
            parent[c * chain_len + i] = -1 if i == 0 else c * chain_len + i - 1
    return parent


def kary_tree(branch: int, gamma: int) -> np.ndarray:
    """Complete branch-ary tree of depth gamma, flattened level by level.

    Node 0 is the root; the children of node p are branch*p + 1 .. branch*p +
    branch, so parents precede children.  1 + sum_{g=1..gamma} branch^g nodes.
    """
    n = sum(branch ** g for g in range(gamma + 1))
    parent = np.full(n, -1, dtype=np.int32)
    for v in range(1, n):
        parent[v] = (v - 1) // branch
    return parent


def generate(cfg: VerifyConfig, seed: Optional[int] = None, *, B: Optional[int] = None,
             L: Optional[Tuple[int, int]] = None, n_q: Optional[np.ndarray] = None,
             n_nodes: Optional[np.ndarray] = None,
             with_logits: bool = True) -> Dict[str, np.ndarray]:
    """Draw one full set of inputs for ``cfg``.

    Draw order is fixed: lengths, structure, q, k_cache, v_cache, k_blk, v_blk,
    k_soft, v_soft, logits, accept coins, random tokens.  ``B`` and ``L``
    override the batch and the prefix range (smaller parity cases);
    ``n_q`` overrides the valid query rows per request (ragged padding tests;
    padded rows are the last Tq - n_q rows).  For "msa_tree", ``n_nodes``
    keeps only the first n_nodes[b] tree nodes of request b (a pruned tree;
    its n_nodes[b] * (1 + gamma) rows are valid) and ``n_q`` is not accepted.
    """
    if B is not None:
        cfg = cfg.with_(B=B)
    if L is not None:
        cfg = cfg.with_(L=L)
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    Bn, Tq, T = cfg.B, cfg.Tq, cfg.T

    # -- lengths
    lo, hi = cfg.L
    if cfg.structure == "la_full":
        cache_len = np.zeros(Bn, dtype=np.int32)
    else:
        cache_len = rng.integers(lo, hi + 1, size=Bn, dtype=np.int64).astype(np.int32)
    lmax = int(cache_len.max()) + Tq

    # -- structure
    attn_parent = np.full((Bn, Tq), -1, dtype=np.int32)
    sp_flag = np.zeros((Bn, Tq), dtype=np.uint8)
    # acceptance arrays and logit rows: one per node; for msa_tree one per block
    # row (the LM head runs over every row: main rows verify, the speculative
    # rows of the last accepted node draft the next tree) with the nodes first
    Ta = Tq if cfg.structure == "msa_tree" else T
    acc_parent = np.full((Bn, Ta), -1, dtype=np.int32)
    node_row = np.arange(T, dtype=np.int32)  # block row of node v
    tree_parent = None
    if cfg.structure == "msa_tree":
        if n_q is not None:
            raise ValueError("msa_tree takes n_nodes, not n_q")
        tree = kary_tree(cfg.branch, cfg.gamma)
        if len(tree) != T:
            raise ValueError(f"T = {T} but a complete {cfg.branch}-ary tree of depth {cfg.gamma} "
                             f"has {len(tree)} nodes")
        tree_parent = np.tile(tree, (Bn, 1))
        acc_parent[:, :T] = tree_parent
        nn = np.full(Bn, T, dtype=np.int32) if n_nodes is None else np.asarray(n_nodes, dtype=np.int32)
        if nn.shape != (Bn,) or nn.min() < 0 or nn.max() > T:
            raise ValueError("n_nodes out of range")
        n_q = nn * (1 + cfg.gamma)
    elif n_nodes is not None:
        raise ValueError("n_nodes is only taken by msa_tree")
    for b in range(Bn):
        if cfg.structure == "msa_tree":
            continue
        if cfg.structure == "la_cache":
            acc_parent[b] = np.arange(-1, T - 1, dtype=np.int32)
        elif cfg.structure == "la_full":
            n = cfg.L[0]
            attn_parent[b, :n] = np.arange(-1, n - 1, dtype=np.int32)
            attn_parent[b, n:] = n - 1
            acc_parent[b] = np.arange(-1, T - 1, dtype=np.int32)
        elif cfg.structure == "confu_tree":
            par = random_forest(rng, T, cfg.depth_cap)
            attn_parent[b, :T] = par
            attn_parent[b, T:] = np.arange(T, dtype=np.int32)
            sp_flag[b, T:] = 1
            acc_parent[b] = par
        elif cfg.structure == "stream_chains":
            par = chain_forest(T // cfg.chain_len, cfg.chain_len)
            attn_parent[b] = par
            acc_parent[b] = par
        else:
            raise ValueError(cfg.structure)
    if cfg.structure == "la_full":
        node_row = np.arange(cfg.L[0], cfg.L[0] + T, dtype=np.int32)
    if n_q is None:
        n_q = np.full(Bn, Tq, dtype=np.int32)
    n_q = np.asarray(n_q, dtype=np.int32)
    if cfg.structure == "msa_tree":
        n_nodes = (n_q // (1 + cfg.gamma)).astype(np.int32)
    else:
        n_nodes = np.full(Bn, T, dtype=np.int32)
    if cfg.structure in ("la_cache", "stream_chains"):
        n_nodes = np.minimum(n_nodes, n_q).astype(np.int32)

    # -- values
    D, Hq, Hkv, dt = cfg.D, cfg.Hq, cfg.Hkv, cfg.dtype
    q = _values(rng, (Bn, Tq, Hq, D), dt)
    k_cache = _values(rng, (Bn, lmax, Hkv, D), dt)
    v_cache = _values(rng, (Bn, lmax, Hkv, D), dt)
    k_blk = _values(rng, (Bn, Tq, Hkv, D), dt)
    v_blk = _values(rng, (Bn, Tq, Hkv, D), dt)
    k_soft = _values(rng, (cfg.S, Hkv, D), dt)
    v_soft = _values(rng, (cfg.S, Hkv, D), dt)
    nan = _nan_fill(q, dt)
    for b in range(Bn):
        k_cache[b, cache_len[b]:] = nan
        v_cache[b, cache_len[b]:] = nan
        q[b, n_q[b]:] = nan
        k_blk[b, n_q[b]:] = nan
        v_blk[b, n_q[b]:] = nan

    out = dict(
        cache_len=cache_len, attn_parent=attn_parent, sp_flag=sp_flag, n_q=n_q,
        acc_parent=acc_parent, n_nodes=n_nodes, node_row=node_row,
        q=q, k_cache=k_cache, v_cache=v_cache, k_blk=k_blk, v_blk=v_blk,
        k_soft=k_soft, v_soft=v_soft,
    )
    if tree_parent is not None:
        out["tree_parent"] = tree_parent

    # -- logits and drafts
    if with_logits:
        V = cfg.V
        logits = _values(rng, (Bn, Ta, V), cfg.logits_dtype)
        if cfg.exact_accepts is not None:
            coins = np.zeros((Bn, T), dtype=bool)
            for b in range(Bn):
                pick = rng.permutation(T)[: cfg.exact_accepts]
                coins[b, pick] = True
        else:
            coins = rng.random(size=(Bn, T)) < cfg.accept_p
        tokens = np.zeros((Bn, Ta), dtype=np.int32)
        tokens[:, :T] = rng.integers(0, V, size=(Bn, T), dtype=np.int64).astype(np.int32)
        planted = (f32_to_bf16_bits(np.array([PLANTED_LOGIT], np.float32))[0]
                   if cfg.logits_dtype == "bf16" else np.float32(PLANTED_LOGIT))
        for b in range(Bn):
            for v in range(T):
                if not coins[b, v]:
                    continue
                if cfg.structure == "msa_tree":
                    # a node is checked against its parent's main-stream output
                    if tree_parent[b, v] >= 0:
                        logits[b, tree_parent[b, v], tokens[b, v]] = planted
                else:
                    logits[b, v, tokens[b, v]] = planted
        out.update(logits=logits, draft_tok=tokens, planted=coins)
    return out


def nbytes_of(inputs: Dict[str, np.ndarray]) -> int:
    return sum(int(a.nbytes) for a in inputs.values())
