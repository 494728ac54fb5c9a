"""Device buffers for one verification step and the calls that run it.

Uploads one seeded workload (``workloads.generate``) to HBM as torch tensors,
allocates every output, and runs the four entry points on one stream:
spec_build_mask -> spec_verify_attn -> spec_argmax_accept_commit (the fused
form of spec_argmax_accept + spec_commit_kv, which are also exposed); multi-
stream workloads use spec_build_msa_mask, verification rows and
spec_draft_tree for the next draft.
This module only moves memory and marshals arguments; all arithmetic runs in
the HIP kernels.  torch supplies the device memory and the stream.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import binding as bd
from .workloads import VerifyConfig

DTYPE_CODE = {"f32": bd.SPEC_F32, "bf16": bd.SPEC_BF16}

# SPEC_V_TILE32: a 32-key tile is [D/16][4][16][8] (head-dim block, key group g, head dim in the
# block, key slot e); key k of the tile is at group/slot position 8 g + e = VT_POS_OF[k]
VT_POS_OF = [8 * ((k % 16) // 4) + k % 4 + 4 * (k // 16) for k in range(32)]
VT_KEY_AT = [VT_POS_OF.index(p) for p in range(32)]


def to_device(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload a generator array; bf16 arrays arrive as uint16 bit patterns."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    if dtype == "i32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)
    if dtype == "u8":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(device)
    raise ValueError(dtype)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy with the exact bits (bf16 as uint16, int32 words as uint32)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class VerifyStep:
    """One verification step's device state for a workload."""

    def __init__(self, cfg: VerifyConfig, x: Dict[str, np.ndarray], device="cuda", kv_splits: int = 0,
                 scale: float = 0.0, max_depth: Optional[int] = None, layout: str = "blhd",
                 accept: str = "greedy", threshold: float = 1e-3, draft_prob=None, uniform=None,
                 fused_mask: Optional[bool] = None, out_dtype: str = "f32"):
        """``layout`` of the K/V cache in HBM: "blhd" = [B, lmax, Hkv, D] (token-major, the
        generator's order), "bhld" = [B, Hkv, lmax, D] (head-major), or "bhld_vt" = K head-major
        and V in transposed 32-key tiles [B, Hkv, lmax/32, D, 32] (SPEC_V_TILE32; lmax is
        rounded up to a multiple of 32, the extra slots holding NaN like every unused slot).
        The strides and V layout go to the library through the descriptor; ``cache_host()``
        returns the cache in the generator's order and capacity either way.  ``accept`` selects the acceptance rule
        of ``run()``: "greedy" (hard matching), "threshold" (target probability above
        ``threshold``) or "soft" (soft matching with the given ``draft_prob`` and
        ``uniform`` arrays [B, T]).  ``fused_mask``: ``run()`` builds the block mask inside the
        attention launch (spec_verify_attn_tree) instead of with spec_build_mask first; by
        default wherever it applies (bf16 inputs); multi-stream workloads use
        spec_verify_attn_msa, which does not write n_q (build_mask() does).  ``out_dtype``
        of the attention output: "f32", or "bf16" (bf16 inputs only: the float32 result
        rounded to nearest even)."""
        self.cfg = cfg
        self.device = torch.device(device)
        dt = cfg.dtype
        dev = self.device
        self.B, self.Tq = x["q"].shape[0], x["q"].shape[1]
        self.T = x["acc_parent"].shape[1]
        self.W = (self.Tq + 31) // 32
        self.lmax = x["k_cache"].shape[1]
        self.max_depth = int(max_depth if max_depth is not None else min(cfg.max_depth, bd.SPEC_MAX_DEPTH))
        self.q = to_device(x["q"], dt, dev)
        if layout not in ("blhd", "bhld", "bhld_vt"):
            raise ValueError(layout)
        self.layout = layout
        self.lmax_gen = self.lmax
        self.k_cache = to_device(x["k_cache"], dt, dev)
        self.v_cache = to_device(x["v_cache"], dt, dev)
        if layout == "bhld_vt":
            pad = (-self.lmax) % 32
            if pad:
                fill = torch.full((self.B, pad) + tuple(self.k_cache.shape[2:]), float("nan"),
                                  dtype=self.k_cache.dtype, device=dev)
                self.k_cache = torch.cat([self.k_cache, fill], dim=1)
                self.v_cache = torch.cat([self.v_cache, fill], dim=1)
                self.lmax += pad
        if layout in ("bhld", "bhld_vt"):
            self.k_cache = self.k_cache.permute(0, 2, 1, 3).contiguous()
            self.v_cache = self.v_cache.permute(0, 2, 1, 3).contiguous()
        if layout == "bhld_vt":
            B_, H_, L_, D_ = self.v_cache.shape
            tiles = self.v_cache.reshape(B_, H_, L_ // 32, 32, D_)[:, :, :, VT_KEY_AT, :]   # [.., pos, D]
            tiles = tiles.reshape(B_, H_, L_ // 32, 4, 8, D_ // 16, 16)                     # [.., g, e, db, r]
            self.v_cache = tiles.permute(0, 1, 2, 5, 3, 6, 4).contiguous()                 # [.., db, g, r, e]
        self.k_blk = to_device(x["k_blk"], dt, dev)
        self.v_blk = to_device(x["v_blk"], dt, dev)
        self.k_soft = to_device(x["k_soft"], dt, dev) if cfg.S else None
        self.v_soft = to_device(x["v_soft"], dt, dev) if cfg.S else None
        self.cache_len = to_device(x["cache_len"], "i32", dev)
        self.attn_parent = to_device(x["attn_parent"], "i32", dev)
        self.sp_flag = to_device(x["sp_flag"], "u8", dev)
        self.n_q = to_device(x["n_q"], "i32", dev)
        self.acc_parent = to_device(x["acc_parent"], "i32", dev)
        self.n_nodes = to_device(x["n_nodes"], "i32", dev)
        self.draft_tok = to_device(x["draft_tok"], "i32", dev) if "draft_tok" in x else None
        self.logits = to_device(x["logits"], cfg.logits_dtype, dev) if "logits" in x else None
        self.V = x["logits"].shape[2] if "logits" in x else cfg.V
        # multi-stream rows: the mask comes from the tree, and a node is verified by its
        # parent's main-stream row; main rows are the first rows of the block, so the
        # acceptance parents (the tree, padded with -1 to one entry per row) are also
        # the verification rows
        self.msa = cfg.structure == "msa_tree"
        self.tree_parent = to_device(x["tree_parent"], "i32", dev) if self.msa else None
        can_fuse = cfg.dtype == "bf16"
        if fused_mask and not can_fuse:
            raise ValueError("the fused mask build needs bf16 inputs")
        self.fused_mask = can_fuse if fused_mask is None else bool(fused_mask)

        i32 = dict(dtype=torch.int32, device=dev)
        self.mask_bits = torch.zeros(self.B, self.Tq, self.W, **i32)
        self.sp_bits = torch.zeros(self.B, self.W, **i32)
        if out_dtype not in ("f32", "bf16"):
            raise ValueError(out_dtype)
        self.out_dtype = out_dtype
        self.out = torch.empty(self.B, self.Tq, cfg.Hq, cfg.D,
                               dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32, device=dev)
        self.lse = torch.empty(self.B, self.Tq, cfg.Hq, dtype=torch.float32, device=dev)
        self.argmax = torch.empty(self.B, self.T, **i32)
        self.out_len = torch.empty(self.B, **i32)
        self.out_path = torch.empty(self.B, self.max_depth, **i32)
        self.out_bonus = torch.empty(self.B, **i32)
        if accept not in ("greedy", "threshold", "soft"):
            raise ValueError(accept)
        self.accept, self.threshold = accept, float(threshold)
        self.out_prob = torch.empty(self.B, self.T, dtype=torch.float32, device=dev)
        self.draft_prob = self.uniform = None
        if accept == "soft":
            if draft_prob is None or uniform is None:
                raise ValueError("soft matching needs draft_prob and uniform")
            self.draft_prob = to_device(np.asarray(draft_prob, np.float32), "f32", dev)
            self.uniform = to_device(np.asarray(uniform, np.float32), "f32", dev)
        if self.msa:
            # the next draft: k tokens per stream of the new root, a complete k-ary tree
            k, g = cfg.branch, cfg.gamma
            self.draft_N = sum(k ** e for e in range(g + 1))
            self.next_topk = torch.empty(self.B, max(g, 1), k, **i32)
            self.next_tok = torch.empty(self.B, self.draft_N, **i32)
            self.next_parent = torch.empty(self.B, self.draft_N, **i32)
            self.next_n = torch.empty(self.B, **i32)
        self.cache_len_out = torch.empty(self.B, **i32)

        Hkv, D = cfg.Hkv, cfg.D
        strides = ((self.lmax * Hkv * D, Hkv * D, D) if layout == "blhd"
                   else (Hkv * self.lmax * D, D, self.lmax * D))
        self.desc = bd.make_desc(self.B, self.Tq, cfg.Hq, Hkv, D, cfg.S, DTYPE_CODE[dt], self.lmax,
                                 strides, scale=scale, kv_splits=kv_splits,
                                 v_layout=bd.SPEC_V_TILE32 if layout == "bhld_vt" else bd.SPEC_V_ROWS,
                                 out_dtype=DTYPE_CODE[out_dtype])
        self.ws_bytes = bd.spec_verify_attn_workspace(self.desc)
        self.workspace = (torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
                          if self.ws_bytes else None)

    def cache_host(self, full: bool = False):
        """(k_cache, v_cache) as host arrays in the generator's [B, lmax, Hkv, D] order
        (``full``: with the slots added to round lmax up to a multiple of 32, if any)."""
        k, v = self.k_cache, self.v_cache
        if self.layout == "bhld_vt":
            B_, H_, T_, DB_, _, _, _ = v.shape
            v = v.permute(0, 1, 2, 4, 6, 3, 5).reshape(B_, H_, T_, 32, DB_ * 16)             # [.., pos, D]
            v = v[:, :, :, VT_POS_OF, :].reshape(B_, H_, T_ * 32, DB_ * 16)
        if self.layout in ("bhld", "bhld_vt"):
            k, v = k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)
        if not full:
            k, v = k[:, :self.lmax_gen], v[:, :self.lmax_gen]
        return to_host_bits(k.contiguous()), to_host_bits(v.contiguous())

    # -- the four entry points
    def build_mask(self, stream=None):
        if self.msa:
            bd.spec_build_msa_mask(self.tree_parent, self.n_nodes, self.B, self.tree_parent.shape[1],
                                   self.cfg.gamma, self.Tq,
                                   self.mask_bits, self.sp_bits, self.n_q, stream)
            return
        bd.spec_build_mask(self.attn_parent, self.sp_flag, self.n_q, self.B, self.Tq, self.mask_bits,
                           self.sp_bits, stream)

    def attention(self, stream=None, out=None, lse="self"):
        bd.spec_verify_attn(self.desc, self.q, self.k_cache, self.v_cache, self.cache_len, self.k_blk,
                            self.v_blk, self.k_soft, self.v_soft, self.mask_bits,
                            self.sp_bits if self.cfg.S else self.sp_bits, self.n_q,
                            self.out if out is None else out, self.lse if lse == "self" else lse,
                            self.workspace, self.ws_bytes, stream)

    def attention_tree(self, stream=None, out=None, lse="self"):
        """Mask build and attention in one launch (spec_verify_attn_tree, or spec_verify_attn_msa
        for multi-stream rows); mask_bits, sp_bits and n_q are neither read nor written."""
        o, l = self.out if out is None else out, self.lse if lse == "self" else lse
        if self.msa:
            bd.spec_verify_attn_msa(self.desc, self.q, self.k_cache, self.v_cache, self.cache_len, self.k_blk,
                                    self.v_blk, self.k_soft, self.v_soft, self.tree_parent, self.n_nodes,
                                    self.tree_parent.shape[1], self.cfg.gamma, o, l, self.workspace,
                                    self.ws_bytes, stream)
            return
        bd.spec_verify_attn_tree(self.desc, self.q, self.k_cache, self.v_cache, self.cache_len, self.k_blk,
                                 self.v_blk, self.k_soft, self.v_soft, self.attn_parent, self.sp_flag, self.n_q,
                                 o, l, self.workspace, self.ws_bytes, stream)

    def argmax_accept(self, stream=None):
        if self.msa:
            bd.spec_argmax_accept_rows(self.logits, DTYPE_CODE[self.cfg.logits_dtype], self.B, self.T, self.V,
                                       self.n_nodes, self.draft_tok, self.acc_parent, self.acc_parent,
                                       self.max_depth, self.argmax, self.out_len, self.out_path,
                                       self.out_bonus, stream)
            return
        bd.spec_argmax_accept(self.logits, DTYPE_CODE[self.cfg.logits_dtype], self.B, self.T, self.V,
                              self.n_nodes, self.draft_tok, self.acc_parent, self.max_depth, self.argmax,
                              self.out_len, self.out_path, stream)

    def commit(self, stream=None, in_place=False):
        bd.spec_commit_kv(self.desc, self.k_cache, self.v_cache, self.cache_len,
                          self.cache_len if in_place else self.cache_len_out, self.k_blk, self.v_blk,
                          self.out_len, self.out_path, self.max_depth, stream)

    def accept_commit(self, stream=None, in_place=False):
        """Argmax, acceptance and commit in two launches (spec_argmax_accept_commit); multi-stream
        workloads verify each node against its parent's row and return the correction token."""
        bd.spec_argmax_accept_commit(self.logits, DTYPE_CODE[self.cfg.logits_dtype], self.T, self.V, self.n_nodes,
                                     self.draft_tok, self.acc_parent, self.acc_parent if self.msa else None,
                                     self.max_depth, self.argmax, self.out_len, self.out_path, self.out_bonus,
                                     self.desc, self.k_cache, self.v_cache, self.cache_len,
                                     self.cache_len if in_place else self.cache_len_out, self.k_blk, self.v_blk,
                                     stream)

    def prob_accept(self, stream=None):
        """Acceptance by the target's probability of each draft (spec_prob_accept)."""
        mode = bd.SPEC_ACCEPT_THRESHOLD if self.accept == "threshold" else bd.SPEC_ACCEPT_SOFT
        bd.spec_prob_accept(self.logits, DTYPE_CODE[self.cfg.logits_dtype], self.B, self.T, self.V, self.n_nodes,
                            self.draft_tok, self.acc_parent, self.acc_parent if self.msa else None,
                            self.max_depth, mode, self.threshold, self.draft_prob, self.uniform, self.argmax,
                            self.out_prob, self.out_len, self.out_path, self.out_bonus, stream)

    def draft(self, stream=None):
        """The next tree draft from the new root's speculative streams (multi-stream workloads)."""
        bd.spec_draft_tree(self.logits, DTYPE_CODE[self.cfg.logits_dtype], self.B, self.Tq, self.V, self.n_nodes,
                           self.out_len, self.out_path, self.max_depth, self.out_bonus, self.cfg.gamma,
                           self.cfg.branch, self.next_topk, self.next_tok, self.next_parent, self.next_n, stream)

    def tail(self, stream=None):
        """Everything after the attention: greedy tokens, acceptance and commit (and the
        next draft of multi-stream workloads)."""
        if self.accept == "greedy":
            self.accept_commit(stream)
        else:
            self.prob_accept(stream)
            self.commit(stream)
        if self.msa:
            self.draft(stream)

    def run(self, stream=None):
        """One pass of the whole hot path (the cache length is not advanced in place);
        multi-stream workloads also draft the next tree in the same pass."""
        if self.fused_mask:
            self.attention_tree(stream)
        else:
            self.build_mask(stream)
            self.attention(stream)
        self.tail(stream)

    def prepare(self, stream=None):
        """The calls of run() with their arguments converted once, as three lists of
        zero-argument callables (mask, attention, tail) on ``stream``."""
        P = bd.Prepared
        dt = DTYPE_CODE[self.cfg.logits_dtype]
        if self.fused_mask:
            mask = []
            if self.msa:
                attn = [P("spec_verify_attn_msa", self.desc, self.q, self.k_cache, self.v_cache, self.cache_len,
                          self.k_blk, self.v_blk, self.k_soft, self.v_soft, self.tree_parent, self.n_nodes,
                          int(self.tree_parent.shape[1]), int(self.cfg.gamma), self.out, self.lse, self.workspace,
                          int(self.ws_bytes), stream=stream)]
            else:
                attn = [P("spec_verify_attn_tree", self.desc, self.q, self.k_cache, self.v_cache, self.cache_len,
                          self.k_blk, self.v_blk, self.k_soft, self.v_soft, self.attn_parent, self.sp_flag,
                          self.n_q, self.out, self.lse, self.workspace, int(self.ws_bytes), stream=stream)]
        else:
            if self.msa:
                mask = [P("spec_build_msa_mask", self.tree_parent, self.n_nodes, self.B, self.tree_parent.shape[1],
                          self.cfg.gamma, self.Tq, self.mask_bits, self.sp_bits, self.n_q, stream=stream)]
            else:
                mask = [P("spec_build_mask", self.attn_parent, self.sp_flag, self.n_q, self.B, self.Tq,
                          self.mask_bits, self.sp_bits, stream=stream)]
            attn = [P("spec_verify_attn", self.desc, self.q, self.k_cache, self.v_cache, self.cache_len, self.k_blk,
                      self.v_blk, self.k_soft, self.v_soft, self.mask_bits, self.sp_bits, self.n_q, self.out,
                      self.lse, self.workspace, int(self.ws_bytes), stream=stream)]
        vrow = self.acc_parent if self.msa else None
        if self.accept == "greedy":
            tail = [P("spec_argmax_accept_commit", self.logits, dt, self.T, self.V, self.n_nodes, self.draft_tok,
                      self.acc_parent, vrow, self.max_depth, self.argmax, self.out_len, self.out_path,
                      self.out_bonus, self.desc, self.k_cache, self.v_cache, self.cache_len, self.cache_len_out,
                      self.k_blk, self.v_blk, stream=stream)]
        else:
            mode = bd.SPEC_ACCEPT_THRESHOLD if self.accept == "threshold" else bd.SPEC_ACCEPT_SOFT
            tail = [P("spec_prob_accept", self.logits, dt, self.B, self.T, self.V, self.n_nodes, self.draft_tok,
                      self.acc_parent, vrow, self.max_depth, mode, self.threshold, self.draft_prob, self.uniform,
                      self.argmax, self.out_prob, self.out_len, self.out_path, self.out_bonus, stream=stream),
                    P("spec_commit_kv", self.desc, self.k_cache, self.v_cache, self.cache_len, self.cache_len_out,
                      self.k_blk, self.v_blk, self.out_len, self.out_path, self.max_depth, stream=stream)]
        if self.msa:
            tail.append(P("spec_draft_tree", self.logits, dt, self.B, self.Tq, self.V, self.n_nodes, self.out_len,
                          self.out_path, self.max_depth, self.out_bonus, self.cfg.gamma, self.cfg.branch,
                          self.next_topk, self.next_tok, self.next_parent, self.next_n, stream=stream))
        return mask, attn, tail
