"""Thin ctypes binding of ``libspecverify.so`` (the C ABI in include/spec_verify.h).

Argument marshalling only: every function forwards to the entry point of the
same name.  Array arguments may be torch tensors (their ``data_ptr()`` is
passed), plain integer addresses, or None (NULL).  ``stream`` defaults to
torch's current HIP stream on the current device.  A non-zero status raises
``SpecError`` carrying the library's own message.

There is no fallback: if the HIP library is not built, the first call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_F32 = 0
SPEC_BF16 = 1
SPEC_OK = 0
SPEC_EINVAL = -1
SPEC_EUNSUPPORTED = -2
SPEC_EWORKSPACE = -3
SPEC_EHIP = -4
SPEC_MAX_TQ = 256
SPEC_MAX_NODES = 256
SPEC_MAX_DEPTH = 16
SPEC_MAX_SOFT = 256
SPEC_MAX_TOPK = 8
SPEC_NOALLOC_SCRATCH_BYTES = 32 << 20
SPEC_V_ROWS = 0
SPEC_V_TILE32 = 1
SPEC_ACCEPT_THRESHOLD = 1
SPEC_ACCEPT_SOFT = 2

# every symbol the header declares
EXPORTS = ("spec_build_mask", "spec_build_msa_mask", "spec_verify_attn_workspace", "spec_verify_attn",
           "spec_verify_attn_noalloc", "spec_verify_attn_tree", "spec_verify_attn_msa",
           "spec_argmax_accept", "spec_argmax_accept_rows", "spec_prob_accept", "spec_commit_kv",
           "spec_argmax_accept_commit", "spec_draft_tree",
           "spec_strerror", "spec_last_error", "spec_version")


class SpecError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func} failed with status {status}: {detail}")


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Tq", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("S", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("lmax", ctypes.c_int64), ("kv_stride_b", ctypes.c_int64), ("kv_stride_l", ctypes.c_int64),
        ("kv_stride_h", ctypes.c_int64), ("kv_splits", ctypes.c_int32), ("v_layout", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def load() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m masked_verification_attention_amd.build` (there is no CPU fallback)")
    # torch ships its own HIP runtime under the same soname; loading torch first makes the
    # library bind to that one, so that torch's streams and ours belong to a single runtime
    # (loaded the other way round, the process would hold two runtimes)
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    lib.spec_build_mask.argtypes = [_P, _P, _P, _I, _I, _P, _P, _P]
    lib.spec_build_mask.restype = ctypes.c_int
    lib.spec_build_msa_mask.argtypes = [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P]
    lib.spec_build_msa_mask.restype = ctypes.c_int
    lib.spec_draft_tree.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _I, _I, _P, _P, _P, _P, _P]
    lib.spec_draft_tree.restype = ctypes.c_int
    lib.spec_prob_accept.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _P, _I, _I, ctypes.c_float, _P, _P, _P, _P,
                                     _P, _P, _P, _P]
    lib.spec_prob_accept.restype = ctypes.c_int
    lib.spec_argmax_accept_commit.argtypes = [_P, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P,
                                              ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P]
    lib.spec_argmax_accept_commit.restype = ctypes.c_int
    lib.spec_verify_attn_workspace.argtypes = [ctypes.POINTER(AttnDesc)]
    lib.spec_verify_attn_workspace.restype = ctypes.c_size_t
    lib.spec_verify_attn.argtypes = [ctypes.POINTER(AttnDesc)] + [_P] * 14 + [ctypes.c_size_t, _P]
    lib.spec_verify_attn.restype = ctypes.c_int
    lib.spec_verify_attn_noalloc.argtypes = [ctypes.POINTER(AttnDesc)] + [_P] * 14
    lib.spec_verify_attn_noalloc.restype = ctypes.c_int
    lib.spec_verify_attn_tree.argtypes = [ctypes.POINTER(AttnDesc)] + [_P] * 14 + [ctypes.c_size_t, _P]
    lib.spec_verify_attn_tree.restype = ctypes.c_int
    lib.spec_verify_attn_msa.argtypes = [ctypes.POINTER(AttnDesc)] + [_P] * 10 + [_I, _I] + [_P] * 3 + \
        [ctypes.c_size_t, _P]
    lib.spec_verify_attn_msa.restype = ctypes.c_int
    lib.spec_argmax_accept.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P]
    lib.spec_argmax_accept.restype = ctypes.c_int
    lib.spec_argmax_accept_rows.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P]
    lib.spec_argmax_accept_rows.restype = ctypes.c_int
    lib.spec_commit_kv.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, _P, _I, _P]
    lib.spec_commit_kv.restype = ctypes.c_int
    lib.spec_strerror.argtypes = [ctypes.c_int]
    lib.spec_strerror.restype = ctypes.c_char_p
    lib.spec_last_error.argtypes = []
    lib.spec_last_error.restype = ctypes.c_char_p
    lib.spec_version.argtypes = []
    lib.spec_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x) -> Optional[int]:
    """Device address of a tensor argument.  The C ABI takes base pointers of
    dense arrays (the K/V cache's layout goes through the descriptor's strides),
    so a strided view or a host tensor is refused here rather than handed to a
    kernel that would read the wrong memory."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("array arguments must be device (GPU) tensors")
    if not x.is_contiguous():
        raise ValueError("array arguments must be contiguous tensors")
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, func: str):
    if status != SPEC_OK:
        raise SpecError(status, func, load().spec_last_error().decode())


class Prepared:
    """One entry-point call with its arguments converted once (device addresses,
    descriptor reference, stream handle): calling it only crosses the C ABI.  For
    loops that launch the same calls many times, where converting arguments per
    call would cost more host time than the kernels take on the device."""

    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name: str, *args, stream=None):
        lib = load()
        self.name = name
        self.fn = getattr(lib, name)
        self.keep = args                       # keeps tensors and descriptors alive
        conv = []
        for a in args:
            if isinstance(a, AttnDesc):
                conv.append(ctypes.byref(a))
            elif a is None or isinstance(a, (int, float)):
                conv.append(a)
            else:
                conv.append(_ptr(a))
        conv.append(_stream(stream))
        self.args = tuple(conv)

    def __call__(self):
        status = self.fn(*self.args)
        if status != SPEC_OK:
            _check(status, self.name)


def make_desc(B, Tq, Hq, Hkv, D, S, dtype, lmax, strides, scale=0.0, kv_splits=0, v_layout=SPEC_V_ROWS,
              out_dtype=SPEC_F32) -> AttnDesc:
    sb, sl, sh = strides
    return AttnDesc(B, Tq, Hq, Hkv, D, S, dtype, scale, lmax, sb, sl, sh, kv_splits, v_layout, out_dtype)


def spec_build_mask(attn_parent, sp_flag, n_q, B, Tq, mask_bits, sp_bits, stream=None):
    lib = load()
    _check(lib.spec_build_mask(_ptr(attn_parent), _ptr(sp_flag), _ptr(n_q), B, Tq, _ptr(mask_bits),
                               _ptr(sp_bits), _stream(stream) if B else None), "spec_build_mask")


def spec_build_msa_mask(tree_parent, n_nodes, B, N, gamma, Tq, mask_bits, sp_bits, n_q, stream=None):
    lib = load()
    _check(lib.spec_build_msa_mask(_ptr(tree_parent), _ptr(n_nodes), B, N, gamma, Tq, _ptr(mask_bits),
                                   _ptr(sp_bits), _ptr(n_q), _stream(stream) if B else None),
           "spec_build_msa_mask")


def spec_verify_attn_workspace(desc: AttnDesc) -> int:
    return int(load().spec_verify_attn_workspace(ctypes.byref(desc)))


def spec_verify_attn(desc: AttnDesc, q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft, v_soft,
                     mask_bits, sp_bits, n_q, out, lse=None, workspace=None, workspace_bytes=0,
                     stream=None):
    lib = load()
    _check(lib.spec_verify_attn(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len),
                                _ptr(k_blk), _ptr(v_blk), _ptr(k_soft), _ptr(v_soft), _ptr(mask_bits),
                                _ptr(sp_bits), _ptr(n_q), _ptr(out), _ptr(lse), _ptr(workspace),
                                int(workspace_bytes), _stream(stream) if desc.B else None),
           "spec_verify_attn")


def spec_verify_attn_noalloc(desc: AttnDesc, q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft, v_soft,
                             mask_bits, sp_bits, n_q, out, lse=None, stream=None):
    lib = load()
    _check(lib.spec_verify_attn_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len),
                                        _ptr(k_blk), _ptr(v_blk), _ptr(k_soft), _ptr(v_soft), _ptr(mask_bits),
                                        _ptr(sp_bits), _ptr(n_q), _ptr(out), _ptr(lse),
                                        _stream(stream) if desc.B else None),
           "spec_verify_attn_noalloc")


def spec_verify_attn_tree(desc: AttnDesc, q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft, v_soft,
                          attn_parent, sp_flag, n_q, out, lse=None, workspace=None, workspace_bytes=0,
                          stream=None):
    lib = load()
    _check(lib.spec_verify_attn_tree(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len),
                                     _ptr(k_blk), _ptr(v_blk), _ptr(k_soft), _ptr(v_soft), _ptr(attn_parent),
                                     _ptr(sp_flag), _ptr(n_q), _ptr(out), _ptr(lse), _ptr(workspace),
                                     int(workspace_bytes), _stream(stream) if desc.B else None),
           "spec_verify_attn_tree")


def spec_verify_attn_msa(desc: AttnDesc, q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft, v_soft,
                         tree_parent, n_nodes, N, gamma, out, lse=None, workspace=None, workspace_bytes=0,
                         stream=None):
    lib = load()
    _check(lib.spec_verify_attn_msa(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len),
                                    _ptr(k_blk), _ptr(v_blk), _ptr(k_soft), _ptr(v_soft), _ptr(tree_parent),
                                    _ptr(n_nodes), int(N), int(gamma), _ptr(out), _ptr(lse), _ptr(workspace),
                                    int(workspace_bytes), _stream(stream) if desc.B else None),
           "spec_verify_attn_msa")


def spec_argmax_accept(logits, logits_dtype, B, T, V, n_nodes, draft_tok, acc_parent, max_depth,
                       out_argmax, out_len, out_path, stream=None):
    lib = load()
    _check(lib.spec_argmax_accept(_ptr(logits), logits_dtype, B, T, V, _ptr(n_nodes), _ptr(draft_tok),
                                  _ptr(acc_parent), max_depth, _ptr(out_argmax), _ptr(out_len),
                                  _ptr(out_path), _stream(stream) if B else None),
           "spec_argmax_accept")


def spec_argmax_accept_rows(logits, logits_dtype, B, T, V, n_nodes, draft_tok, acc_parent, verify_row,
                            max_depth, out_argmax, out_len, out_path, out_bonus, stream=None):
    lib = load()
    _check(lib.spec_argmax_accept_rows(_ptr(logits), logits_dtype, B, T, V, _ptr(n_nodes), _ptr(draft_tok),
                                       _ptr(acc_parent), _ptr(verify_row), max_depth, _ptr(out_argmax),
                                       _ptr(out_len), _ptr(out_path), _ptr(out_bonus),
                                       _stream(stream) if B else None),
           "spec_argmax_accept_rows")


def spec_commit_kv(desc: AttnDesc, k_cache, v_cache, cache_len_in, cache_len_out, k_blk, v_blk, out_len,
                   out_path, max_depth, stream=None):
    lib = load()
    _check(lib.spec_commit_kv(ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len_in),
                              _ptr(cache_len_out), _ptr(k_blk), _ptr(v_blk), _ptr(out_len), _ptr(out_path),
                              max_depth, _stream(stream) if desc.B else None),
           "spec_commit_kv")


def spec_strerror(status: int) -> str:
    return load().spec_strerror(status).decode()


def spec_last_error() -> str:
    return load().spec_last_error().decode()


def spec_version() -> str:
    return load().spec_version().decode()


def spec_draft_tree(logits, logits_dtype, B, R, V, n_nodes, acc_len, acc_path, max_depth, root_tok, gamma, k,
                    out_topk, draft_tok, tree_parent, n_out, stream=None):
    lib = load()
    _check(lib.spec_draft_tree(_ptr(logits), logits_dtype, B, R, V, _ptr(n_nodes), _ptr(acc_len), _ptr(acc_path),
                               max_depth, _ptr(root_tok), gamma, k, _ptr(out_topk), _ptr(draft_tok),
                               _ptr(tree_parent), _ptr(n_out), _stream(stream) if B else None),
           "spec_draft_tree")


def spec_prob_accept(logits, logits_dtype, B, T, V, n_nodes, draft_tok, acc_parent, verify_row, max_depth, mode,
                     threshold, draft_prob, uniform, out_argmax, out_prob, out_len, out_path, out_bonus,
                     stream=None):
    lib = load()
    _check(lib.spec_prob_accept(_ptr(logits), logits_dtype, B, T, V, _ptr(n_nodes), _ptr(draft_tok),
                                _ptr(acc_parent), _ptr(verify_row), max_depth, mode, float(threshold),
                                _ptr(draft_prob), _ptr(uniform), _ptr(out_argmax), _ptr(out_prob), _ptr(out_len),
                                _ptr(out_path), _ptr(out_bonus), _stream(stream) if B else None),
           "spec_prob_accept")


def spec_argmax_accept_commit(logits, logits_dtype, T, V, n_nodes, draft_tok, acc_parent, verify_row, max_depth,
                              out_argmax, out_len, out_path, out_bonus, desc: AttnDesc, k_cache, v_cache,
                              cache_len_in, cache_len_out, k_blk, v_blk, stream=None):
    lib = load()
    _check(lib.spec_argmax_accept_commit(_ptr(logits), logits_dtype, T, V, _ptr(n_nodes), _ptr(draft_tok),
                                         _ptr(acc_parent), _ptr(verify_row), max_depth, _ptr(out_argmax),
                                         _ptr(out_len), _ptr(out_path), _ptr(out_bonus), ctypes.byref(desc),
                                         _ptr(k_cache), _ptr(v_cache), _ptr(cache_len_in), _ptr(cache_len_out),
                                         _ptr(k_blk), _ptr(v_blk), _stream(stream) if desc.B else None),
           "spec_argmax_accept_commit")
