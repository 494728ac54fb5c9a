"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from masked_verification_attention_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")

pytestmark = pytest.mark.skipif(not os.path.exists(bd.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_\w+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(bd.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bd.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror_and_version():
    assert bd.spec_strerror(0) == "success"
    assert bd.spec_strerror(bd.SPEC_EWORKSPACE).startswith("workspace")
    assert bd.spec_strerror(12345) == "unknown status"
    assert re.match(r"\d+\.\d+\.\d+$", bd.spec_version())


def good_desc(**kw):
    d = dict(B=2, Tq=60, Hq=32, Hkv=8, D=128, S=16, dtype=bd.SPEC_BF16, lmax=4156,
             strides=(4156 * 8 * 128, 8 * 128, 128))
    d.update(kw)
    return bd.make_desc(d["B"], d["Tq"], d["Hq"], d["Hkv"], d["D"], d["S"], d["dtype"], d["lmax"],
                        d["strides"], scale=d.get("scale", 0.0), kv_splits=d.get("kv_splits", 0))


FAKE = 1 << 20  # a 16-byte aligned non-NULL address that is never dereferenced on this path


def attn(desc, **over):
    args = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, cache_len=FAKE, k_blk=FAKE, v_blk=FAKE,
                k_soft=FAKE if desc.S else None, v_soft=FAKE if desc.S else None, mask_bits=FAKE,
                sp_bits=FAKE, n_q=FAKE, out=FAKE, lse=None, workspace=None, workspace_bytes=0)
    args.update(over)
    bd.spec_verify_attn(desc, args["q"], args["k_cache"], args["v_cache"], args["cache_len"], args["k_blk"],
                        args["v_blk"], args["k_soft"], args["v_soft"], args["mask_bits"], args["sp_bits"],
                        args["n_q"], args["out"], args["lse"], args["workspace"], args["workspace_bytes"],
                        stream=0)


@pytest.mark.parametrize("kw,status", [
    (dict(Tq=0), bd.SPEC_EINVAL), (dict(Tq=257), bd.SPEC_EINVAL), (dict(B=-1), bd.SPEC_EINVAL),
    (dict(Hq=30), bd.SPEC_EINVAL), (dict(Hkv=0), bd.SPEC_EINVAL), (dict(D=96), bd.SPEC_EUNSUPPORTED),
    (dict(S=-1), bd.SPEC_EINVAL), (dict(S=257), bd.SPEC_EINVAL), (dict(dtype=7), bd.SPEC_EINVAL),
    (dict(lmax=-5), bd.SPEC_EINVAL), (dict(strides=(0, 1024, 128)), bd.SPEC_EINVAL),
    (dict(strides=(4156 * 1024, 1028, 128)), bd.SPEC_EINVAL), (dict(scale=float("nan")), bd.SPEC_EINVAL),
    (dict(scale=-1.0), bd.SPEC_EINVAL), (dict(kv_splits=65), bd.SPEC_EINVAL),
    (dict(B=9000), bd.SPEC_EUNSUPPORTED),
])
def test_verify_attn_rejects_bad_descriptor(kw, status):
    d = good_desc(**kw)
    with pytest.raises(bd.SpecError) as e:
        attn(d)
    assert e.value.status == status
    assert bd.spec_last_error() != ""
    assert bd.spec_verify_attn_workspace(d) == 0


def test_verify_attn_rejects_bad_pointers_and_workspace():
    d = good_desc()
    for name in ("q", "k_cache", "cache_len", "mask_bits", "n_q", "out"):
        with pytest.raises(bd.SpecError) as e:
            attn(d, **{name: None})
        assert e.value.status == bd.SPEC_EINVAL
    with pytest.raises(bd.SpecError) as e:       # soft prompt missing although S > 0
        attn(d, k_soft=None)
    assert e.value.status == bd.SPEC_EINVAL
    with pytest.raises(bd.SpecError) as e:       # soft prompt given with S == 0
        attn(good_desc(S=0), k_soft=FAKE, v_soft=FAKE)
    assert e.value.status == bd.SPEC_EINVAL
    with pytest.raises(bd.SpecError) as e:       # misaligned
        attn(d, q=FAKE + 2)
    assert e.value.status == bd.SPEC_EINVAL
    dsplit = good_desc(kv_splits=4)
    need = bd.spec_verify_attn_workspace(dsplit)
    assert need > 0
    with pytest.raises(bd.SpecError) as e:
        attn(dsplit, workspace=FAKE, workspace_bytes=need - 1)
    assert e.value.status == bd.SPEC_EWORKSPACE
    with pytest.raises(bd.SpecError) as e:
        attn(dsplit, workspace=None, workspace_bytes=need)
    assert e.value.status == bd.SPEC_EWORKSPACE


def test_empty_batch_is_a_noop_without_touching_memory():
    attn(good_desc(B=0), q=None, out=None)
    bd.spec_build_mask(None, None, None, 0, 8, None, None, stream=0)
    bd.spec_build_msa_mask(None, None, 0, 40, 3, 160, None, None, None, stream=0)
    bd.spec_argmax_accept_commit(None, bd.SPEC_BF16, 4, 100, None, None, None, None, 4, None, None, None, None,
                                 good_desc(B=0), None, None, None, None, None, None, stream=0)
    bd.spec_prob_accept(None, bd.SPEC_BF16, 0, 4, 100, None, None, None, None, 4, bd.SPEC_ACCEPT_SOFT, 0.0, None,
                        None, None, None, None, None, None, stream=0)
    bd.spec_draft_tree(None, bd.SPEC_BF16, 0, 160, 100, None, None, None, 4, None, 3, 3, None, None, None, None,
                       stream=0)
    bd.spec_argmax_accept(None, bd.SPEC_BF16, 0, 4, 100, None, None, None, 4, None, None, None, stream=0)
    bd.spec_commit_kv(good_desc(B=0), None, None, None, None, None, None, None, None, 4, stream=0)


def test_other_entry_points_reject_bad_arguments():
    cases = [
        lambda: bd.spec_build_mask(FAKE, None, FAKE, 2, 0, FAKE, FAKE, stream=0),
        lambda: bd.spec_build_mask(FAKE, None, FAKE, 2, 300, FAKE, FAKE, stream=0),
        lambda: bd.spec_build_mask(None, None, FAKE, 2, 8, FAKE, FAKE, stream=0),
        lambda: bd.spec_build_msa_mask(FAKE, FAKE, 2, 40, 3, 159, FAKE, FAKE, FAKE, stream=0),   # rows > Tq
        lambda: bd.spec_build_msa_mask(FAKE, FAKE, 2, 0, 3, 160, FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_build_msa_mask(FAKE, FAKE, 2, 40, -1, 160, FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_build_msa_mask(FAKE, FAKE, 2, 2, 200, 257, FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_build_msa_mask(FAKE, FAKE, 2, 40, 3, 160, FAKE, FAKE, None, stream=0),
        lambda: bd.spec_build_msa_mask(FAKE, FAKE + 1, 2, 40, 3, 160, FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_build_msa_mask(FAKE, FAKE, -1, 40, 3, 160, FAKE, FAKE, FAKE, stream=0),
        # spec_prob_accept: bad mode, negative / NaN threshold, soft without draws, NULL prob, T, misaligned
        lambda: bd.spec_prob_accept(FAKE, bd.SPEC_BF16, 2, 4, 100, FAKE, FAKE, FAKE, None, 4, 0, 0.5, FAKE, FAKE,
                                    FAKE, FAKE, FAKE, FAKE, None, stream=0),
        lambda: bd.spec_prob_accept(FAKE, bd.SPEC_BF16, 2, 4, 100, FAKE, FAKE, FAKE, None, 4,
                                    bd.SPEC_ACCEPT_THRESHOLD, -0.1, None, None, FAKE, FAKE, FAKE, FAKE, None, stream=0),
        lambda: bd.spec_prob_accept(FAKE, bd.SPEC_BF16, 2, 4, 100, FAKE, FAKE, FAKE, None, 4,
                                    bd.SPEC_ACCEPT_THRESHOLD, float("nan"), None, None, FAKE, FAKE, FAKE, FAKE, None,
                                    stream=0),
        lambda: bd.spec_prob_accept(FAKE, bd.SPEC_BF16, 2, 4, 100, FAKE, FAKE, FAKE, None, 4, bd.SPEC_ACCEPT_SOFT,
                                    0.0, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, stream=0),
        lambda: bd.spec_prob_accept(FAKE, bd.SPEC_BF16, 2, 4, 100, FAKE, FAKE, FAKE, None, 4,
                                    bd.SPEC_ACCEPT_THRESHOLD, 0.5, None, None, FAKE, None, FAKE, FAKE, None, stream=0),
        lambda: bd.spec_prob_accept(FAKE, bd.SPEC_BF16, 2, 0, 100, FAKE, FAKE, FAKE, None, 4,
                                    bd.SPEC_ACCEPT_THRESHOLD, 0.5, None, None, FAKE, FAKE, FAKE, FAKE, None, stream=0),
        lambda: bd.spec_prob_accept(FAKE, bd.SPEC_BF16, 2, 4, 100, FAKE, FAKE, FAKE, None, 4, bd.SPEC_ACCEPT_SOFT,
                                    0.0, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, stream=0),
        # spec_argmax_accept_commit: T over the block, bad descriptor, NULL cache, misaligned block
        lambda: bd.spec_argmax_accept_commit(FAKE, bd.SPEC_BF16, 64, 100, FAKE, FAKE, FAKE, None, 4, FAKE, FAKE,
                                             FAKE, None, good_desc(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_argmax_accept_commit(FAKE, bd.SPEC_BF16, 4, 100, FAKE, FAKE, FAKE, None, 4, FAKE, FAKE,
                                             FAKE, None, good_desc(D=80), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                             stream=0),
        lambda: bd.spec_argmax_accept_commit(FAKE, bd.SPEC_BF16, 4, 100, FAKE, FAKE, FAKE, None, 4, FAKE, FAKE,
                                             FAKE, None, good_desc(), None, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_argmax_accept_commit(FAKE, bd.SPEC_BF16, 4, 100, FAKE, FAKE, FAKE, None, 4, FAKE, FAKE,
                                             FAKE, None, good_desc(), FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE,
                                             stream=0),
        lambda: bd.spec_argmax_accept_commit(FAKE, bd.SPEC_BF16, 4, 100, FAKE, FAKE, FAKE, None, 17, FAKE, FAKE,
                                             FAKE, None, good_desc(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0),
        # spec_draft_tree: k out of range, tree over 256 nodes, V < k, bad dtype, max_depth, NULL, misaligned
        lambda: bd.spec_draft_tree(FAKE, bd.SPEC_BF16, 2, 160, 100, FAKE, FAKE, FAKE, 4, FAKE, 3, 0, FAKE, FAKE,
                                   FAKE, FAKE, stream=0),
        lambda: bd.spec_draft_tree(FAKE, bd.SPEC_BF16, 2, 160, 100, FAKE, FAKE, FAKE, 4, FAKE, 3, 9, FAKE, FAKE,
                                   FAKE, FAKE, stream=0),
        lambda: bd.spec_draft_tree(FAKE, bd.SPEC_BF16, 2, 160, 100, FAKE, FAKE, FAKE, 4, FAKE, 4, 4, FAKE, FAKE,
                                   FAKE, FAKE, stream=0),
        lambda: bd.spec_draft_tree(FAKE, bd.SPEC_BF16, 2, 160, 2, FAKE, FAKE, FAKE, 4, FAKE, 3, 3, FAKE, FAKE,
                                   FAKE, FAKE, stream=0),
        lambda: bd.spec_draft_tree(FAKE, 5, 2, 160, 100, FAKE, FAKE, FAKE, 4, FAKE, 3, 3, FAKE, FAKE,
                                   FAKE, FAKE, stream=0),
        lambda: bd.spec_draft_tree(FAKE, bd.SPEC_BF16, 2, 160, 100, FAKE, FAKE, FAKE, 17, FAKE, 3, 3, FAKE, FAKE,
                                   FAKE, FAKE, stream=0),
        lambda: bd.spec_draft_tree(FAKE, bd.SPEC_BF16, 2, 160, 100, FAKE, FAKE, FAKE, 4, FAKE, 3, 3, None, FAKE,
                                   FAKE, FAKE, stream=0),
        lambda: bd.spec_draft_tree(FAKE, bd.SPEC_BF16, 2, 160, 100, FAKE, FAKE, FAKE + 2, 4, FAKE, 3, 3, FAKE, FAKE,
                                   FAKE, FAKE, stream=0),
        lambda: bd.spec_draft_tree(FAKE, bd.SPEC_BF16, 2, 300, 100, FAKE, FAKE, FAKE, 4, FAKE, 3, 3, FAKE, FAKE,
                                   FAKE, FAKE, stream=0),
        lambda: bd.spec_argmax_accept(FAKE, bd.SPEC_BF16, 2, 0, 100, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_argmax_accept(FAKE, bd.SPEC_BF16, 2, 4, 0, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_argmax_accept(FAKE, bd.SPEC_BF16, 2, 4, 100, FAKE, FAKE, FAKE, 17, FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_argmax_accept(FAKE, 3, 2, 4, 100, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_argmax_accept(FAKE, bd.SPEC_BF16, 2, 4, 100, FAKE, None, FAKE, 4, FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_argmax_accept_rows(FAKE, bd.SPEC_BF16, 2, 0, 100, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE,
                                           FAKE, FAKE, stream=0),
        lambda: bd.spec_argmax_accept_rows(FAKE, bd.SPEC_BF16, 2, 4, 100, FAKE, FAKE, None, FAKE, 4, FAKE, FAKE,
                                           FAKE, FAKE, stream=0),
        lambda: bd.spec_argmax_accept_rows(FAKE, bd.SPEC_BF16, 2, 4, 100, FAKE, FAKE, FAKE, FAKE + 2, 4, FAKE,
                                           FAKE, FAKE, FAKE, stream=0),
        lambda: bd.spec_argmax_accept_rows(FAKE, bd.SPEC_BF16, 2, 4, 100, FAKE, FAKE, FAKE, FAKE, 17, FAKE, FAKE,
                                           FAKE, FAKE, stream=0),
        lambda: bd.spec_commit_kv(good_desc(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, stream=0),
        lambda: bd.spec_commit_kv(good_desc(), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, stream=0),
        lambda: bd.spec_commit_kv(good_desc(D=80), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, stream=0),
    ]
    for f in cases:
        with pytest.raises(bd.SpecError):
            f()


def test_workspace_policy():
    # bf16 runs on the matrix cores and splits the prefix only when the (request, kv-head, row
    # chunk) items cannot fill 256 CUs: the tree/contemplate shape and the 8-row lookahead shape
    # over 32 heads both fill the chip unsplit
    assert bd.spec_verify_attn_workspace(good_desc(B=16)) == 0
    la = good_desc(B=8, Tq=8, Hq=32, Hkv=32, S=0, lmax=2056, strides=(2056 * 32 * 128, 32 * 128, 128))
    assert bd.spec_verify_attn_workspace(la) == 0
    # a single request over 8 kv-heads splits its long prefix (>= 512 keys per split)
    one = good_desc(B=1, lmax=8192, strides=(8192 * 8 * 128, 8 * 128, 128))
    assert bd.spec_verify_attn_workspace(one) > 0
    # fp32 runs on the vector ALUs, which split every prefix into ~512-key pieces
    la32 = good_desc(B=8, Tq=8, Hq=32, Hkv=32, S=0, lmax=2056, dtype=bd.SPEC_F32,
                     strides=(2056 * 32 * 128, 32 * 128, 128))
    assert bd.spec_verify_attn_workspace(la32) > 0


def test_binding_refuses_host_tensors():
    # a host tensor's address must never reach a kernel: the binding refuses it
    # before calling into the library
    import torch
    host = torch.zeros(2, 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="device"):
        bd.spec_build_mask(host, None, FAKE, 2, 8, FAKE, FAKE, stream=0)


def test_noalloc_refuses_more_scratch_than_it_holds_before_any_hip_call():
    # 64 requests x 8 kv-heads x 2048 rows x 8 splits of partials: far above the scratch size
    desc = good_desc(B=64, Tq=256, Hq=64, Hkv=8, lmax=16384, strides=(16384 * 8 * 128, 8 * 128, 128), kv_splits=8)
    need = bd.spec_verify_attn_workspace(desc)
    assert need > bd.SPEC_NOALLOC_SCRATCH_BYTES
    with pytest.raises(bd.SpecError) as e:
        bd.spec_verify_attn_noalloc(desc, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    None, stream=0)
    assert e.value.status == bd.SPEC_EWORKSPACE
    assert str(need) in str(e.value) and str(bd.SPEC_NOALLOC_SCRATCH_BYTES) in str(e.value)
    # the argument checks are those of spec_verify_attn
    with pytest.raises(bd.SpecError) as e:
        bd.spec_verify_attn_noalloc(good_desc(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE + 4, None, stream=0)
    assert e.value.status == bd.SPEC_EINVAL and "16-byte aligned" in str(e.value)
    # B == 0 is a no-op that touches no device
    bd.spec_verify_attn_noalloc(good_desc(B=0), None, None, None, None, None, None, None, None, None, None, None,
                                None, None, stream=0)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define SPEC_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == bd.SPEC_NOALLOC_SCRATCH_BYTES


def test_out_dtype_validation():
    ok_desc = good_desc()
    ok_desc.out_dtype = bd.SPEC_BF16
    assert bd.spec_verify_attn_workspace(ok_desc) > 0
    cases = [
        (dict(), 5, bd.SPEC_EINVAL, "out_dtype"),                            # not a dtype
        (dict(), -1, bd.SPEC_EINVAL, "out_dtype"),
        (dict(dtype=bd.SPEC_F32), bd.SPEC_BF16, bd.SPEC_EUNSUPPORTED, "bf16"),  # bf16 out of f32 inputs
    ]
    for kw, od, status, word in cases:
        desc = good_desc(**kw)
        desc.out_dtype = od
        assert bd.spec_verify_attn_workspace(desc) == 0
        with pytest.raises(bd.SpecError) as e:
            attn(desc)
        assert e.value.status == status and word in str(e.value), (kw, od, str(e.value))


def test_v_layout_validation():
    hm = dict(lmax=4160, strides=(8 * 4160 * 128, 128, 4160 * 128))
    ok_desc = good_desc(**hm)
    ok_desc.v_layout = bd.SPEC_V_TILE32
    assert bd.spec_verify_attn_workspace(ok_desc) > 0             # valid (two requests: split)
    cases = [
        (dict(**hm), 7, bd.SPEC_EINVAL, "v_layout"),                              # not a layout
        (dict(dtype=bd.SPEC_F32, **hm), bd.SPEC_V_TILE32, bd.SPEC_EUNSUPPORTED, "bf16"),
        (dict(), bd.SPEC_V_TILE32, bd.SPEC_EINVAL, "head-major"),                 # token-major strides
        (dict(lmax=4156, strides=(8 * 4156 * 128, 128, 4156 * 128)), bd.SPEC_V_TILE32, bd.SPEC_EINVAL, "lmax"),
    ]
    for kw, vl, status, word in cases:
        desc = good_desc(**kw)
        desc.v_layout = vl
        assert bd.spec_verify_attn_workspace(desc) == 0
        with pytest.raises(bd.SpecError) as e:
            attn(desc)
        assert e.value.status == status and word in str(e.value), (kw, vl, str(e.value))
        with pytest.raises(bd.SpecError) as e:
            bd.spec_commit_kv(desc, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, stream=0)
        assert e.value.status == status


def test_attn_tree_validation_before_any_hip_call():
    F = FAKE

    def tree(desc, parent=F, flags=F, q=F, out=F, ws=None, ws_bytes=0, soft=True):
        ks = F if (desc.S and soft) else None
        bd.spec_verify_attn_tree(desc, q, F, F, F, F, F, ks, ks, parent, flags, F, out, None, ws, ws_bytes,
                                 stream=0)

    # fp32 inputs take the two-call path
    with pytest.raises(bd.SpecError) as e:
        tree(good_desc(dtype=bd.SPEC_F32))
    assert e.value.status == bd.SPEC_EUNSUPPORTED and "bf16" in str(e.value)
    # the parent array is required and word-aligned; the byte flags need no alignment
    with pytest.raises(bd.SpecError) as e:
        tree(good_desc(), parent=None)
    assert e.value.status == bd.SPEC_EINVAL and "attn_parent" in str(e.value)
    with pytest.raises(bd.SpecError) as e:
        tree(good_desc(), parent=F + 2)
    assert e.value.status == bd.SPEC_EINVAL and "4-byte aligned" in str(e.value)
    # spec_verify_attn's other checks apply
    with pytest.raises(bd.SpecError) as e:
        tree(good_desc(), q=F + 4)
    assert e.value.status == bd.SPEC_EINVAL and "16-byte aligned" in str(e.value)
    with pytest.raises(bd.SpecError) as e:
        tree(good_desc(), out=None)
    assert e.value.status == bd.SPEC_EINVAL
    # soft prompt rows: k_soft / v_soft are needed, sp_flag is not
    with pytest.raises(bd.SpecError) as e:
        tree(good_desc(S=16), soft=False)
    assert e.value.status == bd.SPEC_EINVAL and "k_soft" in str(e.value)
    # a split plan needs its workspace, as spec_verify_attn
    desc = good_desc(kv_splits=4)
    need = bd.spec_verify_attn_workspace(desc)
    assert need > 0
    with pytest.raises(bd.SpecError) as e:
        tree(desc, ws=F, ws_bytes=need - 1)
    assert e.value.status == bd.SPEC_EWORKSPACE
    # B == 0 is a no-op that touches no device
    bd.spec_verify_attn_tree(good_desc(B=0), None, None, None, None, None, None, None, None, None, None, None,
                             None, None, None, 0, stream=0)


def test_attn_msa_validation_before_any_hip_call():
    F = FAKE

    def msa(desc, tree=F, nodes=F, N=40, gamma=3, q=F):
        ks = F if desc.S else None
        bd.spec_verify_attn_msa(desc, q, F, F, F, F, F, ks, ks, tree, nodes, N, gamma, F, None, None, 0, stream=0)

    d160 = dict(Tq=160, Hq=32, Hkv=32, D=64, S=0)
    with pytest.raises(bd.SpecError) as e:
        msa(good_desc(dtype=bd.SPEC_F32, **d160))
    assert e.value.status == bd.SPEC_EUNSUPPORTED
    for kw, word in [(dict(N=0), "N = 0"), (dict(gamma=-1), "gamma"), (dict(N=41), "exceed Tq"),
                     (dict(tree=None), "tree_parent"), (dict(nodes=None), "n_nodes"),
                     (dict(tree=F + 2), "4-byte aligned"), (dict(q=F + 4), "16-byte aligned")]:
        with pytest.raises(bd.SpecError) as e:
            msa(good_desc(**d160), **kw)
        assert e.value.status == bd.SPEC_EINVAL and word in str(e.value), (kw, str(e.value))
    # B == 0 is a no-op that touches no device
    bd.spec_verify_attn_msa(good_desc(B=0, **d160), None, None, None, None, None, None, None, None, None, None,
                            40, 3, None, None, None, 0, stream=0)
