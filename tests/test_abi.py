"""C-ABI checks that need no GPU: the library loads, exports every function
include/bsa.h declares, and stage-1 / stage-2 argument checks return the
documented status codes before any device work."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_varlen_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "bsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_]+)\s*\(", src)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert "bsa_fwd" in names and "bsa_bwd" in names and "bsa_get_workspace_size" in names
    lib = bsa.library()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bsa.EXPORTS)


def test_struct_layout():
    assert ctypes.sizeof(bsa.bsa_problem_t) == 128
    assert bsa.bsa_problem_t.pre_tokens.offset == 112
    assert bsa.bsa_problem_t.next_tokens.offset == 120
    assert bsa.bsa_problem_t.total_q.offset == 24
    assert bsa.bsa_problem_t.page_stride.offset == 88
    assert bsa.bsa_problem_t.scale.offset == 96


def good(**kw):
    base = dict(dtype=bsa.BSA_DTYPE_BF16, batch=2, num_heads_q=4, num_heads_kv=2, head_dim=128, total_q=600,
                total_kv=600, max_seqlen_q=400, max_seqlen_kv=400, block_x=128, block_y=128,
                sparse_kind=bsa.BSA_SPARSE_BLOCK_MASK, sparse_heads=4, sparse_rows=4, sparse_width=4,
                mask_type=bsa.BSA_MASK_CAUSAL, kv_layout=bsa.BSA_KV_TND, scale=0.0)
    base.update(kw)
    return bsa.problem(**base)


def status(p, fwd=True, bwd=True):
    f = ctypes.c_size_t(0)
    b = ctypes.c_size_t(0)
    return bsa.library().bsa_get_workspace_size(ctypes.byref(p) if p is not None else None,
                                                ctypes.byref(f) if fwd else None, ctypes.byref(b) if bwd else None)


def test_dq_flags():
    """BSA_FLAG_DQ_ATOMIC adds the fp32 dQ accumulator (T_q * N1 * D * 4
    bytes) to the backward workspace only; it excludes
    BSA_FLAG_DETERMINISTIC; unknown flag bits are rejected."""
    f0, b0 = bsa.bsa_get_workspace_size(good())
    f1, b1 = bsa.bsa_get_workspace_size(good(flags=bsa.BSA_FLAG_DQ_ATOMIC))
    assert f1 == f0 and b1 - b0 >= 600 * 4 * 128 * 4 and b1 - b0 < 600 * 4 * 128 * 4 + 256
    f2, b2 = bsa.bsa_get_workspace_size(good(flags=bsa.BSA_FLAG_DETERMINISTIC))
    assert (f2, b2) == (f0, b0)
    assert status(good(flags=bsa.BSA_FLAG_DETERMINISTIC | bsa.BSA_FLAG_DQ_ATOMIC)) == bsa.BSA_ERR_PARAM_INVALID
    assert status(good(flags=32)) == bsa.BSA_ERR_PARAM_INVALID


def test_check_values_flag():
    """BSA_FLAG_CHECK_VALUES goes with every other flag and leaves the
    workspace sizes as they are; bsa_fwd_noalloc, which must not wait on the
    stream, rejects it on the host before any device work (the dummy
    pointers are never dereferenced)."""
    f0, b0 = bsa.bsa_get_workspace_size(good())
    assert bsa.bsa_get_workspace_size(good(flags=bsa.BSA_FLAG_CHECK_VALUES)) == (f0, b0)
    for extra in (bsa.BSA_FLAG_INDEX_BUILT, bsa.BSA_FLAG_DETERMINISTIC, bsa.BSA_FLAG_DQ_ATOMIC):
        assert status(good(flags=bsa.BSA_FLAG_CHECK_VALUES | extra)) == bsa.BSA_OK
    p = good(flags=bsa.BSA_FLAG_CHECK_VALUES)
    lib = bsa.library()
    assert lib.bsa_fwd_noalloc(ctypes.byref(p), 1, 1, 1, 1, 1, None, 1, None, None, 1, 1,
                               None) == bsa.BSA_ERR_PARAM_INVALID
    assert [bsa.BSA_CHECK_CU_Q_ENDS, bsa.BSA_CHECK_CU_Q_ORDER, bsa.BSA_CHECK_SQ_LONG, bsa.BSA_CHECK_CU_KV_ENDS,
            bsa.BSA_CHECK_CU_KV_ORDER, bsa.BSA_CHECK_SKV_LONG, bsa.BSA_CHECK_PAGE] == [1, 2, 4, 8, 16, 32, 64]


def test_band_mask_accepted():
    """BSA_MASK_BAND with any pre / next tokens (negative ones included) is a
    valid descriptor; the window does not change the workspace bounds."""
    f0, b0 = bsa.bsa_get_workspace_size(good())
    for pre, nxt in ((128, 0), (-5, 40), (2 ** 40, -(2 ** 40)), (0, 0)):
        f, b = bsa.bsa_get_workspace_size(good(mask_type=bsa.BSA_MASK_BAND, pre_tokens=pre, next_tokens=nxt))
        assert (f, b) == (f0, b0)


def test_workspace_size_ok():
    f, b = bsa.bsa_get_workspace_size(good())
    assert 0 < f <= b
    assert f % 256 == 0 and b % 256 == 0
    # bwd workspace holds the D = rowsum(dO o O) vector: >= T_q * N1 floats
    assert b - f >= 600 * 4 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(struct_size=8), bsa.BSA_ERR_PARAM_INVALID),
    (dict(dtype=3), bsa.BSA_ERR_PARAM_INVALID),
    (dict(head_dim=96), bsa.BSA_ERR_PARAM_INVALID),
    (dict(num_heads_q=6, num_heads_kv=4, sparse_heads=6), bsa.BSA_ERR_PARAM_INVALID),
    (dict(num_heads_q=512, num_heads_kv=4, sparse_heads=512), bsa.BSA_ERR_PARAM_INVALID),
    (dict(num_heads_q=0), bsa.BSA_ERR_PARAM_INVALID),
    (dict(batch=-1), bsa.BSA_ERR_PARAM_INVALID),
    (dict(block_y=100), bsa.BSA_ERR_PARAM_INVALID),
    (dict(block_x=0), bsa.BSA_ERR_PARAM_INVALID),
    (dict(sparse_kind=7), bsa.BSA_ERR_PARAM_INVALID),
    (dict(sparse_heads=3), bsa.BSA_ERR_PARAM_INVALID),
    (dict(sparse_kind=bsa.BSA_SPARSE_IDX_I32, sparse_width=300), bsa.BSA_ERR_PARAM_INVALID),
    (dict(mask_type=3), bsa.BSA_ERR_PARAM_INVALID),
    (dict(scale=-1.0), bsa.BSA_ERR_PARAM_INVALID),
    (dict(scale=float("nan")), bsa.BSA_ERR_PARAM_INVALID),
    (dict(flags=16), bsa.BSA_ERR_PARAM_INVALID),  # unknown flag bit
    (dict(flags=bsa.BSA_FLAG_INDEX_BUILT), bsa.BSA_OK),
    (dict(kv_layout=bsa.BSA_KV_PAGED, page_size=128, max_pages_per_seq=1, page_stride=128 * 2 * 128),
     bsa.BSA_ERR_PARAM_INVALID),  # too few pages per sequence for max_seqlen_kv
    (dict(kv_layout=bsa.BSA_KV_PAGED, page_size=128, max_pages_per_seq=4, page_stride=100),
     bsa.BSA_ERR_PARAM_INVALID),  # page stride shorter than a page
    (dict(block_x=96), bsa.BSA_OK),         # work items of 96 rows, a short dK/dV part
    (dict(block_x=1), bsa.BSA_OK),          # per-token selection
    (dict(block_x=64), bsa.BSA_OK),         # half-height work items
    (dict(block_x=192), bsa.BSA_OK),        # a 128-row and a 64-row work item per q-block
    (dict(block_x=4097), bsa.BSA_ERR_INNER),  # valid, no compiled variant
    (dict(block_y=4096 + 16), bsa.BSA_ERR_INNER),
    (dict(dtype=bsa.BSA_DTYPE_FP8_E4M3), bsa.BSA_ERR_PARAM_INVALID),  # e4m3 needs an fp16 / bf16 out_dtype
    (dict(dtype=bsa.BSA_DTYPE_BF16, out_dtype=bsa.BSA_DTYPE_F16), bsa.BSA_ERR_PARAM_INVALID),
])
def test_stage1_rejects(kw, code):
    assert status(good(**kw)) == code


def test_stage1_nullptr():
    assert status(None) == bsa.BSA_ERR_PARAM_NULLPTR
    assert status(good(), fwd=False, bwd=False) == bsa.BSA_ERR_PARAM_NULLPTR


def test_paged_backward_sizes():
    p = good(kv_layout=bsa.BSA_KV_PAGED, page_size=128, max_pages_per_seq=4, page_stride=128 * 2 * 128,
             total_kv=10)
    assert status(p, fwd=True, bwd=False) == bsa.BSA_OK
    assert status(p, fwd=False, bwd=True) == bsa.BSA_OK
    p64 = good(kv_layout=bsa.BSA_KV_PAGED, page_size=64, max_pages_per_seq=8, page_stride=64 * 2 * 128,
               total_kv=10)
    assert status(p64, fwd=False, bwd=True) == bsa.BSA_OK
    # any multiple of 16 has both passes (the last 128-key dK/dV tile of a block may be partial)
    for by in (16, 48, 64, 80, 192):
        assert status(good(block_y=by), fwd=True, bwd=True) == bsa.BSA_OK


def _fwd_status(p, ws_bytes=1 << 30, **ptrs):
    args = dict(q=1, k=1, v=1, cu_q=1, cu_kv=1, seqused=None, sparse=1, count=None, bt=None, out=1, lse=1, ws=1)
    args.update(ptrs)
    lib = bsa.library()
    return lib.bsa_fwd(ctypes.byref(p), args["q"], args["k"], args["v"], args["cu_q"], args["cu_kv"],
                       args["seqused"], args["sparse"], args["count"], args["bt"], args["out"], args["lse"],
                       args["ws"], ws_bytes, None)


@pytest.mark.parametrize("missing", ["q", "out", "lse", "cu_q", "cu_kv", "sparse", "ws"])
def test_stage2_null_pointers(missing):
    """Each required pointer NULL -> 161001, checked on the host before any
    launch (the non-NULL dummies are never dereferenced)."""
    assert _fwd_status(good(), **{missing: None}) == bsa.BSA_ERR_PARAM_NULLPTR


def test_stage2_idx_needs_count_and_paged_needs_table():
    p = good(sparse_kind=bsa.BSA_SPARSE_IDX_I32, sparse_rows=8, sparse_width=4)
    assert _fwd_status(p) == bsa.BSA_ERR_PARAM_NULLPTR
    pp = good(kv_layout=bsa.BSA_KV_PAGED, page_size=128, max_pages_per_seq=4, page_stride=128 * 2 * 128)
    assert _fwd_status(pp, cu_kv=None, seqused=1) == bsa.BSA_ERR_PARAM_NULLPTR  # block_table
    assert _fwd_status(pp, cu_kv=None, seqused=None, bt=1) == bsa.BSA_ERR_PARAM_NULLPTR


def test_stage2_small_workspace():
    p = good()
    f, _ = bsa.bsa_get_workspace_size(p)
    assert _fwd_status(p, ws_bytes=f - 1) == bsa.BSA_ERR_PARAM_INVALID


def test_stage2_empty_problem_is_a_noop():
    assert _fwd_status(good(batch=0, total_q=0, total_kv=0), q=None, k=None, v=None, out=None, lse=None,
                       ws=None) == bsa.BSA_OK
    assert _fwd_status(good(total_q=0), q=None, out=None, lse=None) == bsa.BSA_OK


def test_status_strings():
    for code in (bsa.BSA_OK, bsa.BSA_ERR_PARAM_NULLPTR, bsa.BSA_ERR_PARAM_INVALID, bsa.BSA_ERR_INNER,
                 bsa.BSA_ERR_RUNTIME):
        assert bsa.status_string(code).startswith("BSA_")
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_get_workspace_size(good(head_dim=32))
    assert e.value.status == bsa.BSA_ERR_PARAM_INVALID


def test_index_view_is_consistent_with_sizes():
    p = good()
    f, b = bsa.bsa_get_workspace_size(p)
    v0 = bsa.bsa_index_view(p, False)
    v1 = bsa.bsa_index_view(p, True)
    assert v0.off_work + 4 * v0.max_rows <= f
    assert v1.off_work_kv + 4 * v1.max_kv_items <= b
    assert v1.max_kv_items == 2 * (600 // 128 + 2)
    # bounds: rows >= every possible Hs * totalQBlocks
    assert v0.max_rows >= 4 * (600 // 128 + 2)


def test_index_view_reports_row_tiles():
    """q-blocks of at most 32 rows that divide 128 are indexed as 128-row
    tiles with row masks (block_y a multiple of 64, at most 2048 KV blocks a
    sequence); everything else keeps its own q-blocks and no masks."""
    def view(with_csc=True, **kw):
        return bsa.bsa_index_view(good(**kw), with_csc)

    for bx in (1, 2, 4, 8, 16, 32):
        v = view(block_x=bx, sparse_kind=bsa.BSA_SPARSE_IDX_I32, sparse_rows=600, sparse_width=8)
        assert v.tile_rows == 128, bx
        assert v.off_row_mask and v.off_col_mask
        assert v.off_row_mask + 16 * v.max_nnz <= bsa.bsa_get_workspace_size(good(block_x=bx))[1]
        assert view(False, block_x=bx).off_col_mask == 0  # no transposed lists, no column masks
        assert view(block_x=bx, dtype=bsa.BSA_DTYPE_FP8_E4M3,
                    out_dtype=bsa.BSA_DTYPE_BF16).tile_rows == 128  # the e4m3 forward too
    for kw in (dict(block_x=128), dict(block_x=64), dict(block_x=48), dict(block_x=24),
               dict(block_x=16, block_y=48), dict(block_x=1, block_y=16),
               dict(block_x=1, block_y=64, max_seqlen_kv=64 * 2049, total_kv=64 * 2049 + 200)):
        v = view(**kw)
        assert v.tile_rows == kw["block_x"] and v.off_row_mask == 0 and v.off_col_mask == 0, kw


def test_fp8_forward_only():
    """e4m3 inputs: forward with an fp16 / bf16 out_dtype and head dim 128;
    no backward variant; head dim 64 has no compiled variant."""
    p = good(dtype=bsa.BSA_DTYPE_FP8_E4M3, out_dtype=bsa.BSA_DTYPE_BF16)
    assert status(p, fwd=True, bwd=False) == bsa.BSA_OK
    assert status(p, fwd=False, bwd=True) == bsa.BSA_ERR_INNER
    assert status(good(dtype=bsa.BSA_DTYPE_FP8_E4M3, out_dtype=bsa.BSA_DTYPE_F16), bwd=False) == bsa.BSA_OK
    assert status(good(dtype=bsa.BSA_DTYPE_FP8_E4M3, out_dtype=bsa.BSA_DTYPE_F16, head_dim=64),
                  bwd=False) == bsa.BSA_ERR_INNER
