"""Python binding of libbsa.so -- block-sparse varlen FlashAttention for
MI355X (gfx950).

Argument marshalling only: every function forwards to the C entry point of the
same name in ``include/bsa.h``; all computation runs in the HIP library.
PyTorch supplies device memory and the current HIP stream.  The library must
have been built (``python block_sparse_varlen_amd/build.py``); importing this
module without it raises ``ImportError``.
"""
from __future__ import annotations

import ctypes
import os

# PyTorch ships its own HIP runtime under the same soname (libamdhip64.so.7)
# as the ROCm one libbsa.so links against, and the first library loaded
# serves the whole process.  Loading torch first keeps a single runtime --
# the one that owns the tensors and streams handed to the library; loading
# libbsa.so first would bind torch to a runtime its bundled libraries were
# not built with, and launches then fail.
import torch  # noqa: F401  (runtime selection only)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

BSA_OK = 0
BSA_ERR_PARAM_NULLPTR = 161001
BSA_ERR_PARAM_INVALID = 161002
BSA_ERR_INNER = 561103
BSA_ERR_RUNTIME = 561000

BSA_DTYPE_F16, BSA_DTYPE_BF16, BSA_DTYPE_FP8_E4M3 = 1, 2, 3
BSA_SPARSE_NONE, BSA_SPARSE_BLOCK_MASK, BSA_SPARSE_SABI_U16, BSA_SPARSE_IDX_I32 = 0, 1, 2, 3
BSA_SPARSE_IDX_BATCH_I32, BSA_SPARSE_KV_IDX_I32, BSA_SPARSE_KV_IDX_BATCH_I32 = 4, 5, 6
BSA_MASK_NONE, BSA_MASK_CAUSAL, BSA_MASK_BAND = 0, 1, 2
BSA_KV_TND, BSA_KV_PAGED = 0, 1
BSA_FLAG_INDEX_BUILT, BSA_FLAG_DETERMINISTIC, BSA_FLAG_DQ_ATOMIC = 1, 2, 4
BSA_FLAG_CHECK_VALUES = 8
(BSA_CHECK_CU_Q_ENDS, BSA_CHECK_CU_Q_ORDER, BSA_CHECK_SQ_LONG, BSA_CHECK_CU_KV_ENDS, BSA_CHECK_CU_KV_ORDER,
 BSA_CHECK_SKV_LONG, BSA_CHECK_PAGE) = 1, 2, 4, 8, 16, 32, 64
(BSA_KERNEL_INDEX, BSA_KERNEL_FWD, BSA_KERNEL_BWD_PRE, BSA_KERNEL_BWD_DKDV, BSA_KERNEL_BWD_DQ) = range(5)
KERNEL_NAMES = {0: "index", 1: "fwd", 2: "bwd_pre", 3: "bwd_dkdv", 4: "bwd_dq"}

EXPORTS = (
    "bsa_get_workspace_size", "bsa_fwd", "bsa_fwd_noalloc", "bsa_bwd", "bsa_index_view", "bsa_build_index",
    "bsa_status_string", "bsa_profile_enable", "bsa_profile_reset", "bsa_profile_read",
)


class bsa_problem_t(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_heads_q", ctypes.c_int32),
        ("num_heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("total_q", ctypes.c_int64),
        ("total_kv", ctypes.c_int64),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_kv", ctypes.c_int32),
        ("block_x", ctypes.c_int32),
        ("block_y", ctypes.c_int32),
        ("sparse_kind", ctypes.c_int32),
        ("sparse_heads", ctypes.c_int32),
        ("sparse_rows", ctypes.c_int32),
        ("sparse_width", ctypes.c_int32),
        ("mask_type", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("page_stride", ctypes.c_int64),
        ("scale", ctypes.c_double),
        ("flags", ctypes.c_uint32),
        ("out_dtype", ctypes.c_int32),
        ("pre_tokens", ctypes.c_int64),
        ("next_tokens", ctypes.c_int64),
    ]


class bsa_index_view_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "off_header", "off_row_ptr", "off_cols", "off_work", "off_col_ptr", "off_qrows", "off_work_kv")] + [
        (n, ctypes.c_int64) for n in ("max_rows", "max_cols", "max_nnz", "max_kv_items")] + [
        ("tile_rows", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("off_row_mask", ctypes.c_uint64), ("off_col_mask", ctypes.c_uint64)]


def problem(**fields) -> bsa_problem_t:
    """A descriptor with ``struct_size`` filled in and the given fields."""
    p = bsa_problem_t()
    p.struct_size = ctypes.sizeof(bsa_problem_t)
    for k, v in fields.items():
        if not hasattr(p, k):
            raise TypeError(f"bsa_problem_t has no field {k!r}")
        setattr(p, k, v)
    return p


class BsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python block_sparse_varlen_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S, VP = ctypes.POINTER, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    prob = P(bsa_problem_t)
    lib.bsa_get_workspace_size.argtypes = [prob, P(S), P(S)]
    lib.bsa_fwd.argtypes = [prob] + [VP] * 11 + [VP, S, VP]
    lib.bsa_fwd_noalloc.argtypes = [prob] + [VP] * 11 + [VP]
    lib.bsa_bwd.argtypes = [prob] + [VP] * 15 + [VP, S, VP]
    lib.bsa_index_view.argtypes = [prob, I, P(bsa_index_view_t)]
    lib.bsa_build_index.argtypes = [prob, VP, VP, VP, VP, VP, I, VP, S, VP]
    lib.bsa_status_string.argtypes = [I]
    lib.bsa_status_string.restype = ctypes.c_char_p
    lib.bsa_profile_enable.argtypes = [I]
    lib.bsa_profile_read.argtypes = [I, P(ctypes.c_int64), P(ctypes.c_double)]
    for name in EXPORTS:
        if name != "bsa_status_string":
            getattr(lib, name).restype = I
    return lib


_lib = _load()


def library():
    return _lib


def status_string(status: int) -> str:
    return _lib.bsa_status_string(int(status)).decode()


def _ptr(x):
    """Device/host address of a tensor, an int address, or None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr() or None


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != BSA_OK:
        raise BsaError(status, where)


def bsa_get_workspace_size(p: bsa_problem_t, fwd: bool = True, bwd: bool = True):
    """Returns ``(fwd_bytes, bwd_bytes)``; an entry not asked for is None."""
    f = ctypes.c_size_t(0)
    b = ctypes.c_size_t(0)
    st = _lib.bsa_get_workspace_size(ctypes.byref(p), ctypes.byref(f) if fwd else None,
                                     ctypes.byref(b) if bwd else None)
    _check(st, "bsa_get_workspace_size")
    return (f.value if fwd else None), (b.value if bwd else None)


def bsa_fwd(p, q, k, v, cu_seqlens_q, cu_seqlens_kv, seqused_kv, sparse, sparse_count, block_table,
            out, lse, workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.bsa_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv),
                      _ptr(seqused_kv), _ptr(sparse), _ptr(sparse_count), _ptr(block_table), _ptr(out), _ptr(lse),
                      _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check(st, "bsa_fwd")


NOALLOC_SCRATCH_BYTES = 16 << 20  # BSA_NOALLOC_SCRATCH_BYTES


def bsa_fwd_noalloc(p, q, k, v, cu_seqlens_q, cu_seqlens_kv, seqused_kv, sparse, sparse_count, block_table,
                    out, lse, stream=None):
    st = _lib.bsa_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                              _ptr(cu_seqlens_kv), _ptr(seqused_kv), _ptr(sparse), _ptr(sparse_count),
                              _ptr(block_table), _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "bsa_fwd_noalloc")


def bsa_bwd(p, q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_kv, seqused_kv, sparse, sparse_count,
            block_table, dq, dk, dv, workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.bsa_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                      _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), _ptr(seqused_kv), _ptr(sparse), _ptr(sparse_count),
                      _ptr(block_table), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), int(workspace_bytes),
                      _stream(stream))
    _check(st, "bsa_bwd")


def bsa_index_view(p, with_csc: bool) -> bsa_index_view_t:
    v = bsa_index_view_t()
    _check(_lib.bsa_index_view(ctypes.byref(p), int(bool(with_csc)), ctypes.byref(v)), "bsa_index_view")
    return v


def bsa_build_index(p, cu_seqlens_q, cu_seqlens_kv, seqused_kv, sparse, sparse_count, with_csc, workspace,
                    workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.bsa_build_index(ctypes.byref(p), _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), _ptr(seqused_kv),
                              _ptr(sparse), _ptr(sparse_count), int(bool(with_csc)), _ptr(workspace),
                              int(workspace_bytes), _stream(stream))
    _check(st, "bsa_build_index")


def bsa_profile_enable(enable: bool):
    _check(_lib.bsa_profile_enable(int(bool(enable))), "bsa_profile_enable")


def bsa_profile_reset():
    _check(_lib.bsa_profile_reset(), "bsa_profile_reset")


def bsa_profile_read(kernel: int):
    """Returns ``(launches, total_ms)`` for kernel id ``kernel``."""
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(_lib.bsa_profile_read(int(kernel), ctypes.byref(n), ctypes.byref(ms)), "bsa_profile_read")
    return n.value, ms.value
