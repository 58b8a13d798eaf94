"""Marshalling helpers: put an input set on the GPU and call the C entry
points through the binding.  ``case`` is any object with the attributes of
``synth.Case`` (shapes, dtypes, selection and the ``*_bits`` storage arrays).
No attention arithmetic happens here.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import (
    BSA_DTYPE_BF16, BSA_DTYPE_F16, BSA_DTYPE_FP8_E4M3, BSA_KV_PAGED, BSA_KV_TND, BSA_MASK_BAND, BSA_MASK_CAUSAL,
    BSA_MASK_NONE,
    BSA_FLAG_INDEX_BUILT, BSA_SPARSE_BLOCK_MASK, BSA_SPARSE_IDX_BATCH_I32, BSA_SPARSE_IDX_I32,
    BSA_SPARSE_KV_IDX_BATCH_I32, BSA_SPARSE_KV_IDX_I32, BSA_SPARSE_NONE, BSA_SPARSE_SABI_U16,
    bsa_build_index, bsa_bwd, bsa_fwd, bsa_get_workspace_size, bsa_index_view, problem,
)

_DTYPE = {"bf16": BSA_DTYPE_BF16, "f16": BSA_DTYPE_F16, "fp8": BSA_DTYPE_FP8_E4M3}
_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "fp8": torch.uint8}
_KIND = {"none": BSA_SPARSE_NONE, "mask": BSA_SPARSE_BLOCK_MASK, "sabi": BSA_SPARSE_SABI_U16,
         "idx": BSA_SPARSE_IDX_I32, "idx_b": BSA_SPARSE_IDX_BATCH_I32, "kvidx": BSA_SPARSE_KV_IDX_I32,
         "kvidx_b": BSA_SPARSE_KV_IDX_BATCH_I32}


def problem_for(case):
    lens_q = np.diff(case.cu_q)
    if case.paged:
        lens_kv = np.asarray(case.seqused_kv, dtype=np.int64)
    else:
        lens_kv = np.diff(case.cu_kv)
    sp = case.sparse
    band = getattr(case, "band", None)
    if band is not None:
        mask = dict(mask_type=BSA_MASK_BAND, pre_tokens=int(band[0]), next_tokens=int(band[1]))
    else:
        mask = dict(mask_type=BSA_MASK_CAUSAL if case.causal else BSA_MASK_NONE)
    return problem(
        dtype=_DTYPE[case.dtype],
        out_dtype=_DTYPE[case.out_dtype] if getattr(case, "out_dtype", "") else 0,
        batch=case.B, num_heads_q=case.N1, num_heads_kv=case.N2, head_dim=case.D,
        total_q=int(case.cu_q[-1]), total_kv=int(case.k_bits.shape[0]),
        max_seqlen_q=int(lens_q.max()) if case.B else 0,
        max_seqlen_kv=int(lens_kv.max()) if case.B else 0,
        block_x=case.bx, block_y=case.by, sparse_kind=_KIND[case.sparse_kind],
        sparse_heads=case.sparse_heads,
        sparse_rows=int(sp.shape[-2]) if sp is not None else 0,
        sparse_width=int(sp.shape[-1]) if sp is not None else 0,
        kv_layout=BSA_KV_PAGED if case.paged else BSA_KV_TND,
        page_size=case.page_size if case.paged else 0,
        max_pages_per_seq=int(case.block_table.shape[1]) if case.paged else 0,
        page_stride=case.page_size * case.N2 * case.D if case.paged else 0,
        scale=float(case.scale),
        **mask,
    )


def _dev(a, device, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def ctypes_copy(dst, src):
    ctypes.memmove(ctypes.byref(dst), ctypes.byref(src), ctypes.sizeof(src))


class DeviceCase:
    """Inputs resident on the GPU plus output and workspace buffers."""

    def __init__(self, case, device="cuda", with_bwd=None, flags=0):
        self.case = case
        self.p = problem_for(case)
        self.p.flags |= flags  # e.g. BSA_FLAG_DQ_ATOMIC (sizes the workspace too)
        tdt = _TORCH[case.dtype]  # inputs (e4m3 codes as uint8)
        odt = _TORCH[case.out_dtype] if getattr(case, "out_dtype", "") else tdt  # outputs
        self.tdt = tdt
        self.odt = odt
        self.q = _dev(case.q_bits, device, tdt)
        self.k = _dev(case.k_bits, device, tdt)
        self.v = _dev(case.v_bits, device, tdt)
        self.dout = _dev(case.dout_bits, device, tdt) if case.dout_bits is not None else None
        self.cu_q = _dev(case.cu_q.astype(np.int64), device)
        self.cu_kv = _dev(case.cu_kv.astype(np.int64), device) if case.cu_kv is not None else None
        self.seqused_kv = _dev(case.seqused_kv.astype(np.int32), device) if case.seqused_kv is not None else None
        sp = case.sparse
        if sp is not None and case.sparse_kind == "sabi":
            self.sparse = _dev(sp.astype(np.uint16).view(np.int16), device)
        elif sp is not None and case.sparse_kind == "mask":
            self.sparse = _dev(sp.astype(np.uint8), device)
        elif sp is not None:
            self.sparse = _dev(sp.astype(np.int32), device)
        else:
            self.sparse = None
        self.count = _dev(case.count.astype(np.int32), device) if case.count is not None else None
        self.block_table = _dev(case.block_table.astype(np.int32), device) if case.block_table is not None else None
        T, N1, D = int(case.cu_q[-1]), case.N1, case.D
        self.out = torch.empty((T, N1, D), dtype=odt, device=device)
        self.lse = torch.empty((T, N1), dtype=torch.float32, device=device)
        want_bwd = (self.dout is not None) if with_bwd is None else with_bwd
        fwd_b, bwd_b = bsa_get_workspace_size(self.p, True, want_bwd)
        self.ws_fwd_bytes = fwd_b
        self.ws_bwd_bytes = bwd_b
        self.ws = torch.empty((max(fwd_b, bwd_b or 0),), dtype=torch.uint8, device=device)
        if want_bwd:
            self.dq = torch.empty_like(self.q)
            self.dk = torch.empty_like(self.k)
            self.dv = torch.empty_like(self.v)

    def _prob(self, prebuilt: bool):
        if not prebuilt:
            return self.p
        p = type(self.p)()
        ctypes_copy(p, self.p)
        p.flags |= BSA_FLAG_INDEX_BUILT
        return p

    def build_index(self, with_csc: bool, stream=None):
        """Enqueues the block index build into the workspace (no readback)."""
        bsa_build_index(self.p, self.cu_q, self.cu_kv, self.seqused_kv, self.sparse, self.count, with_csc,
                        self.ws, None, stream)

    def fwd(self, stream=None, prebuilt: bool = False):
        """``prebuilt``: use the index build_index() left in the workspace."""
        bsa_fwd(self._prob(prebuilt), self.q, self.k, self.v, self.cu_q, self.cu_kv, self.seqused_kv, self.sparse,
                self.count, self.block_table, self.out, self.lse, self.ws, None, stream)

    def bwd(self, stream=None, prebuilt: bool = False):
        """``prebuilt``: use the index build_index(with_csc=True) left in the workspace."""
        bsa_bwd(self._prob(prebuilt), self.q, self.k, self.v, self.out, self.dout, self.lse, self.cu_q,
                self.cu_kv, self.seqused_kv, self.sparse, self.count, self.block_table, self.dq, self.dk, self.dv,
                self.ws, None, stream)

    def index(self, with_csc: bool):
        """Builds the block index and returns its products as numpy arrays."""
        bsa_build_index(self.p, self.cu_q, self.cu_kv, self.seqused_kv, self.sparse, self.count, with_csc,
                        self.ws)
        torch.cuda.synchronize()
        v = bsa_index_view(self.p, with_csc)
        ws = self.ws.cpu().numpy()

        def arr(off, n):
            return np.frombuffer(ws[off:off + 4 * n].tobytes(), dtype=np.int32).copy()

        hdr = arr(v.off_header, 8)
        tqb, tkb, R, C, nnz, kvi = (int(x) for x in hdr[:6])
        out = dict(TQB=tqb, TKB=tkb, R=R, nnz=nnz, row_ptr=arr(v.off_row_ptr, R + 1),
                   cols=arr(v.off_cols, nnz), work=arr(v.off_work, R), tile_rows=int(v.tile_rows))
        if v.off_row_mask:
            out["row_mask"] = arr(v.off_row_mask, 4 * nnz).view(np.uint32).reshape(-1, 4)
        if with_csc:
            out.update(C=C, col_ptr=arr(v.off_col_ptr, C + 1), qrows=arr(v.off_qrows, nnz),
                       work_kv=arr(v.off_work_kv, kvi))
            if v.off_col_mask:
                out["col_mask"] = arr(v.off_col_mask, 4 * nnz).view(np.uint32).reshape(-1, 4)
        return out
