"""The allocation-free forward entry point (bsa_fwd_noalloc), called through
the C ABI: same results as bsa_fwd with a caller workspace, bit for bit, on two
calls in a row (the second with a smaller problem, so it reuses the library's
scratch left by the first), and a clear error for a problem whose index does
not fit the scratch."""
import sys

import numpy as np
import pytest
import torch

import synth
import block_sparse_varlen_amd as bsa
from block_sparse_varlen_amd.runner import DeviceCase

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _noalloc(dc, out, lse):
    bsa.bsa_fwd_noalloc(dc.p, dc.q, dc.k, dc.v, dc.cu_q, dc.cu_kv, dc.seqused_kv, dc.sparse, dc.count,
                        dc.block_table, out, lse)


def _same(case, tag):
    dc = DeviceCase(case, with_bwd=False)
    dc.out.fill_(float("nan"))
    dc.lse.fill_(float("nan"))
    dc.fwd()
    o2 = torch.full_like(dc.out, float("nan"))
    l2 = torch.full_like(dc.lse, float("nan"))
    _noalloc(dc, o2, l2)
    torch.cuda.synchronize()
    say(f"  {tag}: fwd workspace {dc.ws_fwd_bytes} B")
    assert torch.equal(dc.out.view(torch.int16), o2.view(torch.int16)), f"{tag}: out differs"
    assert torch.equal(dc.lse.view(torch.int32), l2.view(torch.int32)), f"{tag}: lse differs"


def test_noalloc_matches_workspace_entry_point():
    say("noalloc: larger case, then a smaller one")
    big = synth.random_case(301, lens_q=[900, 650, 1300], N1=4, N2=2, D=128, kind="idx", sparse_heads=2,
                            causal=True, paged=True, messy=True, with_dout=False)
    small = synth.random_case(302, lens_q=[200, 70], N1=2, D=64, dtype="f16", kind="mask", with_dout=False)
    _same(big, "big")
    _same(small, "small")
    # and the long-context workload's shape of index (block-causal mask)
    _same(synth.config1(), "tiny")
    # per-token selection as 128-row tiles (row masks in the scratch index)
    _same(synth.random_case(303, lens_q=[700, 129], N1=4, N2=2, D=128, kind="idx", sparse_heads=2, bx=1, width=5,
                            causal=True, with_dout=False), "row tiles")


def test_noalloc_rejects_oversize_problem():
    say("noalloc: oversize index")
    # 4096 sequences x 64 heads of 128-token q-blocks: the forward index needs
    # more than the library's scratch array
    T = 4096 * 256
    p = bsa.problem(dtype=bsa.BSA_DTYPE_BF16, batch=4096, num_heads_q=64, num_heads_kv=64, head_dim=128,
                    total_q=T, total_kv=T, max_seqlen_q=256, max_seqlen_kv=256, block_x=128, block_y=128,
                    sparse_kind=bsa.BSA_SPARSE_NONE, sparse_heads=64, mask_type=bsa.BSA_MASK_CAUSAL,
                    kv_layout=bsa.BSA_KV_TND)
    fwd, _ = bsa.bsa_get_workspace_size(p, True, False)
    assert fwd > bsa.NOALLOC_SCRATCH_BYTES
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_fwd_noalloc(p, 1, 1, 1, 1, 1, None, None, None, None, 1, 1)
    assert e.value.status == bsa.BSA_ERR_PARAM_INVALID
    # a prebuilt index cannot be handed in
    p2 = bsa.problem(dtype=bsa.BSA_DTYPE_BF16, batch=1, num_heads_q=2, num_heads_kv=2, head_dim=64, total_q=128,
                     total_kv=128, max_seqlen_q=128, max_seqlen_kv=128, block_x=128, block_y=128,
                     sparse_kind=bsa.BSA_SPARSE_NONE, sparse_heads=2, flags=bsa.BSA_FLAG_INDEX_BUILT)
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_fwd_noalloc(p2, 1, 1, 1, 1, 1, None, None, None, None, 1, 1)
    assert e.value.status == bsa.BSA_ERR_PARAM_INVALID
