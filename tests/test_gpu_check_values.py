"""BSA_FLAG_CHECK_VALUES on the GPU.  Consistent inputs give bit-identical
results with and without the flag and a zero check word.  Each inconsistency
the flag checks comes back as BSA_ERR_PARAM_INVALID with its BSA_CHECK_* bits
in header[6] of the workspace, and the call leaves its outputs untouched: no
kernel past the validator ran.  The validator reads each array only inside
its declared extent, so these inputs are safe to hand it."""
import sys

import numpy as np
import pytest
import torch

import synth
import block_sparse_varlen_amd as bsa
from block_sparse_varlen_amd.runner import DeviceCase

pytestmark = pytest.mark.gpu

LENS = [200, 300, 100]  # max_seqlen 300, total 600 tokens


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def checked(case):
    return DeviceCase(case, with_bwd=True, flags=bsa.BSA_FLAG_CHECK_VALUES)


def word(dc):
    torch.cuda.synchronize()
    off = bsa.bsa_index_view(dc.p, False).off_header
    return int(dc.ws[off + 24:off + 28].cpu().numpy().view(np.int32)[0])


def fwd(dc, cu_q=None, cu_kv=None, seqused=None, bt=None):
    bsa.bsa_fwd(dc.p, dc.q, dc.k, dc.v, dc.cu_q if cu_q is None else cu_q, dc.cu_kv if cu_kv is None else cu_kv,
                dc.seqused_kv if seqused is None else seqused, dc.sparse, dc.count,
                dc.block_table if bt is None else bt, dc.out, dc.lse, dc.ws)


def bwd(dc, cu_q=None, cu_kv=None, seqused=None, bt=None):
    bsa.bsa_bwd(dc.p, dc.q, dc.k, dc.v, dc.out, dc.dout, dc.lse, dc.cu_q if cu_q is None else cu_q,
                dc.cu_kv if cu_kv is None else cu_kv, dc.seqused_kv if seqused is None else seqused, dc.sparse,
                dc.count, dc.block_table if bt is None else bt, dc.dq, dc.dk, dc.dv, dc.ws)


def tnd_case():
    return synth.random_case(501, lens_q=LENS, N1=2, D=64, kind="mask", density=0.6)


def paged_case():
    return synth.random_case(502, lens_q=LENS, N1=2, D=64, kind="mask", density=0.6, paged=True, page_size=128)


@pytest.mark.parametrize("make", [tnd_case, paged_case], ids=["tnd", "paged"])
def test_consistent_values_pass_and_change_nothing(make):
    case = make()
    say(f"check_values consistent {case.name}")
    ref = DeviceCase(case, with_bwd=True)
    dc = checked(case)
    for d in (ref, dc):  # paged dK / dV leave the pool's unused slots as they were
        d.dk.zero_()
        d.dv.zero_()
    ref.fwd()
    ref.bwd()
    fwd(dc)
    assert word(dc) == 0
    bwd(dc)
    assert word(dc) == 0
    torch.cuda.synchronize()
    for n in ("out", "lse", "dq", "dk", "dv"):
        a, b = getattr(ref, n), getattr(dc, n)
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a,
                           b.view(torch.uint8) if b.dtype != torch.float32 else b), n


def _sentinel(dc):
    for n in ("out", "dq", "dk", "dv"):
        getattr(dc, n).fill_(7.0)
    dc.lse.fill_(-3.0)


def _untouched(dc):
    torch.cuda.synchronize()
    for n in ("out", "dq", "dk", "dv"):
        assert bool((getattr(dc, n).float() == 7.0).all()), n
    assert bool((dc.lse == -3.0).all())


def _i64(xs):
    return torch.tensor(xs, dtype=torch.int64, device="cuda")


def _i32(xs):
    return torch.tensor(xs, dtype=torch.int32, device="cuda")


# (name, argument, values, expected bits); cu_seqlens of LENS are [0, 200, 500, 600]
TND_BAD = [
    ("cu_q_first", "cu_q", [10, 200, 500, 600], bsa.BSA_CHECK_CU_Q_ENDS),
    ("cu_q_last", "cu_q", [0, 200, 500, 590], bsa.BSA_CHECK_CU_Q_ENDS),
    ("sq_long", "cu_q", [0, 320, 500, 600], bsa.BSA_CHECK_SQ_LONG),
    # a decrease has to be made up by a sequence longer than max_seqlen_q
    ("cu_q_order", "cu_q", [0, 250, 200, 600], bsa.BSA_CHECK_CU_Q_ORDER | bsa.BSA_CHECK_SQ_LONG),
    ("cu_kv_last", "cu_kv", [0, 200, 500, 700], bsa.BSA_CHECK_CU_KV_ENDS),
    ("cu_kv_first", "cu_kv", [-4, 200, 500, 600], bsa.BSA_CHECK_CU_KV_ENDS),
    ("skv_long", "cu_kv", [0, 320, 500, 600], bsa.BSA_CHECK_SKV_LONG),
    ("cu_kv_order", "cu_kv", [0, 250, 200, 600], bsa.BSA_CHECK_CU_KV_ORDER | bsa.BSA_CHECK_SKV_LONG),
]


@pytest.mark.parametrize("name,arg,vals,bits", TND_BAD, ids=[t[0] for t in TND_BAD])
def test_inconsistent_cu_seqlens_are_rejected(name, arg, vals, bits):
    say(f"check_values tnd {name}")
    dc = checked(tnd_case())
    bad = {arg: _i64(vals)}
    for call in (fwd, bwd):
        _sentinel(dc)
        with pytest.raises(bsa.BsaError) as e:
            call(dc, **bad)
        assert e.value.status == bsa.BSA_ERR_PARAM_INVALID
        assert word(dc) == bits, (call.__name__, word(dc))
        _untouched(dc)
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_build_index(dc.p, bad.get("cu_q", dc.cu_q), bad.get("cu_kv", dc.cu_kv), None, dc.sparse, dc.count,
                            True, dc.ws)
    assert e.value.status == bsa.BSA_ERR_PARAM_INVALID and word(dc) == bits
    # the same workspace then serves a consistent call as usual
    fwd(dc)
    assert word(dc) == 0


def test_paged_values():
    """seqused_kv outside [0, max_seqlen_kv] and block_table entries outside
    the page pool are reported for the pages a pass would read; an entry past
    a sequence's last used page is never read, so it passes."""
    case = paged_case()
    dc = checked(case)
    ref = DeviceCase(case, with_bwd=True)
    ref.fwd()
    bt = case.block_table.astype(np.int64)
    pages = int(dc.p.total_kv)  # pages in the pool
    assert bt.shape == (3, dc.p.max_pages_per_seq)

    def table(i, j, val):
        t = bt.copy()
        t[i, j] = val
        return _i32(t.astype(np.int32))

    bad = [
        ("seqused_long", dict(seqused=_i32([200, 301, 100])), bsa.BSA_CHECK_SKV_LONG),
        ("seqused_negative", dict(seqused=_i32([-5, 300, 100])), bsa.BSA_CHECK_SKV_LONG),
        ("page_past_pool", dict(bt=table(0, 1, pages)), bsa.BSA_CHECK_PAGE),
        ("page_negative", dict(bt=table(1, 0, -3)), bsa.BSA_CHECK_PAGE),
    ]
    for name, kw, bits in bad:
        say(f"check_values paged {name}")
        for call in (fwd, bwd):
            _sentinel(dc)
            with pytest.raises(bsa.BsaError) as e:
                call(dc, **kw)
            assert e.value.status == bsa.BSA_ERR_PARAM_INVALID, name
            assert word(dc) == bits, (name, call.__name__, word(dc))
            _untouched(dc)
    # sequence 2 holds 100 keys: only its first page entry is read
    say("check_values paged unused entry")
    fwd(dc, bt=table(2, 2, 9999))
    assert word(dc) == 0
    torch.cuda.synchronize()
    assert torch.equal(dc.out.view(torch.uint8), ref.out.view(torch.uint8))
    assert torch.equal(dc.lse, ref.lse)
