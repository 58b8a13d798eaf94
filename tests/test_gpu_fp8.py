"""GPU parity of the e4m3 forward (GenericBlockSparseAttention quantType 5)
with the oracle: O within the bound derived in fp8_tol (the rounding of P to
e4m3 is the only error beyond fp32 and the output rounding), lse within
1e-3, +inf lse on the same rows."""
import sys

import numpy as np
import pytest
import torch

import fp8_tol
import oracle
import synth
from block_sparse_varlen_amd.runner import DeviceCase

pytestmark = pytest.mark.gpu


def cases():
    R = synth.random_case
    F = dict(D=128, dtype="fp8", with_dout=False)
    return {
        "mask_bf16": R(401, lens_q=[300, 0, 517], N1=2, kind="mask", out_dtype="bf16", **F),
        "mask_gqa_causal_f16": R(402, lens_q=[200, 385], N1=4, N2=2, kind="mask", sparse_heads=2, causal=True,
                                 density=0.6, out_dtype="f16", **F),
        "sabi_messy_by256": R(403, lens_q=[257, 130], lens_kv=[600, 70], N1=2, kind="sabi", by=256, messy=True,
                              out_dtype="bf16", **F),
        "idx_paged_causal": R(404, lens_q=[500, 310], lens_kv=[400, 700], N1=4, N2=2, kind="idx",
                              sparse_heads=2, causal=True, paged=True, out_dtype="bf16", **F),
        "none_bx64_long_kv": R(405, lens_q=[100, 180], lens_kv=[1500, 900], N1=2, kind="none", bx=64,
                               out_dtype="bf16", **F),
        "sabi_bx16_causal_f16": R(406, lens_q=[150, 77], N1=2, kind="sabi", bx=16, causal=True,
                                  out_dtype="f16", **F),
        "mask_paged_ps64_perhead": R(407, lens_q=[300, 200], lens_kv=[333, 450], N1=4, N2=2, kind="mask",
                                     paged=True, page_size=64, out_dtype="bf16", **F),
        # a large scale: frequent moves of the reference maximum (P stays <= 256)
        "mask_scale08": R(408, lens_q=[400, 300], N1=2, kind="mask", scale=0.8, density=0.7, out_dtype="bf16",
                          **F),
        # band mask with Sq != Skv
        "sabi_band_f16": R(409, lens_q=[450, 200], lens_kv=[520, 330], N1=2, kind="sabi", band=(150, 30),
                           dense_q=True, out_dtype="f16", **F),
        # 48-key blocks: 64-key windows with masked groups
        "mask_by48_paged": R(410, lens_q=[300, 200], lens_kv=[333, 450], N1=4, N2=2, kind="mask", by=48,
                             paged=True, out_dtype="bf16", **F),
        # per-token selection as 128-row tiles with row masks
        "tile_idx_bx1_gqa_causal": R(411, lens_q=[700, 129], N1=4, N2=2, kind="idx", sparse_heads=2, bx=1,
                                     width=5, causal=True, out_dtype="bf16", **F),
        "tile_mask_bx8_band_f16": R(412, lens_q=[333, 200], lens_kv=[500, 250], N1=2, kind="mask", bx=8, by=64,
                                    density=0.4, band=(150, 20), out_dtype="f16", **F),
    }


CASES = cases()


@pytest.mark.parametrize("name", list(CASES))
def test_fwd_fp8(name):
    case = CASES[name]
    print(f"fp8 fwd {name}", flush=True)
    sys.stdout.flush()
    dc = DeviceCase(case, with_bwd=False)
    dc.out.fill_(float("nan"))
    dc.lse.fill_(float("nan"))
    dc.fwd()
    torch.cuda.synchronize()
    O = dc.out.float().cpu().numpy()
    L = dc.lse.cpu().numpy()
    bound, O_ref = fp8_tol.o_bound(case)
    _, L_ref = oracle.forward(case)
    err = np.abs(O - O_ref)
    ratio = float((err / bound).max()) if err.size else 0.0
    inf_r = np.isinf(L_ref)
    assert np.array_equal(np.isinf(L), inf_r), "+inf lse positions differ"
    fin = ~inf_r
    lerr = float(np.abs(L[fin] - L_ref[fin]).max()) if fin.any() else 0.0
    print(f"  {name}: max|dO|={err.max():.3e} max err/bound={ratio:.3f} max|dlse|={lerr:.3e}", flush=True)
    assert not np.isnan(O).any()
    assert ratio <= 1.0, f"O error above the e4m3 bound ({ratio:.3f})"
    assert lerr <= 1e-3


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n", [3, 5])
def test_fwd_fp8_config(n):
    """Full-size sabi prefill and long-context workloads in e4m3 (the
    bench's --fp8 lines), checked on sampled q-blocks: the longest rows,
    random ones and every sequence's last q-block."""
    from test_gpu_parity import _sample_rows
    print(f"fp8 config {n}: generating", flush=True)
    case = synth.to_fp8(synth.CONFIGS[n](), "bf16")
    dc = DeviceCase(case, with_bwd=False)
    dc.out.fill_(float("nan"))
    dc.lse.fill_(float("nan"))
    print(f"fp8 config {n}: fwd on GPU", flush=True)
    dc.fwd()
    torch.cuda.synchronize()
    assert not torch.isnan(dc.out).any() and not torch.isnan(dc.lse).any()
    idx = oracle.index_products(case, with_csc=False)
    sample = sorted(_sample_rows(case, idx, 16, n))
    bound, O_ref = fp8_tol.o_bound(case, sample)
    _, L_ref = oracle.forward(case, sample)
    sel = ~np.isnan(L_ref)
    O = dc.out.float().cpu().numpy()
    L = dc.lse.cpu().numpy()
    ratio = float((np.abs(O - O_ref)[sel] / bound[sel]).max())
    lerr = float(np.abs(L[sel] - L_ref[sel]).max())
    print(f"  config {n}: rows={int(sel.sum())} max err/bound={ratio:.3f} max|dlse|={lerr:.3e}", flush=True)
    assert ratio <= 1.0 and lerr <= 1e-3
