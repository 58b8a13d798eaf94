"""Error bound for the e4m3 forward (GenericBlockSparseAttention quantType 5:
Q, K, V in FLOAT8_E4M3, P cast to e4m3 by the operator before the PV
product).

The scores are exact in fp32 (e4m3 x e4m3 products have 8 significant bits)
and the softmax statistics are fp32, so lse keeps the bf16 path's 1e-3.  O
differs from the exact result by the rounding of P alone:

    O_gpu - O = sum_j (q8(c p_j) - c p_j) v_j / (c l),

with p_j = exp(s_j - m) over the row's allowed keys, l = sum_j p_j and c >= 1
the factor between the kernel's reference maximum and the row maximum (the
kernel moves its reference only when a score exceeds it by more than 8 in
log2 units).  Round-to-nearest-even to e4m3 errs by at most half an ulp:
ulp(x) / x <= 2^-3 for normal values (x >= 2^-6), and 2^-9 absolute below.
So |q8(c p) - c p| <= c * u(p) / 2 with u(p) = max(2^-3 p, 2^-9) (c >= 1
only makes the subnormal term smaller relative to c l).  Treating the
roundings of different keys as independent and uniform, the error of one
output element has standard deviation

    sigma = sqrt(sum_j u(p_j)^2 v_j^2 / 12) / l,

and the test bound is 6 sigma, plus the half-ulp of rounding O itself to the
16-bit output type and a small fp32 allowance.  A CPU simulation of the
quantised sum over several c (tests/test_fp8_model.py) checks the bound.
"""
from __future__ import annotations

import numpy as np

import oracle.ref as ref

OUT_ULP = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def u_bound(p: np.ndarray) -> np.ndarray:
    return np.maximum(p * 2.0 ** -3, 2.0 ** -9)


def row_terms(case, b, h, qb):
    """(token rows, p [rows, keys] with exp(s - m), v [keys, D]) of one
    q-block of q-head h, from the oracle's own row problem."""
    sq, skv, nqb, nkb, qbase, kbase = ref._blocking(case)
    sigma = ref.scale_of(case.scale, case.D)
    G = case.N1 // case.N2
    i_loc, keys, allowed = ref._row_problem(case, b, h, qb, sq, skv, nkb, qbase)
    t = int(case.cu_q[b]) + i_loc
    q = case.q[t, h, :].astype(np.float64)
    k = ref._gather_kv(case, case.k, b, h // G, keys)
    v = ref._gather_kv(case, case.v, b, h // G, keys)
    s = np.where(allowed, sigma * (q @ k.T), -np.inf)
    if s.shape[1] == 0:
        return t, np.zeros_like(s), v
    m = np.where(allowed.any(axis=1, keepdims=True), s.max(axis=1, keepdims=True), 0.0)
    p = np.exp(s - m)
    return t, p, v


def o_bound(case, sample=None):
    """Per-element bound [T_q, N1, D] on |O_gpu - O| for an e4m3 case, and
    the oracle's O.  ``sample``: optional (b, h, qb) triples; entries of
    other q-blocks are NaN in both."""
    sq, skv, nqb, nkb, qbase, kbase = ref._blocking(case)
    T = int(case.cu_q[-1])
    O_ref, _ = ref.forward(case, sample)
    sig = np.full((T, case.N1, case.D), np.nan if sample is not None else 0.0)
    if sample is None:
        sample = [(b, h, qb) for b in range(case.B) for h in range(case.N1) for qb in range(nqb[b])]
    for b, h, qb in sample:
        t, p, v = row_terms(case, b, h, qb)
        ell = p.sum(axis=1, keepdims=True)
        ell = np.where(ell > 0, ell, 1.0)
        var = (u_bound(p) ** 2 * (p > 0)) @ (v ** 2) / 12.0
        sig[t, h, :] = np.sqrt(var) / ell
    return 6.0 * sig + OUT_ULP[case.out_dtype] * np.abs(O_ref) + 1e-5, O_ref
