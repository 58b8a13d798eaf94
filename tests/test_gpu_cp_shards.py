"""Context-parallel shards on the GPU: a causal sequence split into query
shards, each run as a band-masked case (tests/cp_shards.py), gives the whole
sequence's O, lse and dQ rows, and its dK / dV as the sum of the shards'
partial gradients; query rows whose keys are split over two shards merge
through their lse.  Every shard output is checked against the oracle of the
whole sequence with the parity tolerances (O: 1e-2 plus half a bf16 ulp at
|O|; lse 1e-3; gradients 2e-2 relative Frobenius)."""
import sys

import numpy as np
import pytest
import torch

import cp_shards
import oracle
import synth
from block_sparse_varlen_amd.runner import DeviceCase

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE, TOL_G = 1e-2, 1e-3, 2e-2


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def half_ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
    return 2.0 ** (e - 8)


def rel_fro(x, r):
    return np.linalg.norm((x - r).ravel()) / np.linalg.norm(r.ravel())


def run(case, bwd=True):
    dc = DeviceCase(case, with_bwd=bwd)
    dc.fwd()
    if bwd:
        dc.bwd()
    torch.cuda.synchronize()
    out = dict(O=dc.out.float().cpu().numpy().astype(np.float64), lse=dc.lse.cpu().numpy().astype(np.float64))
    if bwd:
        for n in ("dq", "dk", "dv"):
            out[n] = getattr(dc, n).float().cpu().numpy().astype(np.float64)
    return out


def check_rows(O, lse, Or, Lr, tag):
    d = np.abs(O - Or)
    worst = (d / (TOL_O + half_ulp_bf16(np.abs(Or) + TOL_O))).max()
    lerr = np.abs(lse - Lr).max()
    say(f"  {tag}: max|dO| {d.max():.3e} (err/bound {worst:.3f}) max|dlse| {lerr:.3e}")
    assert worst <= 1.0 and lerr <= TOL_LSE, tag


def test_query_shards_and_key_split_merge():
    case = synth.random_case(91, lens_q=[1500], lens_kv=[1900], N1=4, N2=2, D=128, kind="none", causal=True)
    say("cp shards: oracle of the whole sequence")
    O, lse = oracle.forward(case)
    dq, dk, dv = oracle.backward(case)
    shards = [(0, 700), (700, 800)]
    got = []
    for qs, nq in shards:
        s = cp_shards.shard(case, qs, nq, 0, 1900)
        say(f"cp shard rows {qs}..{qs + nq} (next_tokens {s.band[1]})")
        r = run(s)
        check_rows(r["O"], r["lse"], O[qs:qs + nq], lse[qs:qs + nq], f"rows {qs}..{qs + nq}")
        got.append(r)
    gq = np.concatenate([r["dq"] for r in got])
    gk = sum(r["dk"] for r in got)
    gv = sum(r["dv"] for r in got)
    eq, ek, ev = rel_fro(gq, dq), rel_fro(gk, dk), rel_fro(gv, dv)
    say(f"  gradients: rel_fro dq {eq:.3e} dk (sum of shards) {ek:.3e} dv {ev:.3e}")
    assert eq <= TOL_G and ek <= TOL_G and ev <= TOL_G
    # rows 700..1499 with their keys split at 900, merged through the lse
    parts = []
    for ks, nk in ((0, 900), (900, 1000)):
        r = run(cp_shards.shard(case, 700, 800, ks, nk), bwd=False)
        parts.append((r["O"], r["lse"]))
    Om, lm = cp_shards.merge(parts)
    check_rows(Om, lm, O[700:], lse[700:], "rows 700..1499, keys split at 900, merged")
