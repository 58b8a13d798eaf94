"""Seeded sweep of small random problems through the C ABI: each seed draws a
selection form, block shape, token mask, head layout, KV layout, head dim and
dtype, then checks the block index bit for bit and the forward and backward
outputs against the oracle with the parity tolerances of
tests/test_gpu_parity.py.  The draws are fixed by the seed, so a failure
names a reproducible case."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from block_sparse_varlen_amd.runner import DeviceCase
from test_gpu_parity import check_bwd, check_fwd, nan_fill

pytestmark = pytest.mark.gpu

SEEDS = range(40)
KINDS = ["none", "mask", "sabi", "idx", "idx_b", "kvidx", "kvidx_b"]
HEADS = [(2, 2), (4, 2), (4, 1), (6, 3)]


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def draw(seed):
    rng = np.random.default_rng(7000 + seed)
    kind = KINDS[seed % len(KINDS)]
    B = int(rng.integers(1, 4))
    lens_q = [int(x) for x in rng.integers(0, 701, size=B)]
    lens_q[int(rng.integers(B))] = max(lens_q[0], 1 + int(rng.integers(1, 700)))  # some rows
    lens_kv = list(lens_q) if rng.random() < 0.5 else [int(x) for x in rng.integers(0, 701, size=B)]
    N1, N2 = HEADS[int(rng.integers(len(HEADS)))]
    kw = dict(lens_q=lens_q, lens_kv=lens_kv, N1=N1, N2=N2, D=int(rng.choice([64, 128])),
              dtype=str(rng.choice(["bf16", "f16"])), kind=kind,
              bx=int(rng.choice([1, 4, 16, 32, 64, 96, 128, 192, 256])),
              by=int(rng.choice([16, 48, 64, 128, 192, 256])),
              sparse_heads=int(rng.choice([N1, N2])))
    m = rng.random()
    if m < 0.35:
        kw["causal"] = True
    elif m < 0.6:
        kw["band"] = (int(rng.integers(-20, 401)), int(rng.integers(-20, 401)))
    if rng.random() < 0.3:
        kw.update(paged=True, page_size=int(rng.choice([64, 128, 256])))
    if kw["bx"] <= 4:  # per-token selections: keep the oracle's per-row work small
        kw["lens_q"] = [min(x, 400) for x in kw["lens_q"]]
        kw["lens_kv"] = [min(x, 400) for x in kw["lens_kv"]]
    if kind == "mask":
        kw["density"] = float(rng.uniform(0.2, 0.9))
    if kind in ("sabi", "idx", "idx_b", "kvidx", "kvidx_b") and rng.random() < 0.3:
        kw["messy"] = True
    return kw


def label(seed):
    kw = draw(seed)
    mask = "causal" if kw.get("causal") else ("band" if "band" in kw else "nomask")
    return (f"{seed}-{kw['kind']}-bx{kw['bx']}-by{kw['by']}-{mask}-n{kw['N1']}x{kw['N2']}-d{kw['D']}-{kw['dtype']}"
            + ("-paged" if kw.get("paged") else ""))


@pytest.mark.parametrize("seed", SEEDS, ids=[label(s) for s in SEEDS])
def test_random_problem(seed):
    kw = draw(seed)
    case = synth.random_case(8000 + seed, **kw)
    say(f"sweep {label(seed)} lens_q={kw['lens_q']} lens_kv={kw['lens_kv']}")
    dc = DeviceCase(case, with_bwd=True)
    got = dc.index(True)
    keys = ["row_ptr", "cols", "work", "col_ptr", "qrows", "work_kv"]
    if got["tile_rows"] != case.bx:
        ref = oracle.tile_index_products(case, got["tile_rows"], with_csc=True)
        keys += ["row_mask", "col_mask"]
    else:
        ref = oracle.index_products(case, with_csc=True)
    for k in keys:
        assert np.array_equal(got[k], ref[k]), k
    nan_fill(dc.out, dc.lse)
    dc.fwd()
    torch.cuda.synchronize()
    check_fwd(case, dc, tag=label(seed))
    nan_fill(dc.dq, dc.dk, dc.dv)
    dc.bwd()
    torch.cuda.synchronize()
    check_bwd(case, dc, tag=label(seed))
