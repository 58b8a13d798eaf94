"""CPU checks of the e4m3 input type and of the error bound the e4m3 forward
is tested against (no GPU).

* round_to_e4m3 against values fixed by the FLOAT8_E4M3 format (OCP e4m3fn:
  bias 7, 3 mantissa bits, subnormal step 2^-9, largest finite 448, ties to
  the even code);
* the bound of fp8_tol against a direct simulation of the kernel's rounding
  of P: O = sum_j q8(c p_j) v_j / (c l) for several reference-maximum
  factors c, on seeded e4m3 cases.
"""
import numpy as np
import pytest

import fp8_tol
import oracle.ref as ref
import synth


@pytest.mark.parametrize("x,code,val", [
    (0.0, 0x00, 0.0),
    (1.0, 0x38, 1.0),
    (-1.0, 0xB8, -1.0),
    (1.0625, 0x38, 1.0),     # halfway between 1 and 1.125: even code 0x38
    (1.1875, 0x3A, 1.25),    # halfway between 1.125 and 1.25: even code 0x3A
    (448.0, 0x7E, 448.0),    # largest finite
    (2.0 ** -9, 0x01, 2.0 ** -9),   # smallest subnormal
    (2.0 ** -10, 0x00, 0.0),        # halfway to zero: even code 0
    (3 * 2.0 ** -11, 0x01, 2.0 ** -9),
    (2.0 ** -6, 0x08, 2.0 ** -6),   # smallest normal
    (0.3, 0x2A, 0.3125),
    (240.0, 0x77, 240.0),
])
def test_e4m3_rounding(x, code, val):
    c, v = synth.round_to_e4m3(np.array([x], dtype=np.float32))
    assert int(c[0]) == code and float(v[0]) == val


def test_e4m3_codes_round_trip():
    """Every finite code's value rounds back to itself."""
    vals = synth._E4M3.astype(np.float32)
    c, v = synth.round_to_e4m3(np.concatenate([vals, -vals[1:]]))
    assert np.array_equal(c[:127], np.arange(127)) and np.array_equal(c[127:], np.arange(1, 127) | 0x80)
    assert np.array_equal(v[:127], vals)


@pytest.mark.parametrize("seed,kw", [
    (301, dict(lens_q=[200, 90], N1=2, kind="mask", density=0.6)),
    (302, dict(lens_q=[150], lens_kv=[700], N1=4, N2=2, kind="idx", sparse_heads=2, width=4, causal=True)),
])
def test_fp8_bound_covers_simulated_rounding(seed, kw):
    case = synth.random_case(seed, D=128, dtype="fp8", out_dtype="bf16", with_dout=False, **kw)
    bound, O_ref = fp8_tol.o_bound(case)
    sq, skv, nqb, nkb, qbase, kbase = ref._blocking(case)
    worst = 0.0
    for c in (1.0, 1.37, 5.2, 100.0, 255.0):
        for b in range(case.B):
            for h in range(case.N1):
                for qb in range(nqb[b]):
                    t, p, v = fp8_tol.row_terms(case, b, h, qb)
                    ell = p.sum(axis=1, keepdims=True)
                    ok = ell[:, 0] > 0
                    _, pq = synth.round_to_e4m3((c * p).astype(np.float32))
                    o = (pq.astype(np.float64) @ v) / (c * np.where(ell > 0, ell, 1.0))
                    err = np.abs(o - O_ref[t, h])[ok]
                    bnd = bound[t, h][ok]
                    assert (err <= bnd).all(), f"c={c}: error exceeds the bound"
                    worst = max(worst, float((err / bnd).max()) if ok.any() else 0.0)
    print(f"largest error / bound: {worst:.3f}")
    assert worst > 0.05, "bound implausibly loose"
