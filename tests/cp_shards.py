"""Context-parallel shards of a one-sequence causal case: the queries
[qs, qs + nq) against the keys [ks, ks + nk), as a case of their own whose
band mask reproduces the whole sequence's causal rule.  Key j of the shard is
global key j + ks and query i is global query i + qs; the whole sequence
allows J <= I + (Skv - Sq), and the shard's band allows
j <= i + (nk - nq) + next_tokens, so next_tokens = qs - ks + (Skv - Sq) -
(nk - nq), with no lower end."""
import dataclasses

import numpy as np

UNBOUNDED = 2 ** 40


def next_tokens(case, qs, nq, ks, nk):
    sq, skv = int(case.lens_q[0]), int(case.lens_kv[0])
    return qs - ks + (skv - sq) - (nk - nq)


def shard(case, qs, nq, ks, nk):
    assert case.B == 1 and case.causal and case.sparse_kind == "none" and not case.paged
    cu_q = np.array([0, nq], dtype=np.int64)
    cu_kv = np.array([0, nk], dtype=np.int64)
    rows = slice(qs, qs + nq)
    keys = slice(ks, ks + nk)
    return dataclasses.replace(
        case, name=f"{case.name}_q{qs}_k{ks}", causal=False, band=(UNBOUNDED, next_tokens(case, qs, nq, ks, nk)),
        cu_q=cu_q, cu_kv=cu_kv, q_bits=case.q_bits[rows], q=case.q[rows], k_bits=case.k_bits[keys], k=case.k[keys],
        v_bits=case.v_bits[keys], v=case.v[keys],
        dout_bits=None if case.dout_bits is None else case.dout_bits[rows],
        dout=None if case.dout is None else case.dout[rows])


def merge(parts):
    """Merges (O, lse) of shards over disjoint key ranges of the same rows:
    lse = log sum exp lse_s, O = sum exp(lse_s - lse) O_s (an empty shard
    stores lse = +inf, a log-sum of -inf)."""
    ls = [np.where(np.isinf(l), -np.inf, l) for _, l in parts]
    lm = ls[0]
    for l in ls[1:]:
        lm = np.logaddexp(lm, l)
    O = 0.0
    with np.errstate(invalid="ignore"):
        for (o, _), l in zip(parts, ls):
            w = np.where(np.isfinite(l), np.exp(l - lm), 0.0)
            O = O + w[..., None] * o
    return O, lm
