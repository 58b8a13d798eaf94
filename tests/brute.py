"""Brute-force reference used to pin the oracle (test code, CPU only).

It never looks at blocks as a unit of work: for every (query token, key token)
pair it decides from the selection tensor whether the pair is allowed, builds
the full ``[Sq, Skv]`` boolean matrix per (sequence, q-head), and evaluates
dense fp64 softmax attention over it.  It is written independently of
``oracle/`` so that a mistake in one is caught by the other.
"""
from __future__ import annotations

import math

import numpy as np


def _lens(case):
    sq = np.diff(case.cu_q).tolist()
    if case.paged:
        skv = [int(x) for x in case.seqused_kv]
    else:
        skv = np.diff(case.cu_kv).tolist()
    return [int(x) for x in sq], [int(x) for x in skv]


def token_allowed(case, b, h):
    """Boolean ``[Sq_b, Skv_b]``: may query ``i`` attend to key ``j``."""
    sq, skv = _lens(case)
    Sq, Skv = sq[b], skv[b]
    G = case.N1 // case.N2
    hs = h if case.sparse_heads == case.N1 else h // G
    bx, by = case.bx, case.by
    gq0 = sum(-(-sq[x] // bx) for x in range(b))
    A = np.zeros((Sq, Skv), dtype=bool)
    for i in range(Sq):
        qb = i // bx
        chosen = set()
        if case.sparse_kind == "none":
            chosen = set(range(-(-Skv // by)))
        elif case.sparse_kind == "mask":
            m = case.sparse
            if qb < m.shape[2]:
                for kb in range(m.shape[3]):
                    if m[b, hs, qb, kb]:
                        chosen.add(kb)
        elif case.sparse_kind == "sabi":
            s = case.sparse
            if qb < s.shape[2]:
                for t in range(s.shape[3]):
                    val = int(s[b, hs, qb, t])
                    if val != 0xFFFF:
                        chosen.add(val)
        elif case.sparse_kind == "idx":
            idx, cnt = case.sparse, case.count
            gq = gq0 + qb
            if gq < idx.shape[1]:
                n = int(cnt[hs, gq])
                n = 0 if n < 0 else min(n, idx.shape[2])
                for t in range(n):
                    val = int(idx[hs, gq, t])
                    if val >= 0:
                        chosen.add(val)
        elif case.sparse_kind == "idx_b":
            idx, cnt = case.sparse, case.count
            if qb < idx.shape[2]:
                n = int(cnt[b, hs, qb])
                n = 0 if n < 0 else min(n, idx.shape[3])
                for t in range(n):
                    val = int(idx[b, hs, qb, t])
                    if val >= 0:
                        chosen.add(val)
        elif case.sparse_kind in ("kvidx", "kvidx_b"):
            # key block kb is chosen for this query's block when kb's own
            # list of query blocks contains it
            idx, cnt = case.sparse, case.count
            gk0 = sum(-(-skv[x] // by) for x in range(b))
            for kb in range(-(-Skv // by)):
                if case.sparse_kind == "kvidx":
                    if gk0 + kb >= idx.shape[1]:
                        continue
                    n = int(cnt[hs, gk0 + kb])
                    lst = idx[hs, gk0 + kb]
                else:
                    if kb >= idx.shape[2]:
                        continue
                    n = int(cnt[b, hs, kb])
                    lst = idx[b, hs, kb]
                n = 0 if n < 0 else min(n, len(lst))
                if qb in [int(x) for x in lst[:n]]:
                    chosen.add(kb)
        for j in range(Skv):
            if (j // by) not in chosen:
                continue
            band = getattr(case, "band", None)
            if band is not None:
                # the window of query i: preTokens earlier and nextTokens later
                # tokens around its bottom-right aligned diagonal key i + Skv - Sq
                if j < i + (Skv - Sq) - band[0] or j > i + (Skv - Sq) + band[1]:
                    continue
            elif case.causal and j > i + (Skv - Sq):
                continue
            A[i, j] = True
    return A


def _keys(case, arr, b, g):
    sq, skv = _lens(case)
    out = np.zeros((skv[b], arr.shape[-1]))
    for j in range(skv[b]):
        if case.paged:
            page = int(case.block_table[b, j // case.page_size])
            out[j] = arr[page, j % case.page_size, g]
        else:
            out[j] = arr[int(case.cu_kv[b]) + j, g]
    return out


def sigma(case):
    s = case.scale if case.scale != 0.0 else 1.0 / math.sqrt(case.D)
    return float(np.float32(s))


def dense_forward(case):
    """O ``[T, N1, D]`` and lse ``[T, N1]`` by dense masked softmax."""
    sq, skv = _lens(case)
    G = case.N1 // case.N2
    T = int(case.cu_q[-1])
    O = np.zeros((T, case.N1, case.D))
    L = np.full((T, case.N1), np.inf)
    sg = sigma(case)
    for b in range(case.B):
        t0 = int(case.cu_q[b])
        for h in range(case.N1):
            A = token_allowed(case, b, h)
            q = case.q[t0:t0 + sq[b], h].astype(np.float64)
            k = _keys(case, case.k, b, h // G)
            v = _keys(case, case.v, b, h // G)
            for i in range(sq[b]):
                js = np.nonzero(A[i])[0]
                if len(js) == 0:
                    continue
                s = sg * (k[js] @ q[i])
                mx = s.max()
                w = np.exp(s - mx)
                O[t0 + i, h] = (w[:, None] * v[js]).sum(0) / w.sum()
                L[t0 + i, h] = mx + math.log(w.sum())
    return O, L


def visited_pairs(case):
    """Set of (hs, b, qb, kb) with at least one allowed token pair."""
    sq, skv = _lens(case)
    G = case.N1 // case.N2
    out = set()
    for b in range(case.B):
        for h in range(case.N1):
            hs = h if case.sparse_heads == case.N1 else h // G
            A = token_allowed(case, b, h)
            ii, jj = np.nonzero(A)
            for i, j in zip(ii, jj):
                out.add((hs, b, int(i) // case.bx, int(j) // case.by))
    return out
