"""Pins for the CPU oracle (no GPU needed).

Each test checks the oracle against something other than itself: values the
pages print for a worked example, closed forms, invariants of the attention
algebra, a brute-force per-token evaluation (tests/brute.py), and library
routines (torch SDPA / autograd in float64 on the CPU).
"""
import copy
import json
import math
import os

import numpy as np
import pytest
import torch

import brute
import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- fixtures --

def tiny_cases():
    """Small varlen cases spanning every selection format, GQA, paging, causal
    masks with Sq != Skv, ragged tails, zero-length sequences, messy index
    lists (duplicates, unsorted, out of range, bad counts)."""
    out = []
    out.append(synth.random_case(11, lens_q=[37, 0, 50], lens_kv=[37, 5, 50], N1=2, D=8, bx=16, by=16,
                                 kind="mask", density=0.5, dtype="f16"))
    out.append(synth.random_case(12, lens_q=[40, 23], N1=4, N2=2, D=8, bx=16, by=8, kind="mask",
                                 sparse_heads=2, causal=True, density=0.6))
    out.append(synth.random_case(13, lens_q=[33, 17], lens_kv=[49, 9], N1=2, D=8, bx=8, by=16, kind="sabi",
                                 causal=True, messy=True))
    out.append(synth.random_case(14, lens_q=[30, 45], lens_kv=[20, 64], N1=4, N2=1, D=8, bx=16, by=16,
                                 kind="idx", sparse_heads=1, messy=True, width=6))
    out.append(synth.random_case(15, lens_q=[50, 31], lens_kv=[40, 70], N1=2, N2=2, D=8, bx=16, by=16,
                                 kind="idx", causal=True, paged=True, page_size=16))
    out.append(synth.random_case(16, lens_q=[29, 41], N1=2, D=8, bx=16, by=32, kind="none", causal=True))
    out.append(synth.random_case(17, lens_q=[21], lens_kv=[35], N1=3, N2=3, D=8, bx=8, by=8, kind="none"))
    out.append(synth.random_case(18, lens_q=[26, 19], N1=4, N2=2, D=8, bx=16, by=16, kind="sabi",
                                 sparse_heads=4, paged=True, page_size=16, causal=False))
    # band masks (preTokens, nextTokens): a window around the diagonal with
    # Sq != Skv, a one-key window, windows that exclude the diagonal (negative
    # preTokens / nextTokens), paged GQA
    out.append(synth.random_case(19, lens_q=[45, 30], lens_kv=[60, 22], N1=2, D=8, bx=16, by=16, kind="mask",
                                 density=0.7, band=(20, 5)))
    out.append(synth.random_case(20, lens_q=[33, 21], N1=4, N2=2, D=8, bx=8, by=16, kind="sabi", sparse_heads=2,
                                 band=(0, 0), dense_q=True))
    out.append(synth.random_case(21, lens_q=[40, 27], lens_kv=[52, 30], N1=2, N2=1, D=8, bx=16, by=8, kind="idx",
                                 sparse_heads=1, paged=True, page_size=16, band=(-3, 12), messy=True))
    out.append(synth.random_case(22, lens_q=[50], lens_kv=[31], N1=2, D=8, bx=16, by=16, kind="none",
                                 band=(40, -2)))
    # the other layoutSparsePattern forms: per-Q-block lists with a batch axis,
    # per-KV-block lists over global KV blocks and with a batch axis (messy
    # entries, counts out of range, fewer list rows than KV blocks)
    out.append(synth.random_case(23, lens_q=[37, 20, 44], lens_kv=[50, 9, 30], N1=4, N2=2, D=8, bx=16, by=8,
                                 kind="idx_b", sparse_heads=2, messy=True, causal=True))
    out.append(synth.random_case(24, lens_q=[45, 0, 33], lens_kv=[40, 12, 52], N1=4, N2=2, D=8, bx=8, by=16,
                                 kind="kvidx", sparse_heads=4, messy=True, paged=True, page_size=16))
    out.append(synth.random_case(25, lens_q=[60, 28], lens_kv=[64, 70], N1=2, D=8, bx=16, by=8, kind="kvidx_b",
                                 messy=True, causal=True, rows=6))
    out.append(synth.random_case(26, lens_q=[41, 30], N1=2, N2=1, D=8, bx=16, by=16, kind="kvidx",
                                 sparse_heads=1, band=(12, 3)))
    return out


CASES = tiny_cases()


def _f64(case):
    """Copy of ``case`` with float64 Q/K/V/dO, for derivative checks."""
    c = copy.copy(case)
    for name in ("q", "k", "v", "dout"):
        setattr(c, name, getattr(case, name).astype(np.float64))
    return c


# ------------------------------------------------------------ worked example --

def test_allones_worked_example_lse_and_output():
    fx = _load("blitz_allones_example.json")
    S, N, D = fx["S"], fx["N"], fx["D"]
    case = synth.ones_case(S=S, N=N, D=D, dtype=fx["dtype"], bx=fx["block_shape"][0], by=fx["block_shape"][1])
    assert list(case.sparse.shape) == fx["sabi_shape"]
    O, lse = oracle.forward(case)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-12)
    # The stated closed form ln S + sqrt(D), to the 4 decimals printed.
    assert abs(lse[0, 0] - fx["expected_lse_stated"]) <= 0.5 * 10 ** -fx["expected_lse_stated_decimals"] + 1e-5
    assert np.allclose(lse, math.log(S) + D * oracle.scale_of(0.0, D), rtol=0, atol=1e-9)
    # The printed Ascend value, reproduced with the fp16-rounded scale.
    fp16_scale = float(np.float16(1.0 / math.sqrt(D)))
    case16 = synth.ones_case(S=S, N=N, D=D, dtype=fx["dtype"], scale=fp16_scale)
    _, lse16 = oracle.forward(case16)
    assert abs(lse16[0, 0] - fx["printed_lse0"]) <= 0.5 * 10 ** -fx["printed_lse0_decimals"]
    # output[0] = 0x3C00 is fp16 1.0
    assert np.float16(O[0, 0, 0]).view(np.uint16) == int(fx["printed_output0_bits"], 16)


def test_sabi_example_shape_and_counts():
    fx = _load("blitz_sabi_example.json")
    S = fx["sequence_length"]
    bx, by = fx["block_shape"]
    assert -(-S // bx) == fx["num_rows"] and -(-S // by) == fx["num_cols"]
    case = synth.ones_case(S=S, N=2, D=8, dtype="bf16", bx=bx, by=by)
    sabi = np.full((1, 2, fx["num_rows"], fx["num_cols"]), 0xFFFF, dtype=np.uint16)
    for r in fx["head0_rows_shown"]:
        sabi[0, 0, r["row"]] = r["entries"]
    case.sparse = sabi
    idx = oracle.index_products(case, with_csc=False)
    for r in fx["head0_rows_shown"]:
        assert idx["counts"][r["row"]] == r["computes"]


# ---------------------------------------------------- forward vs brute force --

@pytest.mark.parametrize("ci", range(len(CASES)))
def test_forward_matches_brute_force(ci):
    case = CASES[ci]
    O, lse = oracle.forward(case)
    Ob, lb = brute.dense_forward(case)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_index_products_match_brute_force(ci):
    case = CASES[ci]
    idx = oracle.index_products(case)
    pairs = brute.visited_pairs(case)
    sq, skv = brute._lens(case)
    nqb = [-(-s // case.bx) for s in sq]
    nkb = [-(-s // case.by) for s in skv]
    qbase = np.concatenate([[0], np.cumsum(nqb)]).astype(int)
    kbase = np.concatenate([[0], np.cumsum(nkb)]).astype(int)
    TQB, TKB = int(qbase[-1]), int(kbase[-1])
    got = set()
    rp, cols = idx["row_ptr"], idx["cols"]
    for hs in range(case.sparse_heads):
        for b in range(case.B):
            for qb in range(nqb[b]):
                r = hs * TQB + qbase[b] + qb
                lst = cols[rp[r]:rp[r + 1]].tolist()
                assert lst == sorted(set(lst))
                got |= {(hs, b, qb, kb) for kb in lst}
    assert got == pairs
    # transpose relation and invariants
    cp, qr = idx["col_ptr"], idx["qrows"]
    assert rp[-1] == cp[-1]
    got_t = set()
    for hs in range(case.sparse_heads):
        for b in range(case.B):
            for kb in range(nkb[b]):
                c = hs * TKB + kbase[b] + kb
                lst = qr[cp[c]:cp[c + 1]].tolist()
                assert lst == sorted(set(lst))
                got_t |= {(hs, b, qb, kb) for qb in lst}
    assert got_t == pairs
    # work lists: permutations, non-increasing keys, ties by id
    w = idx["work"]
    cnt = np.diff(rp)
    assert sorted(w.tolist()) == list(range(len(cnt)))
    for a, b_ in zip(w[:-1], w[1:]):
        assert cnt[a] > cnt[b_] or (cnt[a] == cnt[b_] and a < b_)
    wk = idx["work_kv"]
    key = idx["kv_key"]
    assert sorted(wk.tolist()) == list(range(case.N2 * TKB))
    for a, b_ in zip(wk[:-1], wk[1:]):
        assert key[a] > key[b_] or (key[a] == key[b_] and a < b_)
    # kv keys = number of (q-head pattern, q-block) pairs reaching each item
    G = case.N1 // case.N2
    for g in range(case.N2):
        for b in range(case.B):
            for kb in range(nkb[b]):
                heads = [g] if case.sparse_heads == case.N2 else range(g * G, (g + 1) * G)
                n = sum(1 for (hs, bb, qb, k2) in pairs if hs in heads and bb == b and k2 == kb)
                assert key[g * TKB + kbase[b] + kb] == n


def test_work_list_hand_example():
    """Three rows with visited counts 1, 3, 1 and one empty row: work order
    must be [1, 0, 2, 3] (descending count, ties by row id)."""
    case = synth.random_case(3, lens_q=[64], N1=1, D=8, bx=16, by=16, kind="mask")
    m = np.zeros((1, 1, 4, 4), dtype=np.uint8)
    m[0, 0, 0, 0] = 1
    m[0, 0, 1, [0, 2, 3]] = 1
    m[0, 0, 2, 1] = 1
    case.sparse = m
    idx = oracle.index_products(case)
    assert idx["row_ptr"].tolist() == [0, 1, 4, 5, 5]
    assert idx["cols"].tolist() == [0, 0, 2, 3, 1]
    assert idx["work"].tolist() == [1, 0, 2, 3]
    assert idx["col_ptr"].tolist() == [0, 2, 3, 4, 5]
    assert idx["qrows"].tolist() == [0, 1, 2, 1, 1]
    assert idx["work_kv"].tolist() == [0, 1, 2, 3]


def _kv_lists_from_mask(mask_case, kind):
    """The mask case's selection rewritten as per-KV-block lists: KV block kb
    of sequence b lists every q-block whose mask row selects it (the
    layoutSparsePattern table's "each KV block lists the Q blocks that chose
    it"), in ascending order, padded with -1."""
    c = copy.copy(mask_case)
    sq, skv = oracle.lengths(mask_case)
    nqb = [-(-s // mask_case.bx) for s in sq]
    nkb = [-(-s // mask_case.by) for s in skv]
    Hs, W = mask_case.sparse_heads, max(nqb)
    lists = {}
    for b in range(mask_case.B):
        for hs in range(Hs):
            for kb in range(nkb[b]):
                lists[b, hs, kb] = [qb for qb in range(nqb[b])
                                    if kb < mask_case.sparse.shape[3] and mask_case.sparse[b, hs, qb, kb]]
    if kind == "kvidx":
        idx = np.full((Hs, sum(nkb), W), -1, dtype=np.int32)
        cnt = np.zeros((Hs, sum(nkb)), dtype=np.int32)
        for (b, hs, kb), lst in lists.items():
            idx[hs, sum(nkb[:b]) + kb, :len(lst)] = lst
            cnt[hs, sum(nkb[:b]) + kb] = len(lst)
    else:
        idx = np.full((mask_case.B, Hs, max(nkb), W), -1, dtype=np.int32)
        cnt = np.zeros((mask_case.B, Hs, max(nkb)), dtype=np.int32)
        for (b, hs, kb), lst in lists.items():
            idx[b, hs, kb, :len(lst)] = lst
            cnt[b, hs, kb] = len(lst)
    c.sparse_kind, c.sparse, c.count = kind, idx, cnt
    return c, lists


@pytest.mark.parametrize("kind", ["kvidx", "kvidx_b"])
def test_kv_lists_equal_their_per_q_block_transpose(kind):
    """Per-KV-block lists made from a block mask select exactly what the mask
    selects: identical index products and outputs; and without a token mask
    the transposed lists the index builds (col_ptr / qrows) are the input
    lists themselves."""
    m = synth.random_case(35, lens_q=[70, 33, 50], lens_kv=[60, 40, 81], N1=4, N2=2, D=8, bx=16, by=16,
                          kind="mask", sparse_heads=4, density=0.5)
    c, lists = _kv_lists_from_mask(m, kind)
    im, ic = oracle.index_products(m), oracle.index_products(c)
    for k in ("row_ptr", "cols", "work", "col_ptr", "qrows", "work_kv"):
        assert np.array_equal(im[k], ic[k]), k
    (Om, lm), (Oc, lc) = oracle.forward(m), oracle.forward(c)
    assert np.array_equal(Om, Oc) and np.array_equal(lm, lc)
    sq, skv = oracle.lengths(m)
    nkb = [-(-s // 16) for s in skv]
    TKB = sum(nkb)
    for (b, hs, kb), lst in lists.items():
        col = hs * TKB + sum(nkb[:b]) + kb
        assert list(ic["qrows"][ic["col_ptr"][col]:ic["col_ptr"][col + 1]]) == lst


def test_batch_major_idx_equals_global_idx():
    """The same per-Q-block lists laid out [B, Hs, maxQBlocks, W]
    (layoutSparsePattern 0 / 2) and [Hs, totalQBlocks, W] (4 / 6) select the
    same blocks."""
    g = synth.random_case(36, lens_q=[70, 33, 50], lens_kv=[60, 40, 81], N1=4, N2=2, D=8, bx=16, by=16,
                          kind="idx", sparse_heads=2, messy=True)
    sq, _ = oracle.lengths(g)
    nqb = [-(-s // 16) for s in sq]
    Hs, W = g.sparse.shape[0], g.sparse.shape[2]
    idx = np.full((g.B, Hs, max(nqb), W), -1, dtype=np.int32)
    cnt = np.zeros((g.B, Hs, max(nqb)), dtype=np.int32)
    for b in range(g.B):
        for q in range(nqb[b]):
            idx[b, :, q] = g.sparse[:, sum(nqb[:b]) + q]
            cnt[b, :, q] = g.count[:, sum(nqb[:b]) + q]
    c = copy.copy(g)
    c.sparse_kind, c.sparse, c.count = "idx_b", idx, cnt
    ig, ic = oracle.index_products(g), oracle.index_products(c)
    for k in ("row_ptr", "cols", "work", "col_ptr", "qrows", "work_kv"):
        assert np.array_equal(ig[k], ic[k]), k
    (Og, lg), (Oc, lc) = oracle.forward(g), oracle.forward(c)
    assert np.array_equal(Og, Oc) and np.array_equal(lg, lc)


def test_band_extremes_equal_causal_and_no_mask():
    """A band with preTokens beyond every sequence and nextTokens = 0 is the
    bottom-right causal mask; with both beyond every sequence it is no mask:
    the same index products and the same outputs."""
    kw = dict(lens_q=[37, 20, 44], lens_kv=[50, 20, 30], N1=2, D=8, bx=16, by=16, kind="mask", density=0.6)
    causal = synth.random_case(31, causal=True, **kw)
    band_c = synth.random_case(31, band=(10 ** 6, 0), **kw)
    plain = synth.random_case(31, **kw)
    band_n = synth.random_case(31, band=(10 ** 6, 10 ** 6), **kw)
    for a, b in ((causal, band_c), (plain, band_n)):
        ia, ib = oracle.index_products(a), oracle.index_products(b)
        for k in ("row_ptr", "cols", "work", "col_ptr", "qrows", "work_kv"):
            assert np.array_equal(ia[k], ib[k]), k
        (Oa, la), (Ob, lb) = oracle.forward(a), oracle.forward(b)
        assert np.array_equal(Oa, Ob) and np.array_equal(la, lb)


def test_band_single_key_window_closed_form():
    """preTokens = nextTokens = 0 leaves each query exactly one key, the
    diagonal key j = i + Skv - Sq (when it exists and its block is selected):
    O_i = v_j and lse_i = scale q_i . k_j; the other rows are empty."""
    case = synth.random_case(32, lens_q=[30, 41], lens_kv=[45, 33], N1=2, D=8, bx=16, by=16, kind="mask",
                             density=0.6, band=(0, 0))
    O, lse = oracle.forward(case)
    sg = oracle.scale_of(case.scale, case.D)
    sq, skv = oracle.lengths(case)
    for b in range(case.B):
        for h in range(case.N1):
            for i in range(sq[b]):
                t = int(case.cu_q[b]) + i
                j = i + skv[b] - sq[b]
                sel = 0 <= j < skv[b] and case.sparse[b, h, i // 16, j // 16] != 0
                if not sel:
                    assert np.isinf(lse[t, h]) and np.all(O[t, h] == 0)
                    continue
                kj = case.k[int(case.cu_kv[b]) + j, h].astype(np.float64)
                vj = case.v[int(case.cu_kv[b]) + j, h].astype(np.float64)
                np.testing.assert_allclose(O[t, h], vj, rtol=0, atol=1e-12)
                assert abs(lse[t, h] - sg * float(case.q[t, h].astype(np.float64) @ kj)) < 1e-12


def test_band_empty_window():
    """preTokens + nextTokens < 0: no query has a key -- every row is empty
    (O = 0, lse = +inf), the index has no visited block, and the gradients
    vanish."""
    case = synth.random_case(33, lens_q=[40, 25], N1=2, D=8, bx=16, by=16, kind="none", band=(5, -7))
    O, lse = oracle.forward(case)
    assert np.all(O == 0) and np.all(np.isinf(lse))
    idx = oracle.index_products(case)
    assert idx["row_ptr"][-1] == 0 and len(idx["cols"]) == 0
    dq, dk, dv = oracle.backward(case)
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dv == 0)


def test_band_dense_matches_torch_sdpa_window_mask():
    """No block selection, Sq = Skv, band (pre, next): torch's SDPA in float64
    with the boolean window mask j - pre <= ... written as a matrix."""
    pre, nxt = 9, 4
    case = synth.random_case(34, lens_q=[57, 33], N1=2, D=16, bx=16, by=16, kind="none", band=(pre, nxt))
    O, lse = oracle.forward(case)
    sg = oracle.scale_of(case.scale, case.D)
    for b in range(case.B):
        t0, t1 = int(case.cu_q[b]), int(case.cu_q[b + 1])
        S = t1 - t0
        i = np.arange(S)[:, None]
        j = np.arange(S)[None, :]
        m = torch.from_numpy((j >= i - pre) & (j <= i + nxt))
        for h in range(case.N1):
            q = torch.from_numpy(case.q[t0:t1, h].astype(np.float64))[None]
            k = torch.from_numpy(case.k[t0:t1, h].astype(np.float64))[None]
            v = torch.from_numpy(case.v[t0:t1, h].astype(np.float64))[None]
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m[None], scale=sg)[0]
            np.testing.assert_allclose(O[t0:t1, h], ref.numpy(), rtol=0, atol=1e-12)


def test_causal_bottom_right_visited_blocks():
    """Sq=16, Skv=48, by=16 causal: query i sees keys j <= i + 32, so q-block 0
    (rows 0..15) reaches blocks 0, 1, 2; with Sq=48, Skv=16 rows 0..31 see
    nothing and the first two q-blocks are empty."""
    c1 = synth.random_case(4, lens_q=[16], lens_kv=[48], N1=1, D=8, bx=16, by=16, kind="none", causal=True)
    assert oracle.index_products(c1)["cols"].tolist() == [0, 1, 2]
    c2 = synth.random_case(5, lens_q=[48], lens_kv=[16], N1=1, D=8, bx=16, by=16, kind="none", causal=True)
    idx = oracle.index_products(c2)
    assert idx["row_ptr"].tolist() == [0, 0, 0, 1]
    O, lse = oracle.forward(c2)
    assert np.all(np.isinf(lse[:32])) and np.all(O[:32] == 0)
    assert np.all(np.isfinite(lse[32:]))


# --------------------------------------------------------- library routines --

@pytest.mark.parametrize("causal", [False, True])
def test_dense_forward_matches_torch_sdpa(causal):
    case = synth.random_case(21, lens_q=[45, 30], lens_kv=[45, 30], N1=2, N2=2, D=16, bx=16, by=16,
                             kind="none", causal=causal)
    O, lse = oracle.forward(case)
    sg = oracle.scale_of(case.scale, case.D)
    for b in range(case.B):
        t0, t1 = int(case.cu_q[b]), int(case.cu_q[b + 1])
        q = torch.from_numpy(case.q[t0:t1].astype(np.float64)).permute(1, 0, 2)
        k = torch.from_numpy(case.k[t0:t1].astype(np.float64)).permute(1, 0, 2)
        v = torch.from_numpy(case.v[t0:t1].astype(np.float64)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=sg)
        np.testing.assert_allclose(O[t0:t1], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def _torch_dense_grads(case):
    """dq, dk, dv from torch autograd (float64, CPU) of dense attention masked
    with the brute-force allowed matrix."""
    sq, skv = brute._lens(case)
    G = case.N1 // case.N2
    sg = oracle.scale_of(case.scale, case.D)
    dq = np.zeros(case.q.shape)
    dk = np.zeros(case.k.shape)
    dv = np.zeros(case.v.shape)
    for b in range(case.B):
        t0 = int(case.cu_q[b])
        for h in range(case.N1):
            g = h // G
            A = torch.from_numpy(brute.token_allowed(case, b, h))
            q = torch.from_numpy(case.q[t0:t0 + sq[b], h].astype(np.float64)).requires_grad_()
            kk = torch.from_numpy(brute._keys(case, case.k, b, g)).requires_grad_()
            vv = torch.from_numpy(brute._keys(case, case.v, b, g)).requires_grad_()
            do = torch.from_numpy(case.dout[t0:t0 + sq[b], h].astype(np.float64))
            s = (sg * q @ kk.T).masked_fill(~A, -math.inf)
            has = A.any(dim=1, keepdim=True)
            p = torch.softmax(torch.where(has, s, torch.zeros_like(s)), dim=1) * A * has
            o = p @ vv
            (o * do).sum().backward()
            dq[t0:t0 + sq[b], h] = q.grad.numpy()
            for j in range(skv[b]):
                if case.paged:
                    page = int(case.block_table[b, j // case.page_size])
                    dk[page, j % case.page_size, g] += kk.grad[j].numpy()
                    dv[page, j % case.page_size, g] += vv.grad[j].numpy()
                else:
                    dk[int(case.cu_kv[b]) + j, g] += kk.grad[j].numpy()
                    dv[int(case.cu_kv[b]) + j, g] += vv.grad[j].numpy()
    return dq, dk, dv


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_backward_matches_torch_autograd(ci):
    case = CASES[ci]
    dq, dk, dv = oracle.backward(case)
    rq, rk, rv = _torch_dense_grads(case)
    np.testing.assert_allclose(dq, rq, rtol=0, atol=1e-11)
    fin = ~np.isnan(case.k)  # paged tails hold NaN; their gradients stay 0
    np.testing.assert_allclose(np.where(fin, dk, 0), np.where(fin, rk, 0), rtol=0, atol=1e-11)
    np.testing.assert_allclose(np.where(fin, dv, 0), np.where(fin, rv, 0), rtol=0, atol=1e-11)


# ------------------------------------------------------- finite differences --

def test_backward_finite_differences():
    case = _f64(synth.random_case(31, lens_q=[19, 12], lens_kv=[23, 12], N1=2, N2=1, D=4, bx=8, by=8,
                                  kind="mask", sparse_heads=2, causal=True, density=0.7))
    dq, dk, dv = oracle.backward(case)
    rng = np.random.default_rng(0)
    h = 1e-6

    def loss():
        O, _ = oracle.forward(case)
        return float((O * case.dout).sum())

    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        arr = getattr(case, name)
        for _ in range(12):
            ix = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[ix]
            arr[ix] = old + h
            lp = loss()
            arr[ix] = old - h
            lm = loss()
            arr[ix] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[ix]) <= 1e-6 * max(1.0, abs(fd)), (name, ix, fd, grad[ix])


# -------------------------------------------------------------- closed forms --

def test_backward_allones_closed_form():
    """All-ones inputs: dP = D = rowsum(dO o O), so dS = 0, dq = dk = 0, and
    dv_j = sum over (h in group, i with j allowed) of 1/|A_i|."""
    case = synth.random_case(41, lens_q=[40, 24], N1=4, N2=2, D=8, bx=16, by=8, kind="mask",
                             sparse_heads=2, causal=True, density=0.6)
    for name in ("q", "k", "v", "dout"):
        setattr(case, name, np.ones_like(getattr(case, name)))
    dq, dk, dv = oracle.backward(case)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    G = case.N1 // case.N2
    expect = np.zeros(case.v.shape[:2])
    for b in range(case.B):
        for h in range(case.N1):
            A = brute.token_allowed(case, b, h)
            n = A.sum(axis=1)
            for i in range(A.shape[0]):
                if n[i]:
                    for j in np.nonzero(A[i])[0]:
                        expect[int(case.cu_kv[b]) + j, h // G] += 1.0 / n[i]
    np.testing.assert_allclose(dv, np.repeat(expect[:, :, None], case.D, axis=2), rtol=0, atol=1e-12)


def test_backward_invariants():
    """sum_j dS_ij = 0 per row, hence (a) the key-gradient summed over each
    sequence's keys vanishes and (b) dq = 0 when every key row of a head is
    the same vector."""
    case = _f64(synth.random_case(42, lens_q=[37, 22], lens_kv=[41, 30], N1=2, N2=2, D=8, bx=16, by=16,
                                  kind="sabi", causal=True))
    dq, dk, dv = oracle.backward(case)
    for b in range(case.B):
        k0, k1 = int(case.cu_kv[b]), int(case.cu_kv[b + 1])
        s = dk[k0:k1].sum(axis=0)
        assert np.abs(s).max() <= 1e-12 * max(1.0, np.abs(dk[k0:k1]).max())
    case.k[:] = case.k[0:1]
    dq2, _, _ = oracle.backward(case)
    assert np.abs(dq2).max() <= 1e-12


def test_empty_rows_and_unreached_keys():
    case = synth.random_case(43, lens_q=[48], N1=1, D=8, bx=16, by=16, kind="mask")
    m = np.zeros((1, 1, 3, 3), dtype=np.uint8)
    m[0, 0, 0, 0] = 1
    m[0, 0, 2, 0] = 1  # row 1 selects nothing; key block 1 and 2 unreached
    case.sparse = m
    O, lse = oracle.forward(case)
    assert np.all(O[16:32] == 0) and np.all(np.isinf(lse[16:32])) and np.all(lse[16:32] > 0)
    dq, dk, dv = oracle.backward(case)
    assert np.all(dq[16:32] == 0)
    assert np.all(dk[16:] == 0) and np.all(dv[16:] == 0)



@pytest.mark.parametrize("paged", [False, True])
def test_sampled_backward_equals_full_and_marks_the_rest(paged):
    """Sampling q-blocks / KV blocks gives the full backward's values on the
    sampled entries and NaN on every entry it did not compute."""
    case = synth.random_case(44, lens_q=[70, 33], lens_kv=[90, 41], N1=4, N2=2, D=8, bx=16, by=32,
                             kind="mask", sparse_heads=4, causal=True, paged=paged, page_size=16)
    fq, fk, fv = oracle.backward(case)
    rows = [(0, 1, 2), (1, 3, 0)]
    kvs = [(0, 1, 1), (1, 0, 0)]
    dq, dk, dv = oracle.backward(case, sample_rows=rows, sample_kv=kvs)
    want_q = np.zeros(dq.shape[:2], dtype=bool)
    for (b, h, qb) in rows:
        lo = int(case.cu_q[b]) + qb * case.bx
        want_q[lo:min(lo + case.bx, int(case.cu_q[b + 1])), h] = True
    assert np.array_equal(~np.isnan(dq[..., 0]), want_q)
    np.testing.assert_array_equal(dq[want_q], fq[want_q])
    skv = case.seqused_kv if case.paged else np.diff(case.cu_kv)
    want_k = np.zeros(dk.shape[:-1], dtype=bool)
    for (b, g, kb) in kvs:
        for j in range(kb * case.by, min(int(skv[b]), (kb + 1) * case.by)):
            if case.paged:
                want_k[int(case.block_table[b, j // case.page_size]), j % case.page_size, g] = True
            else:
                want_k[int(case.cu_kv[b]) + j, g] = True
    for got, full in ((dk, fk), (dv, fv)):
        assert np.array_equal(~np.isnan(got[..., 0]), want_k)
        np.testing.assert_array_equal(got[want_k], full[want_k])


# ---------------------------------------------------------------- invariants --

def test_rows_sum_to_one_via_unit_values():
    """With V = 1 every non-empty row's output is sum_j P_ij = 1."""
    for case in CASES:
        c = copy.copy(case)
        c.v = np.ones_like(case.v)
        O, lse = oracle.forward(c)
        ne = np.isfinite(lse)
        np.testing.assert_allclose(O[ne], 1.0, rtol=0, atol=1e-12)


def test_gqa_equals_repeated_mha():
    case = synth.random_case(51, lens_q=[40, 27], N1=4, N2=2, D=8, bx=16, by=16, kind="mask",
                             sparse_heads=2, causal=True, density=0.6)
    G = 2
    mha = copy.copy(case)
    mha.N2 = 4
    mha.sparse_heads = 4
    mha.k = np.repeat(case.k, G, axis=1)
    mha.v = np.repeat(case.v, G, axis=1)
    mha.sparse = np.repeat(case.sparse, G, axis=1)
    O1, l1 = oracle.forward(case)
    O2, l2 = oracle.forward(mha)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)
    dq1, dk1, dv1 = oracle.backward(case)
    dq2, dk2, dv2 = oracle.backward(mha)
    np.testing.assert_allclose(dq1, dq2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk1, dk2.reshape(dk2.shape[0], 2, G, -1).sum(2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv1, dv2.reshape(dv2.shape[0], 2, G, -1).sum(2), rtol=0, atol=1e-12)


def test_paged_equals_packed():
    case = CASES[4]
    assert case.paged
    packed = copy.copy(case)
    packed.paged = False
    lens = [int(x) for x in case.seqused_kv]
    packed.cu_kv = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ks, vs = [], []
    for b, L in enumerate(lens):
        for j in range(L):
            page = int(case.block_table[b, j // case.page_size])
            ks.append(case.k[page, j % case.page_size])
            vs.append(case.v[page, j % case.page_size])
    packed.k = np.stack(ks)
    packed.v = np.stack(vs)
    O1, l1 = oracle.forward(case)
    O2, l2 = oracle.forward(packed)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)


def test_varlen_equals_per_sequence():
    case = CASES[1]
    O, lse = oracle.forward(case)
    for b in range(case.B):
        one = copy.copy(case)
        one.B = 1
        t0, t1 = int(case.cu_q[b]), int(case.cu_q[b + 1])
        k0, k1 = int(case.cu_kv[b]), int(case.cu_kv[b + 1])
        one.cu_q = np.array([0, t1 - t0], dtype=np.int64)
        one.cu_kv = np.array([0, k1 - k0], dtype=np.int64)
        one.q, one.k, one.v = case.q[t0:t1], case.k[k0:k1], case.v[k0:k1]
        one.sparse = case.sparse[b:b + 1]
        O1, l1 = oracle.forward(one)
        assert np.array_equal(O1, O[t0:t1]) and np.array_equal(l1, lse[t0:t1])


# ------------------------------------------------- tiles of narrow q-blocks --

TILE_CASES = [
    dict(seed=71, lens_q=[300, 45], N1=4, N2=2, bx=1, by=16, kind="idx", width=6, causal=True),
    dict(seed=72, lens_q=[150, 97], lens_kv=[260, 97], N1=2, N2=2, bx=4, by=32, kind="mask", causal=True),
    dict(seed=73, lens_q=[140], N1=2, N2=1, bx=16, by=16, kind="sabi", width=5),
    dict(seed=74, lens_q=[64, 200], N1=2, N2=2, bx=32, by=16, kind="kvidx", width=9, band=(40, 3)),
    dict(seed=75, lens_q=[129, 33], N1=2, N2=2, bx=8, by=16, kind="none", causal=True),
    dict(seed=76, lens_q=[180, 70], N1=4, N2=2, bx=2, by=16, kind="idx_b", width=5, sparse_heads=4),
]


def _tile_case(kw):
    kw = dict(kw)
    return synth.random_case(kw.pop("seed"), D=8, with_dout=False, **kw)


@pytest.mark.parametrize("ci", range(len(TILE_CASES)))
def test_tile_index_masks_match_brute_force(ci):
    """Row-tile index: a row's mask bit for a visited block is set exactly
    when its q-block holds an allowed (query, key) pair in that block (brute
    force per token), the union lists are those bits' blocks, and the
    transpose carries the same masks."""
    case = _tile_case(TILE_CASES[ci])
    T = 128
    ti = oracle.tile_index_products(case, T)
    pairs = brute.visited_pairs(case)  # (hs, b, qb, kb)
    sq, skv = brute._lens(case)
    nqb = [-(-s // case.bx) for s in sq]
    nt = [-(-s // T) for s in sq]
    tb = np.concatenate([[0], np.cumsum(nt)]).astype(int)
    TT = int(tb[-1])
    per = T // case.bx
    rp, cols, rm = ti["row_ptr"], ti["cols"], ti["row_mask"]
    seen = set()
    for hs in range(case.sparse_heads):
        for b in range(case.B):
            for t in range(nt[b]):
                r = hs * TT + tb[b] + t
                lst = cols[rp[r]:rp[r + 1]].tolist()
                assert lst == sorted(set(lst))
                for e, kb in zip(range(rp[r], rp[r + 1]), lst):
                    bits = [(int(rm[e, i // 32]) >> (i % 32)) & 1 for i in range(T)]
                    for i in range(T):
                        qb = t * per + i // case.bx
                        want = qb < nqb[b] and (hs, b, qb, kb) in pairs
                        assert bits[i] == want, (hs, b, t, kb, i)
                    assert any(bits)
                    seen |= {(hs, b, t * per + i // case.bx, kb) for i in range(T) if bits[i]}
    assert seen == pairs
    cp, qr, cm = ti["col_ptr"], ti["qrows"], ti["col_mask"]
    assert cp[-1] == rp[-1]
    TKB = ti["TKB"]
    nkb = [-(-s // case.by) for s in skv]
    kbase = np.concatenate([[0], np.cumsum(nkb)]).astype(int)
    for hs in range(case.sparse_heads):
        for b in range(case.B):
            for kb in range(nkb[b]):
                c = hs * TKB + kbase[b] + kb
                ts = qr[cp[c]:cp[c + 1]].tolist()
                assert ts == sorted(set(ts))
                for o, t in zip(range(cp[c], cp[c + 1]), ts):
                    r = hs * TT + tb[b] + t
                    e = rp[r] + cols[rp[r]:rp[r + 1]].tolist().index(kb)
                    assert np.array_equal(cm[o], rm[e])


def test_tile_index_with_whole_tiles_is_the_plain_index():
    """With block_x equal to the tile, each tile is one q-block: the products
    are index_products' and every mask word is all ones."""
    case = _tile_case(dict(seed=77, lens_q=[300, 130], N1=4, N2=2, bx=128, by=32, kind="idx", width=7,
                           causal=True))
    a = oracle.index_products(case)
    t = oracle.tile_index_products(case, 128)
    for k in ("row_ptr", "cols", "work", "col_ptr", "qrows", "work_kv"):
        assert np.array_equal(a[k], t[k]), k
    assert (t["row_mask"] == 0xFFFFFFFF).all() and (t["col_mask"] == 0xFFFFFFFF).all()


def test_index_order_and_duplicates_irrelevant():
    case = synth.random_case(61, lens_q=[40, 33], N1=2, D=8, bx=16, by=8, kind="idx", width=8)
    O, lse = oracle.forward(case)
    shuf = copy.copy(case)
    idx = case.sparse.copy()
    cnt = case.count.copy()
    rng = np.random.default_rng(1)
    for h in range(idx.shape[0]):
        for r in range(idx.shape[1]):
            n = int(cnt[h, r])
            e = idx[h, r, :n].copy()
            rng.shuffle(e)
            if 0 < n < idx.shape[2]:
                e = np.concatenate([e, e[:1]])  # duplicate an entry
                cnt[h, r] = n + 1
            idx[h, r, :len(e)] = e
    shuf.sparse, shuf.count = idx, cnt
    O2, l2 = oracle.forward(shuf)
    assert np.array_equal(O, O2) and np.array_equal(lse, l2)


def test_lse_merge_of_disjoint_block_sets():
    """Splitting each row's selected blocks into X and Y: lse = logaddexp and
    O is the lse-weighted mix (the partial-result merge the LSE output is for,
    BlitzSparseAttention page, softmax_lse output)."""
    case = synth.random_case(71, lens_q=[64, 48], N1=2, D=8, bx=16, by=16, kind="mask", density=0.8,
                             causal=True)
    X, Y = copy.copy(case), copy.copy(case)
    cols = np.arange(case.sparse.shape[3])
    X.sparse = case.sparse * (cols % 2 == 0)
    Y.sparse = case.sparse * (cols % 2 == 1)
    O, lse = oracle.forward(case)
    Ox, lx = oracle.forward(X)
    Oy, ly = oracle.forward(Y)
    # an empty partial set stores lse = +inf; as a log-sum it is log(0) = -inf
    lx = np.where(np.isinf(lx), -np.inf, lx)
    ly = np.where(np.isinf(ly), -np.inf, ly)
    lm = np.logaddexp(lx, ly)
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lm[fin], lse[fin], rtol=0, atol=1e-12)
    with np.errstate(invalid="ignore"):
        wx = np.where(np.isfinite(lx), np.exp(lx - lm), 0.0)
        wy = np.where(np.isfinite(ly), np.exp(ly - lm), 0.0)
    mix = wx[..., None] * Ox + wy[..., None] * Oy
    np.testing.assert_allclose(mix[fin], O[fin], rtol=0, atol=1e-12)


def test_context_parallel_shards_as_band_masks():
    """Causal shards of one sequence (queries [qs, qs + nq) against keys
    [ks, ks + nk)) with the band offsets of tests/cp_shards.py give the whole
    sequence's rows: in full when the shard holds every key its rows reach,
    and through the LSE merge when the keys are split over shards."""
    import cp_shards
    case = synth.random_case(81, lens_q=[150], lens_kv=[190], N1=2, D=8, bx=16, by=16, kind="none", causal=True)
    O, lse = oracle.forward(case)
    for qs, nq, ks, nk in ((0, 70, 0, 190), (70, 80, 0, 190), (30, 60, 0, 150)):
        Os, ls = oracle.forward(cp_shards.shard(case, qs, nq, ks, nk))
        np.testing.assert_allclose(Os, O[qs:qs + nq], rtol=0, atol=1e-12)
        np.testing.assert_allclose(ls, lse[qs:qs + nq], rtol=0, atol=1e-12)
    # rows 80..149 against keys [0, 95) and [95, 190), merged
    parts = [oracle.forward(cp_shards.shard(case, 80, 70, ks, nk)) for ks, nk in ((0, 95), (95, 95))]
    Om, lm = cp_shards.merge(parts)
    np.testing.assert_allclose(Om, O[80:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm, lse[80:], rtol=0, atol=1e-12)
    # a negative nextTokens: the first shard's window ends below its diagonal
    assert cp_shards.next_tokens(case, 0, 70, 0, 190) < 0


def test_config_structures():
    """Structural facts of the benchmark workloads: exact visited-pair count
    of the long-context mask and shapes of the other selection tensors."""
    c5 = synth.config5(values=False)
    assert c5.sparse.shape == (2, 16, 128, 128)
    per_row = c5.sparse.sum(axis=3)
    expect = np.array([min(i + 1, 13) for i in range(128)])
    assert np.array_equal(per_row, np.broadcast_to(expect, per_row.shape))
    assert int(per_row.sum()) == 50752 // 1  # visited (b, h, qb, kb) pairs
    c3 = synth.config3(values=False)
    assert c3.sparse.shape == (1, 32, 256, 64) and c3.sparse.dtype == np.uint16
    n = (c3.sparse != 0xFFFF).sum(axis=3)
    assert n.min() >= 1 and n.max() <= 16
    c4 = synth.config4(values=False)
    assert c4.sparse.shape[0] == 8 and c4.sparse.shape[2] == 16
    assert c4.count.min() >= 1 and c4.count.max() <= 16
