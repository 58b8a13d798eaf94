"""Plain, slow, fp64 CPU oracle for variable-length block-sparse attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the library or its binding.

What it computes (exact attention restricted to the selected blocks, no
approximation), with the passage each part follows:

* Forward ``O = softmax(scale * Q K_sel^T, mask) V_sel`` and the natural-log
  log-sum-exp ``lse`` -- BlockSparseAttentionGrad README, "Function
  description" (the forward formula it restates), GenericBlockSparseAttention
  page, "Sparse attention mechanism", BlitzSparseAttention page, "softmax_lse
  output" and its all-ones example (LSE = ln S + sqrt(D)).
* Backward ``dV = P^T dO``, ``dP = dO V^T``, ``dS = P o (dP - rowsum(dO o O))``,
  ``dQ = scale dS K``, ``dK = scale dS^T Q`` -- BlockSparseAttentionGrad README,
  "Function description" backward formulas.
* Block selection formats: bool block mask (BlockSparseAttentionGrad README,
  ``blockSparseMaskOptional``), uint16 sabi padded with 0xFFFF
  (BlitzSparseAttention page, sabi section), int32 sparseBlockIdx/Count padded
  with -1 over global q-blocks (GenericBlockSparseAttention page, parameter
  table and "Blocking and addressing" constraint), and the other
  layoutSparsePattern forms of the same page's table: per-Q-block lists with a
  batch axis (values 0 / 2), and per-KV-block lists -- each KV block names
  the q-blocks that chose it -- over global KV blocks (5 / 7) or with a batch
  axis (1 / 3).
* Varlen ``cu_seqlens`` with a leading 0 and ``seqused_kv`` for the paged
  layout; paged K/V ``[pages, page_size, N2, D]`` addressed through a block
  table (GenericBlockSparseAttention page, parameter table, "Paged Attention").
* Causal masking aligned at the bottom-right corner (FlashAttention
  UnpaddingScoreGradV2 page, sparseMode table, rightDownCausal, the only
  causal form its TND layout accepts).
* Band masking (sparseMode 4, "band", on the FlashAttention
  UnpaddingScoreGradV2 page, section 6.6, and the BlitzSparseAttention page's
  sparseMode limits): query ``i`` may attend to keys ``j`` with
  ``i + Skv - Sq - preTokens <= j <= i + Skv - Sq + nextTokens``, where
  preTokens counts the earlier tokens the sliding window keeps and nextTokens
  the later ones (PromptFlashAttention page, attribute table; the
  BlockSparseAttentionGrad README's preTokens / nextTokens rows).  The
  alignment at the bottom-right corner is the reading that the
  BlitzSparseAttention page's row-dropping conditions for band support (rows
  fall out when preTokens < 0, or when nextTokens + Skv - Sq < 0); the causal
  mask is the band with an unbounded preTokens and nextTokens = 0.

Readings where the pages are silent (each listed in the design doc): a selection is
a *set* (duplicates count once, order is irrelevant); entries outside
``[0, nKB_b)`` are skipped; counts are clamped to ``[0, W]``; KV indices are
local to the sequence; ``g(h) = h // (N1 / N2)``; the band mask is aligned at
the bottom-right corner as the causal mask is; a query row with no allowed
key has ``O = 0`` and ``lse = +inf``; the fp32-rounded scale is used
(``scale == 0`` means ``1/sqrt(D)``).

Everything is evaluated in float64 on the stored (bf16/fp16-rounded) values.
The softmax is evaluated two-pass (max, then sums), not online.
"""
from __future__ import annotations

import math

import numpy as np

SABI_SKIP = 0xFFFF


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def scale_of(scale: float, D: int) -> float:
    """The scale the method applies: ``scale`` or, when 0, ``1/sqrt(D)``
    (GenericBlockSparseAttention page, ``scaleValue``), rounded to fp32."""
    s = scale if scale != 0.0 else 1.0 / math.sqrt(D)
    return float(np.float32(s))


def lengths(case):
    """Per-sequence query and key lengths.

    Query: differences of ``cu_q`` (int64 [B+1], first 0).  Keys: differences
    of ``cu_kv`` for the packed layout, ``seqused_kv`` for the paged layout
    (GenericBlockSparseAttention page, ``cuSeqLengthsQ``/``sequsedKv``).
    """
    B = case.B
    sq = [int(case.cu_q[b + 1]) - int(case.cu_q[b]) for b in range(B)]
    if case.paged:
        skv = [int(case.seqused_kv[b]) for b in range(B)]
    else:
        skv = [int(case.cu_kv[b + 1]) - int(case.cu_kv[b]) for b in range(B)]
    return sq, skv


def _blocking(case):
    sq, skv = lengths(case)
    nqb = [_cdiv(s, case.bx) for s in sq]
    nkb = [_cdiv(s, case.by) for s in skv]
    qbase = [0] * len(nqb)
    kbase = [0] * len(nkb)
    for b in range(1, len(nqb)):
        qbase[b] = qbase[b - 1] + nqb[b - 1]
        kbase[b] = kbase[b - 1] + nkb[b - 1]
    return sq, skv, nqb, nkb, qbase, kbase


def selected_blocks(case, b: int, hs: int, qb: int, nkb_b: int, qbase_b: int):
    """``Sel(b, hs, qb)``: the KV blocks of sequence ``b`` that the selection
    names for q-block ``qb`` of sparse head ``hs``, as a sorted list.

    * none: every block ``[0, nKB_b)``.
    * mask: columns ``kb < nKB_b`` whose byte is nonzero (1 = compute).
    * sabi: entries other than 0xFFFF, below ``nKB_b``.
    * idx: the first ``clamp(count, 0, W)`` entries that lie in ``[0, nKB_b)``;
      the q axis is the global q-block ``qbase_b + qb``.
    Rows past the selection tensor's row dimension select nothing.
    """
    kind = case.sparse_kind
    if kind == "none":
        return list(range(nkb_b))
    sp = case.sparse
    if kind == "mask":
        if qb >= sp.shape[2]:
            return []
        row = sp[b, hs, qb]
        return [kb for kb in range(min(nkb_b, row.shape[0])) if row[kb] != 0]
    if kind == "sabi":
        if qb >= sp.shape[2]:
            return []
        row = sp[b, hs, qb]
        return sorted({int(x) for x in row if int(x) != SABI_SKIP and int(x) < nkb_b})
    if kind == "idx":
        gq = qbase_b + qb
        if gq >= sp.shape[1]:
            return []
        W = sp.shape[2]
        n = min(max(int(case.count[hs, gq]), 0), W)
        return sorted({int(x) for x in sp[hs, gq, :n] if 0 <= int(x) < nkb_b})
    if kind == "idx_b":  # [B, Hs, maxQBlocks, W], local q-blocks
        if qb >= sp.shape[2]:
            return []
        W = sp.shape[3]
        n = min(max(int(case.count[b, hs, qb]), 0), W)
        return sorted({int(x) for x in sp[b, hs, qb, :n] if 0 <= int(x) < nkb_b})
    if kind in ("kvidx", "kvidx_b"):
        # per-KV-block lists: kb is selected for q-block qb when qb is among
        # the first clamp(count, 0, W) entries of kb's list
        chosen = []
        for kb in range(nkb_b):
            lst = kv_list(case, b, hs, kb)
            if qb in lst:
                chosen.append(kb)
        return chosen
    raise ValueError(kind)


def kv_list(case, b: int, hs: int, kb: int):
    """The q-blocks (local to sequence ``b``) that KV block ``kb`` of sparse
    head ``hs`` lists, as a set: the first ``clamp(count, 0, W)`` entries; list
    rows past the tensor's row dimension list nothing.  ``kvidx`` holds
    ``[Hs, totalKBlocks, W]`` over global KV blocks ``kbase_b + kb``
    (layoutSparsePattern 5 / 7), ``kvidx_b`` ``[B, Hs, maxKvBlocks, W]``
    (layoutSparsePattern 1 / 3)."""
    sp, cnt = case.sparse, case.count
    if case.sparse_kind == "kvidx":
        _, _, _, _, _, kbase = _blocking(case)
        gk = kbase[b] + kb
        if gk >= sp.shape[1]:
            return set()
        n = min(max(int(cnt[hs, gk]), 0), sp.shape[2])
        return {int(x) for x in sp[hs, gk, :n]}
    if kb >= sp.shape[2]:
        return set()
    n = min(max(int(cnt[b, hs, kb]), 0), sp.shape[3])
    return {int(x) for x in sp[b, hs, kb, :n]}


def band_of(case):
    """``(preTokens, nextTokens)`` of the case's band mask, or None."""
    return getattr(case, "band", None)


def allowed_key_range(i: int, sq_b: int, skv_b: int, case):
    """Inclusive range ``[lo, hi]`` of keys query ``i`` may attend to before
    the block selection: ``[0, Skv-1]``; under the bottom-right causal mask
    ``hi = min(Skv-1, i + Skv - Sq)``; under the band mask
    ``lo = max(0, i + Skv - Sq - preTokens)``,
    ``hi = min(Skv-1, i + Skv - Sq + nextTokens)``.  Empty when ``lo > hi``."""
    lo, hi = 0, skv_b - 1
    off = skv_b - sq_b
    band = band_of(case)
    if band is not None:
        pre, nxt = band
        lo = max(lo, i + off - pre)
        hi = min(hi, i + off + nxt)
    elif case.causal:
        hi = min(hi, i + off)
    return lo, hi


def visited_blocks(case, b, hs, qb, sq_b, skv_b, nkb_b, qbase_b):
    """``V``: the selected blocks holding at least one allowed (query, key)
    pair for the rows of q-block ``qb``.

    Every row's allowed keys form one range (``allowed_key_range``), and the
    range of row ``i + 1`` is that of row ``i`` moved up by one key (before
    clipping to ``[0, Skv)``), holding ``preTokens + nextTokens + 1`` keys under
    the band mask.  When that count is at least one, consecutive ranges meet,
    so the union over the q-block's rows is the range from the first row's
    lower end to the last row's upper end; a block is visited when it meets
    that union.  When it is below one, no row has any key."""
    sel = selected_blocks(case, b, hs, qb, nkb_b, qbase_b)
    band = band_of(case)
    if band is not None and band[0] + band[1] < 0:
        return []
    first_row = qb * case.bx
    last_row = min((qb + 1) * case.bx, sq_b) - 1
    lo, _ = allowed_key_range(first_row, sq_b, skv_b, case)
    _, hi = allowed_key_range(last_row, sq_b, skv_b, case)
    return [kb for kb in sel if kb * case.by <= hi and min((kb + 1) * case.by, skv_b) - 1 >= lo]


def _q_heads_of_sparse_head(case, hs):
    """q-heads sharing sparse head ``hs``: itself when patterns are per q-head
    (Hs == N1), or its whole GQA group when packed (Hs == N2)."""
    G = case.N1 // case.N2
    if case.sparse_heads == case.N1:
        return [hs]
    return list(range(hs * G, (hs + 1) * G))


def _sparse_head(case, h):
    G = case.N1 // case.N2
    return h if case.sparse_heads == case.N1 else h // G


def index_products(case, with_csc=True):
    """The block-index products, defined exactly so that another
    implementation can be compared bit for bit.

    * rows ``r = hs * totalQBlocks + qbase_b + qb`` (head-major over global
      q-blocks, the order of GenericBlockSparseAttention's
      ``[N2, totalQBlocks, topK]`` index tensor);
    * ``row_ptr`` / ``cols``: CSR of the visited sets, each ascending;
    * ``work``: every row, ordered by visited count descending, ties by row id;
    * ``col_ptr`` / ``qrows``: the transpose, column ``c = hs * totalKBlocks +
      kbase_b + kb`` listing its q-blocks ascending (the per-KV-block layout of
      GenericBlockSparseAttention's layoutSparsePattern table, value 5);
    * ``work_kv``: items ``g * totalKBlocks + kbase_b + kb`` for every KV head
      ``g`` and block, keyed by the number of (q-head-pattern, q-block) pairs
      that reach it, descending, ties by item id.
    """
    sq, skv, nqb, nkb, qbase, kbase = _blocking(case)
    B = case.B
    Hs = case.sparse_heads
    TQB, TKB = sum(nqb), sum(nkb)
    R = Hs * TQB
    counts = np.zeros(R, dtype=np.int64)
    lists = [[] for _ in range(R)]
    for hs in range(Hs):
        for b in range(B):
            for qb in range(nqb[b]):
                r = hs * TQB + qbase[b] + qb
                v = visited_blocks(case, b, hs, qb, sq[b], skv[b], nkb[b], qbase[b])
                lists[r] = v
                counts[r] = len(v)
    row_ptr = np.zeros(R + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    cols = np.array([kb for lst in lists for kb in lst], dtype=np.int64)
    # Stable sort on the negated count: descending count, ties keep row order.
    work = np.argsort(-counts, kind="stable").astype(np.int64)
    out = dict(TQB=TQB, TKB=TKB, R=R, row_ptr=row_ptr, cols=cols, work=work, counts=counts)
    if not with_csc:
        return out
    C = Hs * TKB
    col_lists = [[] for _ in range(C)]
    for hs in range(Hs):
        for b in range(B):
            for qb in range(nqb[b]):
                for kb in lists[hs * TQB + qbase[b] + qb]:
                    col_lists[hs * TKB + kbase[b] + kb].append(qb)
    col_cnt = np.array([len(x) for x in col_lists], dtype=np.int64)
    col_ptr = np.zeros(C + 1, dtype=np.int64)
    col_ptr[1:] = np.cumsum(col_cnt)
    qrows = np.array([qb for lst in col_lists for qb in sorted(lst)], dtype=np.int64)
    N2 = case.N2
    G = case.N1 // N2
    key = np.zeros(N2 * TKB, dtype=np.int64)
    for g in range(N2):
        heads = [g] if Hs == N2 else list(range(g * G, (g + 1) * G))
        for hs in heads:
            key[g * TKB:(g + 1) * TKB] += col_cnt[hs * TKB:(hs + 1) * TKB]
    work_kv = np.argsort(-key, kind="stable").astype(np.int64)
    out.update(C=C, col_ptr=col_ptr, qrows=qrows, work_kv=work_kv, kv_key=key)
    return out


def tile_index_products(case, tile_rows=128, with_csc=True):
    """The block index over row tiles of ``tile_rows`` query rows, for
    selections whose q-blocks are narrower than a tile (``block_x`` divides
    ``tile_rows``): tile ``t`` of sequence ``b`` holds q-blocks
    ``t * (tile_rows // bx) ..`` (those below ``nQB_b``) and visits the union
    of their visited sets :func:`visited_blocks`.  This regrouping is a
    schedule, not a different method: a query row still attends only to the
    blocks its own q-block visits, which the row masks record.

    * rows ``r = hs * totalTiles + tbase_b + t`` and the CSR ``row_ptr`` /
      ``cols`` of the unions, each ascending;
    * ``row_mask``: ``[nnz, tile_rows // 32]`` uint32 per CSR entry: bit
      ``i % 32`` of word ``i // 32`` is set when row ``i`` of the tile lies in
      a q-block of the tile that visits the entry's block (all ``bx`` rows of
      such a q-block, also any past the sequence end);
    * ``work``: rows by union size descending, ties by row id;
    * ``col_ptr`` / ``qrows`` / ``col_mask``: the transpose over tiles, each
      column's tiles ascending, each entry carrying its tile's row mask for
      the column's block;
    * ``work_kv``: as in :func:`index_products`, with tiles in place of
      q-blocks.
    """
    assert tile_rows % case.bx == 0 and tile_rows % 32 == 0
    per = tile_rows // case.bx
    nw = tile_rows // 32
    sq, skv, nqb, nkb, qbase, kbase = _blocking(case)
    B, Hs = case.B, case.sparse_heads
    ntile = [_cdiv(s, tile_rows) for s in sq]
    tbase = [0]
    for n in ntile:
        tbase.append(tbase[-1] + n)
    TT, TKB = tbase[-1], sum(nkb)
    R = Hs * TT
    lists, masks = [None] * R, [None] * R
    for hs in range(Hs):
        for b in range(B):
            for t in range(ntile[b]):
                bits = {}
                for qb in range(t * per, min((t + 1) * per, nqb[b])):
                    row0 = (qb - t * per) * case.bx
                    for kb in visited_blocks(case, b, hs, qb, sq[b], skv[b], nkb[b], qbase[b]):
                        w = bits.setdefault(kb, [0] * nw)
                        for i in range(row0, row0 + case.bx):
                            w[i // 32] |= 1 << (i % 32)
                r = hs * TT + tbase[b] + t
                lists[r] = sorted(bits)
                masks[r] = [bits[kb] for kb in lists[r]]
    counts = np.array([len(x) for x in lists], dtype=np.int64)
    row_ptr = np.zeros(R + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    cols = np.array([kb for lst in lists for kb in lst], dtype=np.int64)
    row_mask = np.array([w for m in masks for w in m], dtype=np.uint32).reshape(-1, nw)
    work = np.argsort(-counts, kind="stable").astype(np.int64)
    out = dict(TQB=TT, TKB=TKB, R=R, row_ptr=row_ptr, cols=cols, row_mask=row_mask, work=work, counts=counts)
    if not with_csc:
        return out
    C = Hs * TKB
    col_lists = [[] for _ in range(C)]
    for hs in range(Hs):
        for b in range(B):
            for t in range(ntile[b]):
                r = hs * TT + tbase[b] + t
                for kb, m in zip(lists[r], masks[r]):
                    col_lists[hs * TKB + kbase[b] + kb].append((t, m))
    col_cnt = np.array([len(x) for x in col_lists], dtype=np.int64)
    col_ptr = np.zeros(C + 1, dtype=np.int64)
    col_ptr[1:] = np.cumsum(col_cnt)
    srt = [sorted(lst) for lst in col_lists]
    qrows = np.array([t for lst in srt for t, _ in lst], dtype=np.int64)
    col_mask = np.array([w for lst in srt for _, m in lst for w in m], dtype=np.uint32).reshape(-1, nw)
    N2, G = case.N2, case.N1 // case.N2
    key = np.zeros(N2 * TKB, dtype=np.int64)
    for g in range(N2):
        heads = [g] if Hs == N2 else list(range(g * G, (g + 1) * G))
        for hs in heads:
            key[g * TKB:(g + 1) * TKB] += col_cnt[hs * TKB:(hs + 1) * TKB]
    work_kv = np.argsort(-key, kind="stable").astype(np.int64)
    out.update(C=C, col_ptr=col_ptr, qrows=qrows, col_mask=col_mask, work_kv=work_kv, kv_key=key)
    return out


def _key_token_rows(case, b: int, keys: np.ndarray):
    """Physical location of local keys ``keys`` of sequence ``b``: a TND row
    ``cu_kv[b] + j``, or ``(page, slot) = (block_table[b, j // ps], j % ps)``."""
    if case.paged:
        ps = case.page_size
        pages = case.block_table[b, keys // ps].astype(np.int64)
        return pages, keys % ps
    return int(case.cu_kv[b]) + keys, None


def _gather_kv(case, arr, b, g, keys):
    rows, slots = _key_token_rows(case, b, keys)
    if slots is None:
        return arr[rows, g, :].astype(np.float64)
    return arr[rows, slots, g, :].astype(np.float64)


def _row_problem(case, b, h, qb, sq, skv, nkb, qbase):
    """Query rows, the gathered keys of the visited blocks and the allowed
    matrix for one (sequence, q-head, q-block)."""
    hs = _sparse_head(case, h)
    i0 = qb * case.bx
    i1 = min(i0 + case.bx, sq[b])
    vis = visited_blocks(case, b, hs, qb, sq[b], skv[b], nkb[b], qbase[b])
    keys = [np.arange(kb * case.by, min((kb + 1) * case.by, skv[b])) for kb in vis]
    keys = np.concatenate(keys) if keys else np.zeros(0, dtype=np.int64)
    i_loc = np.arange(i0, i1)
    rng = [allowed_key_range(int(i), sq[b], skv[b], case) for i in i_loc]
    lo = np.array([r[0] for r in rng], dtype=np.int64)
    hi = np.array([r[1] for r in rng], dtype=np.int64)
    allowed = (keys[None, :] >= lo[:, None]) & (keys[None, :] <= hi[:, None])
    return i_loc, keys, allowed


def forward(case, sample=None):
    """Forward pass.  Returns ``(O, lse)`` as float64 arrays shaped
    ``[T_q, N1, D]`` and ``[T_q, N1]``.

    ``sample``: optional iterable of ``(b, h, qb)``; only those q-blocks are
    computed and every other entry is NaN.
    """
    sq, skv, nqb, nkb, qbase, kbase = _blocking(case)
    sigma = scale_of(case.scale, case.D)
    G = case.N1 // case.N2
    T = int(case.cu_q[-1])
    O = np.full((T, case.N1, case.D), np.nan if sample is not None else 0.0)
    lse = np.full((T, case.N1), np.nan if sample is not None else np.inf)
    if sample is None:
        sample = [(b, h, qb) for b in range(case.B) for h in range(case.N1) for qb in range(nqb[b])]
    for b, h, qb in sample:
        i_loc, keys, allowed = _row_problem(case, b, h, qb, sq, skv, nkb, qbase)
        t = int(case.cu_q[b]) + i_loc
        q = case.q[t, h, :].astype(np.float64)
        g = h // G
        k = _gather_kv(case, case.k, b, g, keys)
        v = _gather_kv(case, case.v, b, g, keys)
        s = sigma * (q @ k.T)
        s = np.where(allowed, s, -np.inf)
        o = np.zeros((len(i_loc), case.D))
        l_out = np.full(len(i_loc), np.inf)
        nonempty = allowed.any(axis=1)
        if nonempty.any():
            sn = s[nonempty]
            m = sn.max(axis=1, keepdims=True)
            e = np.exp(sn - m)  # exp(-inf) = 0 on disallowed pairs
            ell = e.sum(axis=1, keepdims=True)
            o[nonempty] = (e @ v) / ell
            l_out[nonempty] = (m + np.log(ell))[:, 0]
        O[t, h, :] = o
        lse[t, h] = l_out
    return O, lse


def backward(case, sample_rows=None, sample_kv=None):
    """Exact gradient of :func:`forward` at the stored inputs, using the
    oracle's own float64 O and lse.  Returns ``(dq, dk, dv)``; dk/dv have the
    layout of ``case.k`` (TND rows or pages).

    ``sample_rows``: iterable of ``(b, h, qb)`` -- dq only for those q-blocks.
    ``sample_kv``: iterable of ``(b, g, kb)`` -- dk/dv only for those KV
    blocks.  When either is given, every output entry that is not computed
    (dq outside the sampled q-blocks, dk/dv outside the sampled KV blocks'
    keys) is NaN.  With neither, everything is computed.
    """
    sq, skv, nqb, nkb, qbase, kbase = _blocking(case)
    sigma = scale_of(case.scale, case.D)
    G = case.N1 // case.N2
    T = int(case.cu_q[-1])
    full = sample_rows is None and sample_kv is None
    dq = np.full((T, case.N1, case.D), 0.0 if full else np.nan)
    dk = np.full(case.k.shape, 0.0 if full else np.nan, dtype=np.float64)
    dv = np.full(case.v.shape, 0.0 if full else np.nan, dtype=np.float64)
    want_kv = None
    rows = set()
    if full:
        rows = {(b, h, qb) for b in range(case.B) for h in range(case.N1) for qb in range(nqb[b])}
    else:
        if sample_rows is not None:
            rows |= set(map(tuple, sample_rows))
        if sample_kv is not None:
            want_kv = set(map(tuple, sample_kv))
            for (b, g, kb) in want_kv:
                # the sampled blocks' keys start from zero (every other entry stays NaN)
                keys = np.arange(kb * case.by, min((kb + 1) * case.by, skv[b]))
                rws, slots = _key_token_rows(case, b, keys)
                if slots is None:
                    dk[rws, g] = 0.0
                    dv[rws, g] = 0.0
                else:
                    dk[rws, slots, g] = 0.0
                    dv[rws, slots, g] = 0.0
                for h in range(g * G, (g + 1) * G):
                    hs = _sparse_head(case, h)
                    for qb in range(nqb[b]):
                        if kb in visited_blocks(case, b, hs, qb, sq[b], skv[b], nkb[b], qbase[b]):
                            rows.add((b, h, qb))
    dq_rows = set(map(tuple, sample_rows)) if sample_rows is not None else set()
    for b, h, qb in sorted(rows):
        i_loc, keys, allowed = _row_problem(case, b, h, qb, sq, skv, nkb, qbase)
        t = int(case.cu_q[b]) + i_loc
        g = h // G
        q = case.q[t, h, :].astype(np.float64)
        do = case.dout[t, h, :].astype(np.float64)
        k = _gather_kv(case, case.k, b, g, keys)
        v = _gather_kv(case, case.v, b, g, keys)
        s = np.where(allowed, sigma * (q @ k.T), -np.inf)
        nonempty = allowed.any(axis=1)
        P = np.zeros_like(s)
        if nonempty.any():
            sn = s[nonempty]
            m = sn.max(axis=1, keepdims=True)
            lse = m + np.log(np.exp(sn - m).sum(axis=1, keepdims=True))
            P[nonempty] = np.exp(sn - lse)
        o = P @ v
        Dl = (do * o).sum(axis=1)  # rowsum(dO o O)
        dP = do @ v.T
        dS = P * (dP - Dl[:, None])
        if full or (b, h, qb) in dq_rows:
            dq[t, h, :] = sigma * (dS @ k)
        dk_sel = sigma * (dS.T @ q)
        dv_sel = P.T @ do
        rws, slots = _key_token_rows(case, b, keys)
        if want_kv is not None and not full:
            keep = np.array([(b, g, int(j) // case.by) in want_kv for j in keys], dtype=bool)
        else:
            keep = np.ones(len(keys), dtype=bool)
        if slots is None:
            np.add.at(dk, (rws[keep], g), dk_sel[keep])
            np.add.at(dv, (rws[keep], g), dv_sel[keep])
        else:
            np.add.at(dk, (rws[keep], slots[keep], g), dk_sel[keep])
            np.add.at(dv, (rws[keep], slots[keep], g), dv_sel[keep])
    return dq, dk, dv
