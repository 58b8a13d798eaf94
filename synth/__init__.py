"""Seeded synthetic inputs for block-sparse varlen attention.

This module only draws random inputs (sequence lengths, block-selection
structures, page permutations and the Q/K/V/dO values) and rounds them to the
storage dtype.  It holds none of the attention arithmetic; both the CPU oracle
tests and the GPU path consume what it produces.

Conventions (shared by every consumer):

* ``cu_q`` / ``cu_kv``: int64 ``[B+1]`` prefix sums, first entry 0
  (GenericBlockSparseAttention page, parameter table, ``cuSeqLengthsQ``).
* ``seqused_kv``: int32 ``[B]`` valid KV lengths, used with the paged layout.
* Block mask: uint8 ``[B, Hs, rows, W]``, nonzero = compute
  (BlockSparseAttentionGrad README, ``blockSparseMaskOptional``).
* sabi: uint16 ``[B, Hs, rows, W]``, ascending, padded with 0xFFFF
  (BlitzSparseAttention page, "sabi block-sparse index" section).
* idx/count: int32 ``[Hs, totalQBlocks, W]`` padded with -1 and int32
  ``[Hs, totalQBlocks]`` (GenericBlockSparseAttention page,
  ``sparseBlockIdx`` / ``sparseBlockCount``, layoutSparsePattern 4 / 6);
  the table's other layouts: ``idx_b`` ``[B, Hs, maxQBlocks, W]`` (0 / 2),
  ``kvidx`` ``[Hs, totalKBlocks, W]`` listing q-blocks per KV block (5 / 7),
  ``kvidx_b`` ``[B, Hs, maxKvBlocks, W]`` (1 / 3), each with its count
  tensor of the leading shape.
* Paged K/V: ``[pages, page_size, N2, D]`` with an int32 ``block_table``
  ``[B, max_pages]`` padded with -1 (GenericBlockSparseAttention page,
  "Paged Attention" table).

Tensors are returned twice: ``*_bits`` (the storage pattern the GPU reads:
uint16 for bf16 / fp16, uint8 for fp8) and the float32 array holding exactly
the same rounded values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

MASK_NONE, MASK_CAUSAL = 0, 1


def _e4m3_table():
    """Values of the 127 non-negative finite FLOAT8_E4M3 (OCP e4m3fn) codes
    0x00..0x7E: 4 exponent bits with bias 7, 3 mantissa bits, subnormals at
    exponent 0, no infinities, 0x7F the NaN."""
    codes = np.arange(0x7F)
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7)).astype(np.float64)


_E4M3 = _e4m3_table()


def round_to_e4m3(x: np.ndarray):
    """float32 -> FLOAT8_E4M3 (e4m3fn) codes, rounding to nearest with ties to
    the even code and saturating at +-448; NaN -> 0x7F.  Returns
    ``(codes uint8, values float32)``."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    hi = np.clip(np.searchsorted(_E4M3, a, side="left"), 0, len(_E4M3) - 1)  # first code >= a
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3[lo], _E4M3[hi] - a
    pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(hi % 2 == 0, hi, lo)))
    pick = np.where(_E4M3[hi] == a, hi, pick)
    codes = (pick | np.where(np.signbit(x) & (pick > 0), 0x80, 0)).astype(np.uint8)
    nan = np.isnan(x)
    codes[nan] = 0x7F
    vals = np.where(np.signbit(x) & (pick > 0), -1.0, 1.0) * _E4M3[pick]
    vals = vals.astype(np.float32)
    vals[nan] = np.nan
    return codes, vals


def round_to_dtype(x: np.ndarray, dtype: str):
    """Round float32 ``x`` to ``dtype`` ('bf16', 'f16' or 'fp8' = e4m3fn).

    Returns ``(bits, values float32)``, bits uint16 (uint8 for fp8).  bf16
    uses round-to-nearest-even on the float32 bit pattern; NaN stays NaN.
    """
    if dtype == "fp8":
        return round_to_e4m3(x)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        h = x.astype(np.float16)
        return h.view(np.uint16).copy(), h.astype(np.float32)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x.view(np.uint32)
    # finite values never wrap in uint32 here; NaN is replaced below
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    bits = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        bits[nan] = 0x7FC0
    vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits, vals


@dataclasses.dataclass
class Case:
    name: str
    dtype: str  # of q, k, v, dout: 'bf16', 'f16' or 'fp8' (e4m3fn, forward only)
    out_dtype: str  # of out / dq / dk / dv: '' = dtype; 'bf16' or 'f16' with fp8 inputs
    B: int
    N1: int
    N2: int
    D: int
    bx: int
    by: int
    sparse_kind: str  # 'none' | 'mask' | 'sabi' | 'idx'
    sparse_heads: int
    causal: bool
    paged: bool
    page_size: int
    scale: float  # 0.0 means 1/sqrt(D)
    cu_q: np.ndarray
    cu_kv: Optional[np.ndarray]
    seqused_kv: Optional[np.ndarray]
    sparse: Optional[np.ndarray]
    count: Optional[np.ndarray]
    block_table: Optional[np.ndarray]
    q_bits: np.ndarray
    q: np.ndarray
    k_bits: np.ndarray
    k: np.ndarray
    v_bits: np.ndarray
    v: np.ndarray
    dout_bits: Optional[np.ndarray] = None
    dout: Optional[np.ndarray] = None
    band: Optional[tuple] = None  # (preTokens, nextTokens) of a band mask, or None

    # ---- derived shape facts (pure bookkeeping, no attention arithmetic) ----
    @property
    def lens_q(self):
        return np.diff(self.cu_q).astype(np.int64)

    @property
    def lens_kv(self):
        if self.paged:
            return self.seqused_kv.astype(np.int64)
        return np.diff(self.cu_kv).astype(np.int64)

    @property
    def total_q(self):
        return int(self.cu_q[-1])

    @property
    def total_kv(self):
        """Token rows of K/V (TND) or number of pages (paged)."""
        return int(self.k.shape[0])

    @property
    def max_seqlen_q(self):
        return int(self.lens_q.max()) if self.B else 0

    @property
    def max_seqlen_kv(self):
        return int(self.lens_kv.max()) if self.B else 0

    @property
    def sparse_rows(self):
        if self.sparse is None:
            return 0
        return int(self.sparse.shape[-2])

    @property
    def sparse_width(self):
        if self.sparse is None:
            return 0
        return int(self.sparse.shape[-1])

    @property
    def max_pages_per_seq(self):
        return int(self.block_table.shape[1]) if self.paged else 0

    @property
    def page_stride(self):
        return int(self.page_size * self.N2 * self.D) if self.paged else 0


def _cdiv(a, b):
    return -(-int(a) // int(b))


_CHUNK = 1 << 22  # elements per draw; keeps temporaries small and reused


def _values(rng, shape, dtype, nan_mask=None):
    """N(0, 1) float32 draws of ``shape`` rounded to ``dtype``, generated in
    chunks along axis 0 (the generator's stream is the same as one draw).
    ``nan_mask`` (boolean over the leading axes) marks rows set to NaN."""
    shape = tuple(int(x) for x in shape)
    bits = np.empty(shape, dtype=np.uint8 if dtype == "fp8" else np.uint16)
    vals = np.empty(shape, dtype=np.float32)
    if bits.size == 0:
        return bits, vals
    row = int(np.prod(shape[1:]))
    step = max(1, _CHUNK // max(row, 1))
    for a in range(0, shape[0], step):
        b = min(shape[0], a + step)
        x = rng.standard_normal((b - a,) + shape[1:], dtype=np.float32)
        if nan_mask is not None:
            x[nan_mask[a:b]] = np.nan
        bits[a:b], vals[a:b] = round_to_dtype(x, dtype)
    return bits, vals


def _finish(rng, c: dict, with_dout: bool, kv_shape, nan_tail_mask=None, values=True):
    T, N1, D = int(c["cu_q"][-1]), c["N1"], c["D"]
    if not values:  # structure only: the value draws come last, so nothing else changes
        empty = np.zeros((0,), dtype=np.float32)
        for n in ("q", "k", "v"):
            c[n + "_bits"], c[n] = empty.view(np.uint16)[:0], empty
        return Case(**c)
    dt = c["dtype"]
    c["q_bits"], c["q"] = _values(rng, (T, N1, D), dt)
    c["k_bits"], c["k"] = _values(rng, kv_shape, dt, nan_tail_mask)
    c["v_bits"], c["v"] = _values(rng, kv_shape, dt, nan_tail_mask)
    if with_dout:
        c["dout_bits"], c["dout"] = _values(rng, (T, N1, D), dt)
    return Case(**c)


def to_fp8(case: Case, out_dtype: str = "bf16") -> Case:
    """The same case with q, k, v re-rounded to FLOAT8_E4M3 (forward only:
    dout is dropped) and ``out_dtype`` for the output."""
    c = dataclasses.replace(case, dtype="fp8", out_dtype=out_dtype, name=case.name + "_fp8",
                            dout_bits=None, dout=None)
    for n in ("q", "k", "v"):
        bits, vals = round_to_e4m3(getattr(case, n))
        setattr(c, n + "_bits", bits)
        setattr(c, n, vals)
    return c


def _base(name, dtype, B, N1, N2, D, bx, by, kind, hs, causal, paged, page_size, scale, out_dtype=""):
    return dict(name=name, dtype=dtype, out_dtype=out_dtype, B=B, N1=N1, N2=N2, D=D, bx=bx, by=by,
                sparse_kind=kind, sparse_heads=hs, causal=causal, paged=paged,
                page_size=page_size, scale=scale, cu_kv=None, seqused_kv=None,
                sparse=None, count=None, block_table=None)


def _cu(lens):
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int64)


# --------------------------------------------------------------------------
# The five benchmark-shaped workloads.  Draw order: lengths -> sparse
# structure -> page permutation -> Q, K, V, dO; generator PCG64 seeded with
# the config number; integer bounds inclusive.
# --------------------------------------------------------------------------

def config1(seed: int = 1, values: bool = True) -> Case:
    """Tiny fwd+bwd: 1x512 tokens, N1=N2=2, D=64, fp16, 128x128 blocks,
    Bernoulli(0.5) block mask with the diagonal forced on, scale 1/8."""
    rng = np.random.default_rng(seed)
    c = _base("cfg1_tiny_mask", "f16", 1, 2, 2, 64, 128, 128, "mask", 2, False, False, 0, 1.0 / 8.0)
    lens = [512]
    c["cu_q"] = _cu(lens)
    c["cu_kv"] = _cu(lens)
    m = rng.random((1, 2, 4, 4)) < 0.5
    for i in range(4):
        m[:, :, i, i] = True
    c["sparse"] = m.astype(np.uint8)
    return _finish(rng, c, True, (512, 2, 64), values=values)


def config2(seed: int = 2, values: bool = True) -> Case:
    """Dense varlen causal fwd+bwd: B=4, lengths U{512..4096}, N=16, D=128,
    bf16, no block sparsity, causal."""
    rng = np.random.default_rng(seed)
    c = _base("cfg2_dense_varlen_causal", "bf16", 4, 16, 16, 128, 128, 128, "none", 16, True, False, 0,
              1.0 / np.sqrt(128.0))
    lens = rng.integers(512, 4097, size=4)
    c["cu_q"] = _cu(lens)
    c["cu_kv"] = _cu(lens)
    T = int(c["cu_q"][-1])
    return _finish(rng, c, True, (T, 16, 128), values=values)


def config3(seed: int = 3, with_dout: bool = False, values: bool = True) -> Case:
    """sabi prefill fwd: B=1, S=32768, N=32, D=128, bf16, block (128, 512),
    sabi [1,32,256,64] with 1..16 distinct ascending entries per row."""
    rng = np.random.default_rng(seed)
    c = _base("cfg3_sabi_prefill", "bf16", 1, 32, 32, 128, 128, 512, "sabi", 32, False, False, 0,
              1.0 / np.sqrt(128.0))
    S = 32768
    c["cu_q"] = _cu([S])
    c["cu_kv"] = _cu([S])
    sabi = np.full((1, 32, 256, 64), 0xFFFF, dtype=np.uint16)
    for h in range(32):
        for i in range(256):
            n = int(rng.integers(1, 17))
            sel = np.sort(rng.choice(64, n, replace=False))
            sabi[0, h, i, :n] = sel
    c["sparse"] = sabi
    return _finish(rng, c, with_dout, (S, 32, 128), values=values)


def config4(seed: int = 4, with_dout: bool = False, values: bool = True) -> Case:
    """GQA + paged-KV fwd: B=8, lengths U{1024..8192}, N1=32, N2=8, D=128,
    bf16, 128-token pages in a random physical order, 128x128 blocks, idx
    top-16 with counts U{4..16} capped at j+1, causal."""
    rng = np.random.default_rng(seed)
    c = _base("cfg4_gqa_paged_idx", "bf16", 8, 32, 8, 128, 128, 128, "idx", 8, True, True, 128,
              1.0 / np.sqrt(128.0))
    lens = rng.integers(1024, 8193, size=8)
    c["cu_q"] = _cu(lens)
    c["seqused_kv"] = np.asarray(lens, dtype=np.int32)
    nqb = [_cdiv(L, 128) for L in lens]
    tqb = int(sum(nqb))
    idx = np.full((8, tqb, 16), -1, dtype=np.int32)
    cnt = np.zeros((8, tqb), dtype=np.int32)
    for g in range(8):
        base = 0
        for b in range(8):
            for j in range(nqb[b]):
                n = min(int(rng.integers(4, 17)), j + 1)
                sel = np.sort(rng.choice(j + 1, n, replace=False))
                idx[g, base + j, :n] = sel
                cnt[g, base + j] = n
            base += nqb[b]
    c["sparse"] = idx
    c["count"] = cnt
    npages = [_cdiv(L, 128) for L in lens]
    P = int(sum(npages))
    perm = rng.permutation(P)
    bt = np.full((8, max(npages)), -1, dtype=np.int32)
    tail = np.zeros((P, 128), dtype=bool)
    lp = 0
    for b in range(8):
        for i in range(npages[b]):
            phys = int(perm[lp + i])
            bt[b, i] = phys
            used = min(128, int(lens[b]) - 128 * i)
            tail[phys, used:] = True
        lp += npages[b]
    c["block_table"] = bt
    return _finish(rng, c, with_dout, (P, 128, 8, 128), nan_tail_mask=tail, values=values)


def config5(seed: int = 5, values: bool = True) -> Case:
    """Long-context fwd+bwd: B=2 x 16384, N1=N2=16, D=128, bf16, 128x128,
    block-causal mask keeping the diagonal, 4 preceding and 8 random earlier
    blocks per row."""
    rng = np.random.default_rng(seed)
    c = _base("cfg5_longctx_mask", "bf16", 2, 16, 16, 128, 128, 128, "mask", 16, False, False, 0,
              1.0 / np.sqrt(128.0))
    lens = [16384, 16384]
    c["cu_q"] = _cu(lens)
    c["cu_kv"] = _cu(lens)
    m = np.zeros((2, 16, 128, 128), dtype=np.uint8)
    for b in range(2):
        for h in range(16):
            for i in range(128):
                m[b, h, i, i] = 1
                m[b, h, i, max(0, i - 4):i] = 1
                if i >= 5:
                    sel = rng.choice(i - 4, min(8, i - 4), replace=False)
                    m[b, h, i, sel] = 1
    c["sparse"] = m
    return _finish(rng, c, True, (32768, 16, 128), values=values)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def config6(seed: int = 6, values: bool = True, with_dout: bool = True) -> Case:
    """Per-token selection (GenericBlockSparseAttention's default block
    shape [1, 128]): TND B=2 x 4096 tokens, N1=32, N2=8, D=128, bf16; every
    query token picks its own KV blocks: idx [8, 8192, 16], count
    min(U{4..16}, j // 128 + 1) distinct blocks <= its own block, -1 pad;
    causal.  A measurement workload beside the five benchmark ones."""
    rng = np.random.default_rng(seed)
    c = _base("cfg6_per_token", "bf16", 2, 32, 8, 128, 1, 128, "idx", 8, True, False, 0, 1.0 / np.sqrt(128.0))
    lens = [4096, 4096]
    c["cu_q"] = _cu(lens)
    c["cu_kv"] = _cu(lens)
    tq = sum(lens)
    idx = np.full((8, tq, 16), -1, dtype=np.int32)
    cnt = np.zeros((8, tq), dtype=np.int32)
    for g in range(8):
        base = 0
        for L in lens:
            for j in range(L):
                top = j // 128 + 1
                n = min(int(rng.integers(4, 17)), top)
                idx[g, base + j, :n] = np.sort(rng.choice(top, n, replace=False))
                cnt[g, base + j] = n
            base += L
    c["sparse"] = idx
    c["count"] = cnt
    return _finish(rng, c, with_dout, (tq, 8, 128), values=values)


# measurement-only workloads (not among the benchmark configurations)
EXTRA = {6: config6}


# --------------------------------------------------------------------------
# Small randomized cases for parity and edge-case tests.
# --------------------------------------------------------------------------

def random_case(seed: int, *, lens_q, lens_kv=None, N1=2, N2=None, D=64, dtype="bf16",
                bx=128, by=128, kind="mask", sparse_heads=None, causal=False, paged=False,
                page_size=128, density=0.5, width=None, scale=0.0, with_dout=True,
                messy=False, rows=None, dense_q=False, out_dtype="", band=None) -> Case:
    """Random varlen case.

    ``messy`` adds duplicates, unsorted order, out-of-range entries and
    counts outside ``[0, W]`` to sabi/idx inputs (all of which the method
    must treat as set selection with out-of-range entries skipped).
    ``dense_q`` fills the mask/sabi/idx with every block (all-selected).
    ``band`` = (preTokens, nextTokens) selects the band mask (``causal`` is
    then ignored).
    """
    rng = np.random.default_rng(seed)
    N2 = N1 if N2 is None else N2
    hs = N1 if sparse_heads is None else sparse_heads
    lens_q = [int(x) for x in lens_q]
    lens_kv = list(lens_q) if lens_kv is None else [int(x) for x in lens_kv]
    B = len(lens_q)
    c = _base(f"rand{seed}", dtype, B, N1, N2, D, bx, by, kind, hs, causal and band is None, paged, page_size,
              scale, out_dtype)
    c["band"] = None if band is None else (int(band[0]), int(band[1]))
    c["cu_q"] = _cu(lens_q)
    nqb = [_cdiv(L, bx) for L in lens_q]
    nkb = [_cdiv(L, by) for L in lens_kv]
    max_nqb = max(nqb) if B else 0
    max_nkb = max(nkb) if B else 0
    if paged:
        c["seqused_kv"] = np.asarray(lens_kv, dtype=np.int32)
    else:
        c["cu_kv"] = _cu(lens_kv)
    R = max(max_nqb, 1) if rows is None else rows
    if kind == "mask":
        W = max(max_nkb, 1) if width is None else width
        m = (rng.random((B, hs, R, W)) < density)
        if dense_q:
            m[:] = True
        c["sparse"] = m.astype(np.uint8)
    elif kind == "sabi":
        W = max(max_nkb, 1) if width is None else width
        s = np.full((B, hs, R, W), 0xFFFF, dtype=np.uint16)
        for b in range(B):
            for h in range(hs):
                for i in range(R):
                    pool = max(nkb[b], 1)
                    if dense_q:
                        sel = np.arange(min(pool, W))
                    else:
                        n = int(rng.integers(0, min(pool, W) + 1))
                        sel = np.sort(rng.choice(pool, n, replace=False))
                    if messy and len(sel):
                        extra = rng.integers(0, pool + 3, size=int(rng.integers(0, 3)))
                        sel = np.concatenate([sel, extra])
                        rng.shuffle(sel)
                        sel = sel[:W]
                    s[b, h, i, :len(sel)] = sel
        c["sparse"] = s
    elif kind == "idx":
        tqb = int(sum(nqb))
        W = max(max_nkb, 1) if width is None else width
        idx = np.full((hs, tqb, W), -1, dtype=np.int32)
        cnt = np.zeros((hs, tqb), dtype=np.int32)
        base = 0
        for b in range(B):
            for j in range(nqb[b]):
                for h in range(hs):
                    pool = max(nkb[b], 1)
                    if dense_q:
                        sel = np.arange(min(pool, W))
                    else:
                        n = int(rng.integers(0, min(pool, W) + 1))
                        sel = np.sort(rng.choice(pool, n, replace=False))
                    if messy:
                        extra = rng.integers(-2, pool + 3, size=int(rng.integers(0, 3)))
                        sel = np.concatenate([sel, extra])
                        rng.shuffle(sel)
                        sel = sel[:W]
                    idx[h, base + j, :len(sel)] = sel
                    n_cnt = len(sel)
                    if messy and rng.random() < 0.2:
                        n_cnt = int(rng.integers(-1, W + 3))
                    cnt[h, base + j] = n_cnt
            base += nqb[b]
        c["sparse"] = idx
        c["count"] = cnt
    elif kind in ("idx_b", "kvidx", "kvidx_b"):
        # idx_b: [B, Hs, rows, W] lists of KV blocks per local q-block;
        # kvidx: [Hs, totalKBlocks, W] lists of local q-blocks per global KV
        # block; kvidx_b: [B, Hs, rows, W] the same per local KV block
        per_kv = kind != "idx_b"
        lists_n = nkb if per_kv else nqb  # lists per sequence
        pools = nqb if per_kv else nkb    # what a list's entries index
        Wd = max(max(pools) if B else 1, 1)
        W = Wd if width is None else width
        if kind == "kvidx":
            tkb = int(sum(nkb))
            idx = np.full((hs, tkb, W), -1, dtype=np.int32)
            cnt = np.zeros((hs, tkb), dtype=np.int32)
        else:
            Rl = max(max(lists_n) if B else 1, 1) if rows is None else rows
            idx = np.full((B, hs, Rl, W), -1, dtype=np.int32)
            cnt = np.zeros((B, hs, Rl), dtype=np.int32)
        base = 0
        for b in range(B):
            for j in range(lists_n[b]):
                for h in range(hs):
                    pool = max(pools[b], 1)
                    if dense_q:
                        sel = np.arange(min(pool, W))
                    else:
                        n = int(rng.integers(0, min(pool, W) + 1))
                        sel = np.sort(rng.choice(pool, n, replace=False))
                    if messy:
                        extra = rng.integers(-2, pool + 3, size=int(rng.integers(0, 3)))
                        sel = np.concatenate([sel, extra])
                        rng.shuffle(sel)
                        sel = sel[:W]
                    n_cnt = len(sel)
                    if messy and rng.random() < 0.2:
                        n_cnt = int(rng.integers(-1, W + 3))
                    if kind == "kvidx":
                        idx[h, base + j, :len(sel)] = sel
                        cnt[h, base + j] = n_cnt
                    elif j < idx.shape[2]:
                        idx[b, h, j, :len(sel)] = sel
                        cnt[b, h, j] = n_cnt
            base += lists_n[b]
        c["sparse"] = idx
        c["count"] = cnt
    elif kind != "none":
        raise ValueError(kind)
    nan_tail = None
    if paged:
        npages = [_cdiv(L, page_size) for L in lens_kv]
        P = int(sum(npages)) + 1  # one spare page nobody references
        perm = rng.permutation(P)
        bt = np.full((B, max(max(npages), 1) + 1), -1, dtype=np.int32)
        nan_tail = np.zeros((P, page_size), dtype=bool)
        nan_tail[int(perm[-1]), :] = True
        lp = 0
        for b in range(B):
            for i in range(npages[b]):
                phys = int(perm[lp + i])
                bt[b, i] = phys
                used = min(page_size, lens_kv[b] - page_size * i)
                nan_tail[phys, used:] = True
            lp += npages[b]
        c["block_table"] = bt
        kv_shape = (P, page_size, N2, D)
    else:
        kv_shape = (int(sum(lens_kv)), N2, D)
    return _finish(rng, c, with_dout, kv_shape, nan_tail_mask=nan_tail)


def ones_case(S=512, N=8, D=128, dtype="f16", scale=0.0, bx=128, by=128) -> Case:
    """All-ones Q/K/V with a dense sabi, the shape of the BlitzSparseAttention
    page's worked example ([1, 8, 512, 128], sabi [1, 8, 4, 4])."""
    c = _base("ones", dtype, 1, N, N, D, bx, by, "sabi", N, False, False, 0, scale)
    c["cu_q"] = _cu([S])
    c["cu_kv"] = _cu([S])
    nq, nk = _cdiv(S, bx), _cdiv(S, by)
    sabi = np.tile(np.arange(nk, dtype=np.uint16), (1, N, nq, 1))
    c["sparse"] = sabi
    one = np.ones((S, N, D), dtype=np.float32)
    c["q_bits"], c["q"] = round_to_dtype(one, dtype)
    c["k_bits"], c["k"] = round_to_dtype(one, dtype)
    c["v_bits"], c["v"] = round_to_dtype(one, dtype)
    c["dout_bits"], c["dout"] = round_to_dtype(one, dtype)
    return Case(**c)
