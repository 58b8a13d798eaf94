"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Index products must be bit-exact; floating point must meet the tolerances
fixed for the method: max-abs error on O <= 1e-2 (bf16) / 5e-3 (fp16), lse
within 1e-3 (+inf exactly where the oracle has +inf), relative Frobenius error
on dQ/dK/dV <= 2e-2 (bf16) / 1e-2 (fp16).  O is stored in the 16-bit input
type, so an element may also be off by the rounding to that type: the bound of
an element is the tolerance plus the exact half-ulp of the output type at
|O_ref| + tolerance (2^(e-8) for bf16, 2^(e-11) for fp16, e the binary
exponent).  A peaked row whose O is nearly one V row of magnitude 2..4 loses
up to 7.8e-3 (bf16) to storage alone.  Each check prints how many elements
exceed the literal tolerance and by how much.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_varlen_amd as bsa
from block_sparse_varlen_amd.runner import DeviceCase

pytestmark = pytest.mark.gpu

TOL_O = {"bf16": 1e-2, "f16": 5e-3}
SIG_BITS = {"bf16": 8, "f16": 11}  # significand bits of the output type
TOL_G = {"bf16": 2e-2, "f16": 1e-2}
TOL_LSE = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------- cases --

def _short_idx(case, rows):
    """The case with its idx / count tensors cut to their first `rows` global
    q-blocks (fewer than totalQBlocks)."""
    case.sparse = np.ascontiguousarray(case.sparse[:, :rows])
    case.count = np.ascontiguousarray(case.count[:, :rows])
    return case


def fwd_cases():
    R = synth.random_case
    return {
        "mask_f16_d64_ragged_empty_seq": R(101, lens_q=[300, 0, 517], N1=2, D=64, dtype="f16", kind="mask"),
        "mask_gqa_shared_causal": R(102, lens_q=[200, 385], N1=4, N2=2, D=128, kind="mask", sparse_heads=2,
                                    causal=True, density=0.6),
        "sabi_messy_causal_by256": R(103, lens_q=[257, 130], lens_kv=[600, 70], N1=2, D=128, kind="sabi",
                                     by=256, causal=True, messy=True),
        "idx_messy_gqa4_by64": R(104, lens_q=[300, 450], lens_kv=[200, 640], N1=4, N2=1, D=128, kind="idx",
                                 sparse_heads=1, by=64, messy=True, width=6),
        "idx_paged_causal": R(105, lens_q=[500, 310], lens_kv=[400, 700], N1=4, N2=2, D=128, kind="idx",
                              sparse_heads=2, causal=True, paged=True),
        "none_causal": R(106, lens_q=[129, 384, 1], N1=2, D=128, kind="none", causal=True),
        "none_long_kv_by512_f16": R(107, lens_q=[100], lens_kv=[1000], N1=2, D=128, dtype="f16", kind="none",
                                    by=512),
        "sabi_perhead_gqa_paged": R(108, lens_q=[260, 333], N1=4, N2=2, D=128, kind="sabi", sparse_heads=4,
                                    paged=True),
        "mask_d64_bf16_causal_qlong": R(109, lens_q=[700], lens_kv=[260], N1=2, D=64, kind="mask",
                                        causal=True, density=0.7),
        # q-blocks taller than one 128-row work item
        "mask_bx256_causal": R(111, lens_q=[700, 300], N1=2, D=128, kind="mask", bx=256, causal=True),
        "idx_bx512_gqa_paged_by256": R(112, lens_q=[1100, 520], lens_kv=[900, 1300], N1=4, N2=2, D=128,
                                       kind="idx", sparse_heads=2, bx=512, by=256, paged=True, page_size=256),
        # q-blocks of 64 and 192 rows (work items of 64 rows)
        "sabi_bx64_causal": R(113, lens_q=[300, 170], N1=2, D=128, kind="sabi", bx=64, causal=True),
        "mask_bx192_f16_d64": R(114, lens_q=[500, 391], lens_kv=[450, 600], N1=2, D=64, dtype="f16",
                                kind="mask", bx=192),
        # rows of more than 64 visited blocks (the block list is read 64 entries at a time)
        "none_by64_long_rows": R(115, lens_q=[256, 130], lens_kv=[4500, 9000], N1=2, D=64, kind="none", by=64),
        # q-blocks shorter than a wave's 32 rows, per-token selection, and
        # heights that are not multiples of 64
        "mask_bx16_causal": R(116, lens_q=[150, 77], N1=2, D=128, kind="mask", bx=16, causal=True, density=0.4),
        "idx_bx1_gqa": R(117, lens_q=[40, 23], lens_kv=[300, 500], N1=4, N2=2, D=64, kind="idx",
                         sparse_heads=2, bx=1, width=3),
        "sabi_bx96_f16": R(118, lens_q=[300, 161], N1=2, D=64, dtype="f16", kind="sabi", bx=96),
        # large scales: the running maximum often moves by more than the
        # rescale threshold, so the O^T rescale path runs many times per row
        "mask_scale08": R(119, lens_q=[600, 333], N1=2, D=128, kind="mask", scale=0.8, density=0.7),
        "none_causal_scale05_f16": R(120, lens_q=[400, 257], N1=2, D=64, dtype="f16", kind="none", causal=True,
                                     scale=0.5),
        # a sequence with queries but no keys (O = 0, lse = +inf for all its rows)
        "mask_skv0_seq": R(121, lens_q=[300, 200, 150], lens_kv=[400, 0, 260], N1=2, D=64, kind="mask"),
        "idx_skv0_paged_causal": R(122, lens_q=[260, 130], lens_kv=[0, 300], N1=4, N2=2, D=128, kind="idx",
                                   sparse_heads=2, causal=True, paged=True, messy=True),
        # selection tensors with fewer rows than q-blocks: the rows past them select nothing
        "mask_short_rows": R(123, lens_q=[700, 300], N1=2, D=64, kind="mask", rows=2, density=0.8),
        "sabi_short_rows_causal": R(124, lens_q=[520, 640], N1=2, D=128, kind="sabi", rows=3, causal=True),
        "idx_short_rows": _short_idx(R(125, lens_q=[600, 400], N1=4, N2=2, D=64, kind="idx", sparse_heads=2), 5),
        # the largest BlitzSparseAttention block shapes: 1024-row q-blocks
        # (8 work items each) and 1024-key KV blocks
        "mask_bx1024_by1024": R(126, lens_q=[2500, 1100], N1=2, D=64, kind="mask", bx=1024, by=1024, density=0.7),
        "sabi_bx1024_by1024_causal": R(127, lens_q=[2100, 1500], N1=2, D=128, kind="sabi", bx=1024, by=1024,
                                       causal=True),
        # band masks (preTokens, nextTokens): windows narrower and wider than a
        # block, Sq != Skv, windows that leave out the diagonal, an empty
        # window, paged GQA, tall q-blocks, one-token q-blocks
        "none_band_300_40": R(128, lens_q=[700, 333], N1=2, D=128, kind="none", band=(300, 40)),
        "mask_band_37_5_sqskv": R(129, lens_q=[520, 300], lens_kv=[800, 260], N1=2, D=64, kind="mask",
                                  density=0.8, band=(37, 5)),
        "sabi_band_neg_pre_gqa": R(130, lens_q=[400, 260], N1=4, N2=2, D=128, kind="sabi", sparse_heads=2,
                                   band=(-20, 150), dense_q=True),
        "idx_band_paged_f16": R(131, lens_q=[610, 390], lens_kv=[700, 500], N1=4, N2=2, D=128, dtype="f16",
                                kind="idx", sparse_heads=2, paged=True, band=(129, -3), dense_q=True),
        "none_band_empty_window": R(132, lens_q=[300, 150], N1=2, D=64, kind="none", band=(4, -9)),
        "mask_band_bx256_by256": R(133, lens_q=[900, 530], N1=2, D=128, kind="mask", bx=256, by=256,
                                   density=0.9, band=(600, 0)),
        "none_band_bx1_by64": R(134, lens_q=[90, 40], lens_kv=[500, 200], N1=2, D=64, kind="none", bx=1, by=64,
                                band=(70, 10)),
        # the other layoutSparsePattern forms: batch-major per-q-block lists,
        # per-KV-block lists (global and batch-major)
        "idx_b_messy_gqa_causal": R(135, lens_q=[520, 300, 0], lens_kv=[600, 310, 90], N1=4, N2=2, D=128,
                                    kind="idx_b", sparse_heads=2, messy=True, causal=True),
        "kvidx_messy_perhead_paged": R(136, lens_q=[450, 333], lens_kv=[700, 260], N1=4, N2=2, D=128,
                                       kind="kvidx", sparse_heads=4, messy=True, paged=True),
        "kvidx_b_short_rows_band_f16": R(137, lens_q=[600, 420], lens_kv=[900, 400], N1=2, D=64, dtype="f16",
                                         kind="kvidx_b", rows=5, band=(300, 60)),
        "kvidx_bx64_by256_causal": R(138, lens_q=[700, 150], N1=2, D=128, kind="kvidx", bx=64, by=256,
                                     causal=True),
        # block_y a multiple of 16: 64-key windows shared by several small
        # blocks, with the unselected 16-key groups masked
        "mask_by16_causal": R(139, lens_q=[300, 170], lens_kv=[330, 170], N1=2, D=128, kind="mask", by=16,
                              causal=True, density=0.4),
        "sabi_by48_gqa_f16": R(140, lens_q=[400, 260], N1=4, N2=2, D=64, dtype="f16", kind="sabi",
                               sparse_heads=2, by=48),
        "idx_by80_paged_causal": R(141, lens_q=[520, 300], lens_kv=[700, 310], N1=4, N2=2, D=128, kind="idx",
                                   sparse_heads=2, by=80, paged=True, causal=True, messy=True),
        "none_by16_band": R(142, lens_q=[260, 100], N1=2, D=64, kind="none", by=16, band=(100, 17)),
        "kvidx_by32_bx32": R(143, lens_q=[350, 123], lens_kv=[400, 150], N1=2, D=128, kind="kvidx", bx=32, by=32),
        # q-blocks of 1 .. 32 rows grouped into 128-row tiles with row masks:
        # per-token top-k (GenericBlockSparseAttention's default [1, 128]
        # block shape), every selection form, paged, band, short selection
        # tensors, sequences shorter than a tile and empty ones
        "tile_idx_bx1_gqa_causal": R(144, lens_q=[1500, 37, 0, 700], N1=4, N2=2, D=128, kind="idx",
                                     sparse_heads=2, bx=1, by=64, width=5, causal=True),
        "tile_mask_bx2_perhead_band": R(145, lens_q=[333, 200], lens_kv=[500, 180], N1=4, N2=2, D=64,
                                        kind="mask", sparse_heads=4, bx=2, by=64, density=0.3, band=(150, 20)),
        "tile_sabi_bx4_messy_f16": R(146, lens_q=[290, 131], N1=2, D=64, dtype="f16", kind="sabi", bx=4,
                                     messy=True, causal=True),
        "tile_idx_b_bx8_paged": R(147, lens_q=[400, 257], lens_kv=[520, 300], N1=4, N2=2, D=128, kind="idx_b",
                                  sparse_heads=2, bx=8, paged=True, messy=True),
        "tile_kvidx_bx16_causal": R(148, lens_q=[380, 250], N1=2, D=128, kind="kvidx", bx=16, causal=True),
        "tile_kvidx_b_bx32_gqa_f16": R(149, lens_q=[300, 90], lens_kv=[640, 200], N1=4, N2=2, D=128,
                                       dtype="f16", kind="kvidx_b", sparse_heads=2, bx=32, messy=True),
        "tile_none_bx1_sq_lt_skv": R(150, lens_q=[150, 70], lens_kv=[700, 400], N1=2, D=64, kind="none", bx=1,
                                     causal=True),
        "tile_idx_bx1_short_rows": _short_idx(R(151, lens_q=[260, 200], N1=2, D=128, kind="idx", bx=1, width=4,
                                                causal=True), 300),
        # the descriptor's limits: 256 q-heads (a group of 128 sharing one
        # pattern, or 256 per-q-head patterns), 4096 x 4096 blocks, top-256 lists
        "limit_n1_256_group128": R(160, lens_q=[150, 70], N1=256, N2=2, D=64, kind="mask", sparse_heads=2,
                                   causal=True, density=0.6),
        "limit_n1_256_perhead_idx": R(161, lens_q=[130], N1=256, D=64, kind="idx", width=2),
        "limit_bx4096_by4096": R(162, lens_q=[4500, 300], N1=2, D=64, kind="mask", bx=4096, by=4096, density=0.7),
        "limit_topk256_by16": R(163, lens_q=[260], lens_kv=[4200], N1=2, D=64, kind="idx", by=16, width=256),
    }


def bwd_cases():
    R = synth.random_case
    return {
        "mask_f16_d64_ragged_empty_seq": R(201, lens_q=[300, 0, 517], N1=2, D=64, dtype="f16", kind="mask"),
        "mask_gqa_shared_causal": R(202, lens_q=[200, 385], N1=4, N2=2, D=128, kind="mask", sparse_heads=2,
                                    causal=True, density=0.6),
        "sabi_messy_causal_by256": R(203, lens_q=[257, 130], lens_kv=[600, 70], N1=2, D=128, kind="sabi",
                                     by=256, causal=True, messy=True),
        "idx_perhead_gqa": R(204, lens_q=[300, 450], lens_kv=[200, 640], N1=4, N2=2, D=128, kind="idx",
                             sparse_heads=4, width=5),
        "none_causal_f16": R(205, lens_q=[129, 384, 1], N1=2, D=128, dtype="f16", kind="none", causal=True),
        "none_sq_lt_skv": R(206, lens_q=[100], lens_kv=[1000], N1=2, D=128, kind="none", causal=True),
        # paged K/V (dK/dV written in the page layout): GQA with a shared
        # pattern, pages of 64 keys (a 128-key tile spans two pages), pages of
        # 256 keys, and per-q-head sabi rows
        "idx_paged_causal_gqa": R(207, lens_q=[500, 310], lens_kv=[400, 700], N1=4, N2=2, D=128, kind="idx",
                                  sparse_heads=2, causal=True, paged=True),
        "mask_paged_ps64_f16": R(208, lens_q=[300, 200], lens_kv=[333, 450], N1=2, D=64, dtype="f16",
                                 kind="mask", paged=True, page_size=64),
        "sabi_perhead_gqa_paged_ps256": R(209, lens_q=[260, 333], N1=4, N2=2, D=128, kind="sabi",
                                          sparse_heads=4, paged=True, page_size=256, causal=True),
        # q-blocks of 256 and 512 rows (several 128-row items, 64-row dK/dV parts)
        "mask_bx256_causal_f16": R(210, lens_q=[700, 300], N1=2, D=64, dtype="f16", kind="mask", bx=256,
                                   causal=True),
        "sabi_bx512_by256_causal": R(211, lens_q=[1100, 520], lens_kv=[1300, 900], N1=2, D=128,
                                     kind="sabi", bx=512, by=256, causal=True),
        "idx_bx64_gqa_causal": R(212, lens_q=[300, 170], N1=4, N2=2, D=128, kind="idx", sparse_heads=2,
                                 bx=64, causal=True),
        "mask_bx192_paged": R(213, lens_q=[500, 391], lens_kv=[450, 600], N1=2, D=128, kind="mask", bx=192,
                              paged=True),
        "mask_long_rows_by128": R(214, lens_q=[200, 130], lens_kv=[9000, 12000], N1=2, D=64, kind="mask",
                                  density=0.9),
        # q-blocks of 16, 1, 96 and 200 rows: dK/dV parts shorter than 64 rows
        # (the rows past the q-block are masked), per-token selection
        "mask_bx16_causal": R(215, lens_q=[150, 77], N1=2, D=128, kind="mask", bx=16, causal=True, density=0.4),
        "idx_bx1_gqa_paged": R(216, lens_q=[40, 23], lens_kv=[300, 500], N1=4, N2=2, D=128, kind="idx",
                               sparse_heads=2, bx=1, width=3, paged=True),
        "sabi_bx96_causal_f16": R(217, lens_q=[300, 161], N1=2, D=64, dtype="f16", kind="sabi", bx=96,
                                  causal=True),
        "mask_bx200_perhead_gqa": R(218, lens_q=[450, 333], N1=4, N2=2, D=128, kind="mask", bx=200),
        # scale 0.8: scale * log2(e) above 1 and peaked rows (scores of std
        # ~6 at D = 64), where any extra rounding of the exp2 argument shows
        # in dK and dV
        "mask_d64_scale08": R(219, lens_q=[300, 257], N1=2, D=64, kind="mask", scale=0.8),
        "none_scale08_f16": R(220, lens_q=[200, 140], N1=2, D=128, dtype="f16", kind="none", scale=0.8),
        # a sequence with queries but no keys: its dQ is 0
        "mask_skv0_seq": R(221, lens_q=[300, 200, 150], lens_kv=[400, 0, 260], N1=2, D=64, kind="mask"),
        "idx_skv0_paged_causal": R(222, lens_q=[260, 130], lens_kv=[0, 300], N1=4, N2=2, D=128, kind="idx",
                                   sparse_heads=2, causal=True, paged=True, messy=True),
        # selection tensors with fewer rows than q-blocks
        "mask_short_rows": R(223, lens_q=[700, 300], N1=2, D=64, kind="mask", rows=2, density=0.8),
        "idx_short_rows_perhead": _short_idx(R(224, lens_q=[600, 400], N1=4, N2=2, D=64, kind="idx",
                                               sparse_heads=4), 4),
        # 1024 x 1024 blocks
        "mask_bx1024_by1024": R(225, lens_q=[2500, 1100], N1=2, D=64, kind="mask", bx=1024, by=1024, density=0.7),
        "sabi_bx1024_by1024_causal_f16": R(226, lens_q=[2100, 1500], N1=2, D=128, dtype="f16", kind="sabi",
                                           bx=1024, by=1024, causal=True),
        # band masks
        "none_band_300_40": R(227, lens_q=[700, 333], N1=2, D=128, kind="none", band=(300, 40)),
        "mask_band_37_5_sqskv_f16": R(228, lens_q=[520, 300], lens_kv=[800, 260], N1=2, D=64, dtype="f16",
                                      kind="mask", density=0.8, band=(37, 5)),
        "sabi_band_neg_pre_gqa_perhead": R(229, lens_q=[400, 260], N1=4, N2=2, D=128, kind="sabi", sparse_heads=4,
                                           band=(-20, 150), dense_q=True),
        "idx_band_paged": R(230, lens_q=[610, 390], lens_kv=[700, 500], N1=4, N2=2, D=128, kind="idx",
                            sparse_heads=2, paged=True, band=(129, -3), dense_q=True),
        "none_band_empty_window": R(231, lens_q=[300, 150], N1=2, D=64, kind="none", band=(4, -9)),
        "mask_band_bx256_by256": R(232, lens_q=[900, 530], N1=2, D=128, kind="mask", bx=256, by=256,
                                   density=0.9, band=(600, 0)),
        "none_band_bx16_sq_gt_skv": R(233, lens_q=[300, 200], lens_kv=[180, 260], N1=2, D=128, kind="none", bx=16,
                                      band=(90, 20)),
        # the other layoutSparsePattern forms
        "idx_b_messy_gqa_causal": R(234, lens_q=[520, 300, 0], lens_kv=[600, 310, 90], N1=4, N2=2, D=128,
                                    kind="idx_b", sparse_heads=2, messy=True, causal=True),
        "kvidx_messy_perhead_paged": R(235, lens_q=[450, 333], lens_kv=[700, 260], N1=4, N2=2, D=128,
                                       kind="kvidx", sparse_heads=4, messy=True, paged=True),
        "kvidx_b_short_rows_band_f16": R(236, lens_q=[600, 420], lens_kv=[900, 400], N1=2, D=64, dtype="f16",
                                         kind="kvidx_b", rows=5, band=(300, 60)),
        # block_y not a multiple of 128: a KV block's last 128-key dK/dV tile
        # is partial (64, 16, 48, 80 keys)
        "mask_by64": R(237, lens_q=[300, 170], lens_kv=[330, 200], N1=2, D=128, kind="mask", by=64),
        "mask_by16_causal": R(238, lens_q=[300, 170], N1=2, D=64, kind="mask", by=16, causal=True, density=0.4),
        "sabi_by48_gqa_paged_f16": R(239, lens_q=[400, 260], N1=4, N2=2, D=128, dtype="f16", kind="sabi",
                                     sparse_heads=2, by=48, paged=True),
        "idx_by80_band": R(240, lens_q=[520, 300], lens_kv=[700, 310], N1=4, N2=2, D=128, kind="idx",
                           sparse_heads=4, by=80, band=(200, 30)),
        "sabi_by192_causal": R(241, lens_q=[700, 400], N1=2, D=128, kind="sabi", by=192, causal=True),
        # row tiles (q-blocks of 1 .. 32 rows): the dK/dV stages take the
        # column masks, the dQ pass the row masks
        "tile_idx_bx1_gqa_causal": R(242, lens_q=[1500, 37, 0, 700], N1=4, N2=2, D=128, kind="idx",
                                     sparse_heads=2, bx=1, by=64, width=5, causal=True),
        "tile_mask_bx2_perhead_band_f16": R(243, lens_q=[333, 200], lens_kv=[500, 180], N1=4, N2=2, D=64,
                                            dtype="f16", kind="mask", sparse_heads=4, bx=2, by=64, density=0.3,
                                            band=(150, 20)),
        "tile_sabi_bx4_messy": R(244, lens_q=[290, 131], N1=2, D=128, kind="sabi", bx=4, messy=True, causal=True),
        "tile_idx_b_bx8_paged": R(245, lens_q=[400, 257], lens_kv=[520, 300], N1=4, N2=2, D=128, kind="idx_b",
                                  sparse_heads=2, bx=8, paged=True, messy=True),
        "tile_kvidx_bx16_by256": R(246, lens_q=[380, 250], lens_kv=[700, 250], N1=2, D=128, kind="kvidx", bx=16,
                                   by=256, causal=True),
        "tile_kvidx_b_bx32_gqa": R(247, lens_q=[300, 90], lens_kv=[640, 200], N1=4, N2=2, D=64,
                                   kind="kvidx_b", sparse_heads=2, bx=32, messy=True),
        "tile_none_bx1_sq_lt_skv": R(248, lens_q=[150, 70], lens_kv=[700, 400], N1=2, D=128, kind="none", bx=1,
                                     causal=True),
        "tile_mask_bx16_skv0_seq": R(249, lens_q=[300, 200, 150], lens_kv=[400, 0, 260], N1=2, D=64, kind="mask",
                                     bx=16, density=0.3),
        "tile_none_bx4_band_empty_window": R(250, lens_q=[300, 150], N1=2, D=64, kind="none", bx=4, band=(4, -9)),
        "tile_sabi_bx8_paged_ps64_gqa_f16": R(251, lens_q=[333, 260], lens_kv=[400, 512], N1=4, N2=2, D=128,
                                              dtype="f16", kind="sabi", sparse_heads=2, bx=8, paged=True,
                                              page_size=64, causal=True),
        "tile_idx_bx32_short_rows_perhead": _short_idx(R(252, lens_q=[600, 400], N1=4, N2=2, D=64, kind="idx",
                                                         sparse_heads=4, bx=32, width=5), 20),
        "limit_n1_256_group128": R(260, lens_q=[150, 70], N1=256, N2=2, D=64, kind="mask", sparse_heads=2,
                                   causal=True, density=0.6),
        "limit_n1_256_perhead_idx": R(261, lens_q=[130], N1=256, D=64, kind="idx", width=2),
        "limit_bx4096_by4096": R(262, lens_q=[4500, 300], N1=2, D=64, kind="mask", bx=4096, by=4096, density=0.7),
        "limit_topk256_by16": R(263, lens_q=[260], lens_kv=[4200], N1=2, D=64, kind="idx", by=16, width=256),
    }


FWD = fwd_cases()
BWD = bwd_cases()


def empty_rows_case():
    c = synth.random_case(110, lens_q=[384], N1=2, D=128, kind="mask")
    c.sparse[:, :, 1, :] = 0  # q-block 1 selects nothing -> O = 0, lse = +inf
    c.sparse[:, 1, :, 2] = 0  # kv block 2 unreached by head 1 -> dK = dV = 0 there
    return c


# ----------------------------------------------------------------- helpers --

def half_ulp(x, dtype):
    """Half an ulp of the 16-bit type at magnitude x (normal range): the most
    that rounding a value of that size to the type can move it."""
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
    return 2.0 ** (e - SIG_BITS[dtype])


def check_fwd(case, dc, sample=None, tag=""):
    O = dc.out.float().cpu().numpy()
    L = dc.lse.cpu().numpy()
    Or, Lr = oracle.forward(case, sample)
    sel = ~np.isnan(Lr)
    if sample is None:
        assert sel.all()
    d = np.abs(O[sel] - Or[sel])
    err = d.max() if sel.any() else 0.0
    tol = TOL_O[case.dtype]
    bound = tol + half_ulp(np.abs(Or[sel]) + tol, case.dtype)
    worst = (d / bound).max() if sel.any() else 0.0
    over = d > tol
    n_over = int(over.sum())
    lit = f"literal {tol:g}: {n_over} over" + (f" (max {d[over].max():.3e} at |O|={np.abs(Or[sel])[over].max():.2f})"
                                             if n_over else "")
    inf_r = np.isinf(Lr) & sel
    assert np.array_equal(np.isinf(L) & sel, inf_r), f"{tag}: +inf lse positions differ"
    fin = sel & ~inf_r
    lerr = np.abs(L[fin] - Lr[fin]).max() if fin.any() else 0.0
    say(f"  {tag}: max|dO|={err:.3e} (max err/bound {worst:.3f}; {lit}) max|dlse|={lerr:.3e} rows={int(sel.sum())}")
    assert worst <= 1.0, f"{tag}: O error {err}"
    assert lerr <= TOL_LSE, f"{tag}: lse error {lerr}"


def rel_fro(x, r):
    d = np.linalg.norm((x - r).ravel())
    n = np.linalg.norm(r.ravel())
    return d / n if n > 0 else d


def kv_valid(case):
    """Positions of k/v holding a sequence's key: every TND row, or the
    (page, slot) pairs of keys below seqused_kv (the generator leaves NaN in
    the rest of the page pool)."""
    if not case.paged:
        return np.ones(case.k.shape[:1], dtype=bool)
    return ~np.isnan(case.k[:, :, 0, 0])


def check_bwd(case, dc, tag=""):
    dq = dc.dq.float().cpu().numpy()
    dk = dc.dk.float().cpu().numpy()
    dv = dc.dv.float().cpu().numpy()
    rq, rk, rv = oracle.backward(case)
    val = kv_valid(case)
    eq, ek, ev = rel_fro(dq, rq), rel_fro(dk[val], rk[val]), rel_fro(dv[val], rv[val])
    say(f"  {tag}: rel_fro dq={eq:.3e} dk={ek:.3e} dv={ev:.3e}")
    tol = TOL_G[case.dtype]
    assert eq <= tol and ek <= tol and ev <= tol
    # positions of the page pool that hold no key are left as they were (NaN here)
    assert np.all(np.isnan(dk[~val])) and np.all(np.isnan(dv[~val]))
    # structural zeros: q rows with no allowed key (lse = +inf) get dq = 0;
    # keys no row reaches (dv row exactly 0 in the oracle) get dk = dv = 0
    _, lse_r = oracle.forward(case)
    assert np.all(dq[np.isinf(lse_r)] == 0)
    unreached = np.all(rv == 0, axis=-1) & val[..., None]
    assert np.all(dk[unreached] == 0) and np.all(dv[unreached] == 0)


def nan_fill(*ts):
    for t in ts:
        t.fill_(float("nan"))


# ------------------------------------------------------------------- index --

@pytest.mark.parametrize("name", list(FWD))
def test_index_bit_exact(name):
    case = FWD[name]
    say(f"index {name}")
    dc = DeviceCase(case, with_bwd=True)
    got = dc.index(True)
    keys = ["row_ptr", "cols", "work", "col_ptr", "qrows", "work_kv"]
    if got["tile_rows"] != case.bx:  # narrow q-blocks grouped into row tiles
        ref = oracle.tile_index_products(case, got["tile_rows"], with_csc=True)
        keys += ["row_mask", "col_mask"]
    else:
        ref = oracle.index_products(case, with_csc=True)
    assert got["R"] == ref["R"]
    for k in keys:
        assert np.array_equal(got[k], ref[k]), k


# --------------------------------------------------------------------- fwd --

@pytest.mark.parametrize("name", list(FWD) + ["empty_rows"])
def test_fwd_small(name):
    case = FWD[name] if name != "empty_rows" else empty_rows_case()
    say(f"fwd {name}")
    dc = DeviceCase(case, with_bwd=False)
    nan_fill(dc.out, dc.lse)
    dc.fwd()
    torch.cuda.synchronize()
    check_fwd(case, dc, tag=name)


def test_fwd_deterministic():
    case = FWD["idx_paged_causal"]
    dc = DeviceCase(case, with_bwd=False)
    dc.fwd()
    o1, l1 = dc.out.clone(), dc.lse.clone()
    dc.fwd()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), dc.out.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), dc.lse.view(torch.int32))


# --------------------------------------------------------------------- bwd --

@pytest.mark.parametrize("name", list(BWD) + ["empty_rows"])
def test_bwd_small(name):
    case = BWD[name] if name != "empty_rows" else empty_rows_case()
    say(f"bwd {name}")
    dc = DeviceCase(case, with_bwd=True)
    dc.fwd()
    nan_fill(dc.dq, dc.dk, dc.dv)
    dc.bwd()
    torch.cuda.synchronize()
    check_bwd(case, dc, tag=name)


@pytest.mark.parametrize("paged", [False, True], ids=["tnd", "paged"])
def test_bwd_without_queries_zeroes_key_gradients(paged):
    """Every sequence with keys but no queries (T_q = 0): the forward is a
    no-op, and the backward writes dK = dV = 0 at every key below Skv_b (no row
    attends them), leaving the rest of a page pool as it was."""
    case = synth.random_case(160 + int(paged), lens_q=[0, 0], lens_kv=[300, 200], N1=4, N2=2, D=64, kind="mask",
                             paged=paged, page_size=128)
    say(f"bwd without queries ({'paged' if paged else 'tnd'})")
    dc = DeviceCase(case, with_bwd=True)
    dc.fwd()
    nan_fill(dc.dk, dc.dv)
    dc.bwd()
    torch.cuda.synchronize()
    dk = dc.dk.float().cpu().numpy()
    dv = dc.dv.float().cpu().numpy()
    val = kv_valid(case)
    assert np.all(dk[val] == 0) and np.all(dv[val] == 0)
    assert np.all(np.isnan(dk[~val])) and np.all(np.isnan(dv[~val]))


@pytest.mark.parametrize("name", ["mask_gqa_shared_causal", "idx_perhead_gqa", "tile_idx_bx1_gqa_causal"])
def test_bwd_deterministic(name):
    case = BWD[name]
    dc = DeviceCase(case, with_bwd=True)
    dc.fwd()
    dc.bwd()
    g1 = [t.clone() for t in (dc.dq, dc.dk, dc.dv)]
    dc.bwd()
    torch.cuda.synchronize()
    for a, b in zip(g1, (dc.dq, dc.dk, dc.dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ------------------------------------------------------- prebuilt index --

@pytest.mark.parametrize("name", ["mask_gqa_shared_causal", "idx_paged_causal_gqa", "sabi_bx512_by256_causal",
                                  "tile_idx_b_bx8_paged"])
def test_prebuilt_index(name):
    """bsa_build_index (with the transposed lists) once, then bsa_fwd and
    bsa_bwd with BSA_FLAG_INDEX_BUILT: same results as self-indexing calls,
    bit for bit."""
    case = BWD[name]
    say(f"prebuilt {name}")
    dc = DeviceCase(case, with_bwd=True)
    dc.fwd()
    dc.bwd()
    ref = [t.clone() for t in (dc.out, dc.lse, dc.dq, dc.dk, dc.dv)]
    nan_fill(dc.out, dc.lse, dc.dq, dc.dk, dc.dv)
    dc.ws.fill_(0xFF)
    dc.build_index(True)
    dc.fwd(prebuilt=True)
    dc.bwd(prebuilt=True)
    torch.cuda.synchronize()
    val = torch.from_numpy(kv_valid(case)).to(dc.dk.device)
    for a, b, nm in zip(ref, (dc.out, dc.lse, dc.dq, dc.dk, dc.dv), ("out", "lse", "dq", "dk", "dv")):
        if nm in ("dk", "dv"):
            a, b = a[val], b[val]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), nm


# ------------------------------------------------------------ guard regions --

def _guarded(like, guard, fill):
    """A buffer of `like`'s shape and dtype inside a larger one whose `guard`
    leading and trailing elements hold `fill`."""
    n = like.numel()
    big = torch.full((n + 2 * guard,), fill, dtype=like.dtype, device=like.device)
    return big, big[guard:guard + n].view(like.shape)


@pytest.mark.parametrize("name", ["mask_gqa_shared_causal", "idx_paged_causal_gqa", "mask_bx192_paged",
                                  "mask_f16_d64_ragged_empty_seq", "tile_mask_bx2_perhead_band_f16"])
def test_no_writes_outside_buffers(name):
    """Outputs and workspace sit between guard regions (NaN, or a byte pattern
    for the workspace); a forward and a backward call leave every guard as it
    was and still match the oracle."""
    case = BWD[name]
    say(f"guards {name}")
    dc = DeviceCase(case, with_bwd=True)
    G = 8192
    guards = {}
    for attr in ("out", "lse", "dq", "dk", "dv"):
        big, view = _guarded(getattr(dc, attr), G, float("nan"))
        guards[attr] = big
        setattr(dc, attr, view)
    wbig, dc.ws = _guarded(dc.ws, G, 0xA5)
    nan_fill(dc.out, dc.lse)
    dc.fwd()
    nan_fill(dc.dq, dc.dk, dc.dv)
    dc.bwd()
    torch.cuda.synchronize()
    for attr, big in guards.items():
        assert torch.isnan(big[:G]).all() and torch.isnan(big[-G:]).all(), f"{attr}: write outside the buffer"
    assert (wbig[:G] == 0xA5).all() and (wbig[-G:] == 0xA5).all(), "workspace: write outside the buffer"
    check_fwd(case, dc, tag=name)
    check_bwd(case, dc, tag=name)


# ---------------------------------------------------- benchmark workloads --

@functools.lru_cache(maxsize=1)
def _cfg(n):
    return synth.CONFIGS[n]()


def _sample_rows(case, idx, n_rand, seed):
    """Longest rows first, then random (b, h, qb) triples, then the last
    q-block of every sequence."""
    G = case.N1 // case.N2
    rng = np.random.default_rng(seed)
    TQB = idx["TQB"]
    qbase = np.concatenate([[0], np.cumsum([-(-int(s) // case.bx) for s in np.diff(case.cu_q)])])
    out = set()

    def add_row(r):
        hs, qg = divmod(int(r), TQB)
        b = int(np.searchsorted(qbase, qg, side="right") - 1)
        qb = qg - int(qbase[b])
        heads = [hs] if case.sparse_heads == case.N1 else list(range(hs * G, (hs + 1) * G))
        for h in heads[:2]:
            out.add((b, h, qb))

    for r in idx["work"][:4]:
        add_row(r)
    for r in rng.choice(idx["R"], size=min(n_rand, idx["R"]), replace=False):
        add_row(r)
    for b in range(case.B):
        n = -(-int(case.cu_q[b + 1] - case.cu_q[b]) // case.bx)
        if n:
            out.add((b, int(rng.integers(case.N1)), n - 1))
    return sorted(out)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_fwd_config(n):
    say(f"config {n}: generating")
    case = _cfg(n)
    say(f"config {n}: fwd on GPU")
    dc = DeviceCase(case, with_bwd=False)
    nan_fill(dc.out, dc.lse)
    dc.fwd()
    torch.cuda.synchronize()
    assert not torch.isnan(dc.out).any() and not torch.isnan(dc.lse).any()
    idx = oracle.index_products(case, with_csc=False)
    got = dc.index(False)
    for k in ("row_ptr", "cols", "work"):
        assert np.array_equal(got[k], idx[k]), k
    sample = None if n == 1 else _sample_rows(case, idx, 24, n)
    check_fwd(case, dc, sample=sample, tag=f"config{n}")


@functools.lru_cache(maxsize=1)
def _cfg_bwd(n):
    return synth.CONFIGS[n](with_dout=True) if n in (3, 4) else synth.CONFIGS[n]()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_bwd_config(n):
    case = _cfg_bwd(n)
    say(f"config {n}: bwd on GPU")
    dc = DeviceCase(case, with_bwd=True)
    dc.fwd()
    nan_fill(dc.dq, dc.dk, dc.dv)
    dc.bwd()
    torch.cuda.synchronize()
    assert not torch.isnan(dc.dq).any()
    val = torch.from_numpy(kv_valid(case)).to(dc.dk.device)
    for t in (dc.dk, dc.dv):  # every key position written; the rest of a page pool untouched
        assert not torch.isnan(t[val]).any()
        assert torch.isnan(t[~val]).all()
    got = dc.index(True)
    idx = oracle.index_products(case, with_csc=True)
    for k in ("row_ptr", "cols", "work", "col_ptr", "qrows", "work_kv"):
        assert np.array_equal(got[k], idx[k]), k
    if n == 1:
        check_bwd(case, dc, tag="config1")
        return
    rng = np.random.default_rng(100 + n)
    rows = _sample_rows(case, idx, 12, 50 + n)
    skv = case.seqused_kv if case.paged else np.diff(case.cu_kv)
    kbase = np.concatenate([[0], np.cumsum([-(-int(s) // case.by) for s in skv])])
    kvs = set()
    for it in list(idx["work_kv"][:3]) + list(rng.choice(len(idx["work_kv"]), 6, replace=False)):
        g, kg = divmod(int(it), idx["TKB"])
        b = int(np.searchsorted(kbase, kg, side="right") - 1)
        kvs.add((b, g, kg - int(kbase[b])))
    rq, rk, rv = oracle.backward(case, sample_rows=rows, sample_kv=sorted(kvs))
    dq = dc.dq.float().cpu().numpy()
    dk = dc.dk.float().cpu().numpy()
    dv = dc.dv.float().cpu().numpy()
    selq = ~np.isnan(rq[..., 0])
    tol = TOL_G[case.dtype]
    eq = rel_fro(dq[selq], rq[selq])
    keys = []  # (row index tuple, kv head) of every key of the sampled KV blocks
    for (b, g, kb) in kvs:
        for j in range(kb * case.by, min(int(skv[b]), (kb + 1) * case.by)):
            if case.paged:
                keys.append(((int(case.block_table[b, j // case.page_size]), j % case.page_size), g))
            else:
                keys.append(((int(case.cu_kv[b]) + j,), g))
    ix = tuple(np.array([k[0][i] for k in keys]) for i in range(len(keys[0][0]))) + (np.array([k[1] for k in keys]),)
    ek = rel_fro(dk[ix], rk[ix])
    ev = rel_fro(dv[ix], rv[ix])
    say(f"  config{n}: rel_fro dq={eq:.3e} dk={ek:.3e} dv={ev:.3e} (sampled)")
    assert eq <= tol and ek <= tol and ev <= tol


# ------------------------------------------ per-token selection, full size --

@pytest.mark.timeout(900)
def test_per_token_workload_full_size():
    """GenericBlockSparseAttention's default [1, 128] block shape at the
    bench's per-token workload size (2 x 4096 tokens, 32/8 heads, top-16 per
    token, causal), run as 128-row tiles: the tile index bit-exact (masks
    included), sampled tokens' O / lse / dQ and sampled KV blocks' dK / dV
    against the oracle."""
    say("per-token workload: generating")
    case = synth.config6()
    dc = DeviceCase(case, with_bwd=True)
    dc.fwd()
    nan_fill(dc.dq, dc.dk, dc.dv)
    dc.bwd()
    torch.cuda.synchronize()
    assert not torch.isnan(dc.out).any() and not torch.isnan(dc.dq).any()
    assert not torch.isnan(dc.dk).any() and not torch.isnan(dc.dv).any()
    got = dc.index(True)
    assert got["tile_rows"] == 128
    ref = oracle.tile_index_products(case, 128, with_csc=True)
    for k in ("row_ptr", "cols", "work", "col_ptr", "qrows", "work_kv", "row_mask", "col_mask"):
        assert np.array_equal(got[k], ref[k]), k
    rng = np.random.default_rng(66)
    rows = {(int(rng.integers(2)), int(rng.integers(32)), int(rng.integers(4096))) for _ in range(30)}
    rows |= {(0, 0, 0), (1, 31, 4095), (0, 5, 127), (1, 9, 128)}
    rows = sorted(rows)
    check_fwd(case, dc, sample=rows, tag="per-token")
    kvs = [(0, 2, 31), (1, 6, 20)]
    rq, rk, rv = oracle.backward(case, sample_rows=rows[:10], sample_kv=kvs)
    dq = dc.dq.float().cpu().numpy()
    dk = dc.dk.float().cpu().numpy()
    dv = dc.dv.float().cpu().numpy()
    selq = ~np.isnan(rq[..., 0])
    selk = ~np.isnan(rk[..., 0])
    eq, ek, ev = rel_fro(dq[selq], rq[selq]), rel_fro(dk[selk], rk[selk]), rel_fro(dv[selk], rv[selk])
    say(f"  per-token: rel_fro dq={eq:.3e} dk={ek:.3e} dv={ev:.3e} (sampled)")
    tol = TOL_G[case.dtype]
    assert eq <= tol and ek <= tol and ev <= tol


# ------------------------------------------- per-KV-block lists at full size --

def _kv_lists_of_mask(m):
    """The mask case's selection as [Hs, totalKBlocks, W] per-KV-block lists
    (each KV block names the q-blocks whose mask row selects it)."""
    import copy
    c = copy.copy(m)
    lens_q = np.diff(m.cu_q)
    lens_kv = np.diff(m.cu_kv)
    nqb = [-(-int(x) // m.bx) for x in lens_q]
    nkb = [-(-int(x) // m.by) for x in lens_kv]
    Hs, W = m.sparse_heads, max(nqb)
    idx = np.full((Hs, sum(nkb), W), -1, dtype=np.int32)
    cnt = np.zeros((Hs, sum(nkb)), dtype=np.int32)
    for b in range(m.B):
        kb0 = sum(nkb[:b])
        sel = m.sparse[b, :, :nqb[b], :nkb[b]] != 0  # [Hs, qb, kb]
        for hs in range(Hs):
            for kb in range(nkb[b]):
                q = np.nonzero(sel[hs, :, kb])[0]
                idx[hs, kb0 + kb, :len(q)] = q
                cnt[hs, kb0 + kb] = len(q)
    c.sparse_kind, c.sparse, c.count = "kvidx", idx, cnt
    return c


@pytest.mark.timeout(600)
def test_kv_lists_long_context_equal_mask():
    """The long-context workload's block mask given instead as per-KV-block
    lists (layoutSparsePattern 7): the same index products and the same
    forward and backward outputs, bit for bit."""
    say("long-context workload as per-KV-block lists")
    m = _cfg_bwd(5)
    c = _kv_lists_of_mask(m)
    dm, dc = DeviceCase(m, with_bwd=True), DeviceCase(c, with_bwd=True)
    gm, gc = dm.index(True), dc.index(True)
    for k in ("row_ptr", "cols", "work", "col_ptr", "qrows", "work_kv"):
        assert np.array_equal(gm[k], gc[k]), k
    for d in (dm, dc):
        d.fwd()
        d.bwd()
    torch.cuda.synchronize()
    for nm in ("out", "lse", "dq", "dk", "dv"):
        a, b = getattr(dm, nm), getattr(dc, nm)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), nm


# --------------------------------------------------------------- atomic dQ --

ATOMIC = ["mask_f16_d64_ragged_empty_seq", "mask_gqa_shared_causal", "sabi_messy_causal_by256", "idx_perhead_gqa",
          "idx_paged_causal_gqa", "mask_bx16_causal", "sabi_bx512_by256_causal", "mask_d64_scale08",
          "mask_skv0_seq", "idx_band_paged", "mask_by64", "sabi_by48_gqa_paged_f16", "kvidx_messy_perhead_paged",
          "tile_idx_bx1_gqa_causal", "tile_kvidx_bx16_by256", "tile_none_bx1_sq_lt_skv", "tile_mask_bx16_skv0_seq"]


@pytest.mark.parametrize("name", ATOMIC + ["empty_rows"])
def test_bwd_small_atomic_dq(name):
    """dQ accumulated with fp32 atomics inside the dK/dV kernel
    (BSA_FLAG_DQ_ATOMIC): the same tolerances as the separate pass."""
    case = BWD[name] if name != "empty_rows" else empty_rows_case()
    say(f"bwd atomic dQ {name}")
    dc = DeviceCase(case, with_bwd=True, flags=bsa.BSA_FLAG_DQ_ATOMIC)
    dc.fwd()
    nan_fill(dc.dq, dc.dk, dc.dv)
    dc.bwd()
    torch.cuda.synchronize()
    check_bwd(case, dc, tag=name + " atomic")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n", [2, 5])
def test_bwd_config_atomic_dq(n):
    """The atomic dQ at full size: sampled q-blocks against the oracle, and
    dK / dV identical to the separate-pass call's (the flag changes only dQ)."""
    case = _cfg_bwd(n)
    say(f"config {n}: bwd with atomic dQ")
    da = DeviceCase(case, with_bwd=True, flags=bsa.BSA_FLAG_DQ_ATOMIC)
    db = DeviceCase(case, with_bwd=True)
    for d in (da, db):
        d.fwd()
        d.bwd()
    torch.cuda.synchronize()
    assert not torch.isnan(da.dq).any()
    assert torch.equal(da.dk.view(torch.int16), db.dk.view(torch.int16))
    assert torch.equal(da.dv.view(torch.int16), db.dv.view(torch.int16))
    idx = oracle.index_products(case, with_csc=False)
    rows = _sample_rows(case, idx, 12, 70 + n)
    rq, _, _ = oracle.backward(case, sample_rows=rows)
    dq = da.dq.float().cpu().numpy()
    selq = ~np.isnan(rq[..., 0])
    eq = rel_fro(dq[selq], rq[selq])
    eb = rel_fro(db.dq.float().cpu().numpy()[selq], rq[selq])
    say(f"  config{n}: atomic dQ rel_fro {eq:.3e} (separate pass {eb:.3e})")
    assert eq <= TOL_G[case.dtype]
