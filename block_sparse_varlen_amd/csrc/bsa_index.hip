// Block-index preprocessor: turns the per-q-block KV-block selection into the
// schedule the attention kernels walk.
//
//  * rows r = hs * totalQBlocks + qbase_b + qb (head-major over global q-blocks,
//    the order of GenericBlockSparseAttention's [N2, totalQBlocks, topK]
//    sparseBlockIdx tensor);
//  * CSR row_ptr/cols: per row the ascending local KV blocks that hold at least
//    one allowed (query, key) pair -- the selected set (block mask, 0xFFFF
//    padded sabi, or -1 padded idx with count; BlockSparseAttentionGrad README,
//    BlitzSparseAttention sabi section, GenericBlockSparseAttention parameter
//    table) de-duplicated, restricted to [0, nKB_b) and cut by the causal or
//    band mask;
//  * work: rows by visited count descending, ties by row id (longest first for
//    load balance, the role of GenericBlockSparseAttention's metadata
//    pre-operator);
//  * CSC col_ptr/qrows: per KV block the ascending q-blocks that visit it (the
//    per-KV-block layout of GenericBlockSparseAttention's layoutSparsePattern
//    table), and work_kv: dK/dV items by load, descending.
//  * Row tiles (SeqArgs.bx = 128 > sel_bx): the "q-blocks" above are tiles of
//    128 rows, each visiting the union of its selection q-blocks' visited
//    sets, and every CSR / CSC entry gets a 128-bit row mask of the rows whose
//    own q-block visits the entry's block (k_tile_masks, k_col_masks).
//
// Every product is deterministic: counts come from LDS bitmaps and atomics
// whose results do not depend on order, the scans are sequential per block,
// orders come from a stable LSD radix sort, and column lists are re-sorted
// through bitmaps after their order-dependent atomic fill.
#include <algorithm>

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ int seq_kv_len(const SeqArgs& s, int b) {
  if (s.seqused_kv) return s.seqused_kv[b];
  return (int)(s.cu_kv[b + 1] - s.cu_kv[b]);
}

// Block-wide inclusive scan of one int per thread (blockDim.x == 256 or 1024).
template <int NT>
__device__ int block_incl_scan(int x, int* wsum, int& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = wave_incl_scan(x);
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int v = wsum[i];
    if (i < w) off += v;
    tot += v;
  }
  __syncthreads();
  total = tot;
  return inc + off;
}

// ------------------------------------------------------------------ setup --
// One block: per-sequence lengths, q/kv block bases, block -> sequence maps,
// header.
// Blocks past the first clear the per-KV-block lists' bitmap (kv_n words).
__global__ __launch_bounds__(256) void k_setup(SeqArgs seq, IndexPtrs ip, int hs, int n2, uint32_t* kvbm,
                                               int64_t kv_n) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    for (int64_t i = (int64_t)(blockIdx.x - 1) * 256 + tid; i < kv_n; i += (int64_t)(gridDim.x - 1) * 256)
      kvbm[i] = 0u;
    return;
  }
  const int B = seq.batch;
  int carry_q = 0, carry_k = 0, carry_s = 0;
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    int nq = 0, nk = 0, ns = 0;
    if (b < B) {
      const int sq = (int)(seq.cu_q[b + 1] - seq.cu_q[b]);
      const int skv = seq_kv_len(seq, b);
      ip.sq[b] = sq;
      ip.skv[b] = skv;
      nq = cdiv(sq, seq.bx);
      nk = cdiv(skv, seq.by);
      ns = cdiv(sq, seq.sel_bx);
    }
    int tq, tk, ts;
    const int iq = block_incl_scan<256>(nq, wsum, tq);
    const int ik = block_incl_scan<256>(nk, wsum, tk);
    const int is = block_incl_scan<256>(ns, wsum, ts);
    if (b < B) {
      ip.qbase[b] = carry_q + iq - nq;
      ip.kbase[b] = carry_k + ik - nk;
      if (ip.qbase_sel) ip.qbase_sel[b] = carry_s + is - ns;
    }
    carry_q += tq;
    carry_k += tk;
    carry_s += ts;
  }
  if (tid == 0) {
    if (ip.qbase_sel) ip.qbase_sel[B] = carry_s;
    ip.qbase[B] = carry_q;
    ip.kbase[B] = carry_k;
    ip.hdr[H_TQB] = carry_q;
    ip.hdr[H_TKB] = carry_k;
    ip.hdr[H_R] = hs * carry_q;
    ip.hdr[H_C] = hs * carry_k;
    ip.hdr[H_NNZ] = 0;
    ip.hdr[H_KVITEMS] = n2 * carry_k;
    for (int i = H_KVITEMS + 1; i < H_COUNT; ++i) ip.hdr[i] = 0;
  }
  __syncthreads();
  for (int b = 0; b < B; ++b) {
    const int q0 = ip.qbase[b], q1 = ip.qbase[b + 1];
    for (int x = q0 + tid; x < q1; x += 256) ip.qb_seq[x] = b;
    const int k0 = ip.kbase[b], k1 = ip.kbase[b + 1];
    for (int x = k0 + tid; x < k1; x += 256) ip.kb_seq[x] = b;
  }
}

// ------------------------------------------------------- row visited sets --
// Key-block range of the rows of selection q-block m (sel_bx rows): blocks
// [kb_lo, nbits) hold keys inside some row's token window.  The rows'
// allowed key ranges slide up by one key per row, so their union is [first
// row's lower end, last row's upper end]; an empty window (win_lo > win_hi)
// leaves no key at all.
__device__ __forceinline__ void sel_block_range(const SeqArgs& seq, int m, int sq, int skv, int& kb_lo, int& nbits) {
  const int first_row = m * seq.sel_bx;
  const int last_row = min((m + 1) * seq.sel_bx, sq) - 1;
  int lim = skv - 1;
  int lo = 0;
  if (seq.masked) {
    lim = min(lim, last_row + skv - sq + seq.win_hi);
    lo = max(lo, first_row + skv - sq + seq.win_lo);
    if (seq.win_lo > seq.win_hi) lim = -1;
  }
  nbits = lim < lo ? 0 : lim / seq.by + 1;
  kb_lo = lim < lo ? 0 : lo / seq.by;
}

// Row tiles: calls visit(j, kb) for every KV block kb that selection q-block
// m0 + j (j < nm) of sequence b and sparse head hs selects inside its block
// range, the wave's lanes striding over (q-block, selection entry) pairs; a
// block may be visited more than once (duplicate entries).
template <class F>
__device__ void tile_members_visit(const SeqArgs& seq, const SelArgs& sel, const IndexPtrs& ip, int hs, int b, int m0,
                                   int nm, int sq, int skv, F visit) {
  const int lane = lane_id();
  const int qs0 = ip.qbase_sel[b];
  const int nkb_b = cdiv(skv, seq.by);
  const bool by_block = sel.kind == SP_NONE || kv_lists(sel.kind) || sel.kind == SP_MASK;
  const int per_m = sel.kind == SP_MASK ? min(sel.width, nkb_b) : by_block ? nkb_b : sel.width;
  const int total = nm * per_m;
  for (int x = lane; x < total; x += 64) {
    const int j = x / per_m, u = x - j * per_m;
    const int m = m0 + j;
    int kb_lo, nbits;
    sel_block_range(seq, m, sq, skv, kb_lo, nbits);
    int kb = -1;
    if (sel.kind == SP_NONE) {
      kb = u;
    } else if (kv_lists(sel.kind)) {
      const int64_t row = (int64_t)hs * ip.qbase_sel[seq.batch] + qs0 + m;
      if ((sel.kvbm[row * sel.kv_words + (u >> 5)] >> (u & 31)) & 1u) kb = u;
    } else if (sel.kind == SP_MASK || sel.kind == SP_SABI) {
      if (m < sel.rows) {
        const int64_t row = (((int64_t)b * sel.hs + hs) * sel.rows + m) * sel.width;
        if (sel.kind == SP_MASK) {
          if (reinterpret_cast<const uint8_t*>(sel.sparse)[row + u]) kb = u;
        } else {
          const int v = reinterpret_cast<const uint16_t*>(sel.sparse)[row + u];
          if (v != 0xFFFF) kb = v;
        }
      }
    } else {  // SP_IDX over global selection q-blocks, SP_IDX_B over local ones
      const bool in_rows = sel.kind == SP_IDX ? qs0 + m < sel.rows : m < sel.rows;
      if (in_rows) {
        const int64_t rr = sel.kind == SP_IDX ? (int64_t)hs * sel.rows + qs0 + m
                                              : ((int64_t)b * sel.hs + hs) * sel.rows + m;
        const int n = min(max(sel.count[rr], 0), sel.width);
        if (u < n) kb = reinterpret_cast<const int32_t*>(sel.sparse)[rr * sel.width + u];
      }
    }
    if (kb >= kb_lo && kb < nbits) visit(j, kb);
  }
}

// The tile of row r: sparse head, sequence, local tile, lengths and its
// selection q-blocks m0 .. m0 + nm - 1.
struct TileRow {
  int hs, b, t, sq, skv, m0, nm;
};
__device__ __forceinline__ TileRow tile_row(const SeqArgs& seq, const IndexPtrs& ip, int r, int TQB) {
  TileRow w;
  w.hs = r / TQB;
  const int qg = r - w.hs * TQB;
  w.b = ip.qb_seq[qg];
  w.t = qg - ip.qbase[w.b];
  w.sq = ip.sq[w.b];
  w.skv = ip.skv[w.b];
  const int per = seq.bx / seq.sel_bx;
  w.m0 = w.t * per;
  w.nm = min(per, cdiv(w.sq, seq.sel_bx) - w.m0);
  return w;
}

// Builds, in the calling wave's LDS words, the bitmap of row r's visited KV
// blocks and returns the number of bit positions in use (0 for r >= R).  All
// four waves of the block call it together (it contains block barriers).
__device__ int row_bitmap(uint32_t* bm, const SeqArgs& seq, const SelArgs& sel, const IndexPtrs& ip,
                          int r, int R, int TQB) {
  const int lane = lane_id();
  if (ip.qbase_sel) {  // row tiles: the union of the tile's selection q-blocks' visited sets
    TileRow w{};
    int nbits = 0;
    if (r < R) {
      w = tile_row(seq, ip, r, TQB);
      for (int j = lane; j < w.nm; j += 64) {
        int kb_lo, nb;
        sel_block_range(seq, w.m0 + j, w.sq, w.skv, kb_lo, nb);
        nbits = max(nbits, nb);
      }
      nbits = wave_max_i(nbits);
    }
    const int nwords = (nbits + 31) >> 5;
    for (int x = lane; x < nwords; x += 64) bm[x] = 0u;
    __syncthreads();
    if (nbits > 0)
      tile_members_visit(seq, sel, ip, w.hs, w.b, w.m0, w.nm, w.sq, w.skv,
                         [&](int, int kb) { atomicOr(&bm[kb >> 5], 1u << (kb & 31)); });
    __syncthreads();
    return nbits;
  }
  int nbits = 0, kb_lo = 0, b = 0, qb = 0, hs = 0, qg = 0;
  if (r < R) {
    hs = r / TQB;
    qg = r - hs * TQB;
    b = ip.qb_seq[qg];
    qb = qg - ip.qbase[b];
    const int sq = ip.sq[b], skv = ip.skv[b];
    const int first_row = qb * seq.bx;
    const int last_row = min((qb + 1) * seq.bx, sq) - 1;
    // The rows' allowed key ranges slide up by one key per row, so their
    // union is [first row's lower end, last row's upper end]; an empty
    // window (win_lo > win_hi) leaves no key at all.
    int lim = skv - 1;  // largest allowed key of the q-block's last row
    int lo = 0;         // smallest allowed key of its first row
    if (seq.masked) {
      lim = min(lim, last_row + skv - sq + seq.win_hi);
      lo = max(lo, first_row + skv - sq + seq.win_lo);
      if (seq.win_lo > seq.win_hi) lim = -1;
    }
    nbits = lim < lo ? 0 : lim / seq.by + 1;
    kb_lo = lim < lo ? 0 : lo / seq.by;
  }
  const int nwords = (nbits + 31) >> 5;
  for (int w = lane; w < nwords; w += 64) {
    uint32_t v = 0;
    if (sel.kind == SP_NONE || kv_lists(sel.kind)) {
      // the blocks [kb_lo, nbits) that hold allowed keys
      const int hi = nbits - w * 32;
      v = hi >= 32 ? 0xffffffffu : ((1u << hi) - 1u);
      const int lb = kb_lo - w * 32;
      if (lb >= 32)
        v = 0;
      else if (lb > 0)
        v &= ~((1u << lb) - 1u);
      // per-KV-block lists: the blocks whose lists name this row's q-block
      if (kv_lists(sel.kind)) v &= sel.kvbm[(int64_t)r * sel.kv_words + w];
    }
    bm[w] = v;
  }
  __syncthreads();
  if (nbits > 0 && sel.kind != SP_NONE && !kv_lists(sel.kind)) {
    if (sel.kind == SP_MASK || sel.kind == SP_SABI) {
      if (qb < sel.rows) {
        const int64_t row = (((int64_t)b * sel.hs + hs) * sel.rows + qb) * sel.width;
        if (sel.kind == SP_MASK) {
          const uint8_t* m = reinterpret_cast<const uint8_t*>(sel.sparse) + row;
          const int n = min(sel.width, nbits);
          for (int kb = kb_lo + lane; kb < n; kb += 64)
            if (m[kb]) atomicOr(&bm[kb >> 5], 1u << (kb & 31));
        } else {
          const uint16_t* s = reinterpret_cast<const uint16_t*>(sel.sparse) + row;
          for (int t = lane; t < sel.width; t += 64) {
            const int kb = s[t];
            if (kb != 0xFFFF && kb < nbits && kb >= kb_lo) atomicOr(&bm[kb >> 5], 1u << (kb & 31));
          }
        }
      }
    } else {  // SP_IDX over global q-blocks, SP_IDX_B over local ones
      const bool in_rows = sel.kind == SP_IDX ? qg < sel.rows : qb < sel.rows;
      if (in_rows) {
        const int64_t rr = sel.kind == SP_IDX ? (int64_t)hs * sel.rows + qg
                                              : ((int64_t)b * sel.hs + hs) * sel.rows + qb;
        const int n = min(max(sel.count[rr], 0), sel.width);
        const int32_t* ix = reinterpret_cast<const int32_t*>(sel.sparse) + rr * sel.width;
        for (int t = lane; t < n; t += 64) {
          const int kb = ix[t];
          if (kb >= kb_lo && kb < nbits) atomicOr(&bm[kb >> 5], 1u << (kb & 31));
        }
      }
    }
  }
  __syncthreads();
  return nbits;
}

// Per-KV-block lists (one wave per list): KV block kb of sequence b and
// sparse head hs sets bit kb in the bitmap of row (hs, b, qb) for every
// q-block qb among its list's first count entries that lies in [0, nQB_b).
// Atomic ORs give the same bits in any order.
__global__ __launch_bounds__(256) void k_kv_scatter(SeqArgs seq, SelArgs sel, IndexPtrs ip, int64_t nlists) {
  const int wv = threadIdx.x >> 6, lane = lane_id();
  const int64_t L = (int64_t)blockIdx.x * 4 + wv;
  if (L >= nlists) return;
  const int TQB = ip.hdr[H_TQB], TKB = ip.hdr[H_TKB];
  int b, hs, kb;
  if (sel.kind == SP_KV) {  // [Hs, rows = totalKBlocks, W]
    hs = (int)(L / sel.rows);
    const int gk = (int)(L - (int64_t)hs * sel.rows);
    if (gk >= TKB) return;
    b = ip.kb_seq[gk];
    kb = gk - ip.kbase[b];
  } else {  // [B, Hs, rows, W]
    kb = (int)(L % sel.rows);
    const int64_t bh = L / sel.rows;
    hs = (int)(bh % sel.hs);
    b = (int)(bh / sel.hs);
    if (kb >= cdiv(ip.skv[b], seq.by)) return;
  }
  // bitmap rows are the selection's q-blocks (sel_bx rows each)
  const int nqb = cdiv(ip.sq[b], seq.sel_bx);
  const int n = min(max(sel.count[L], 0), sel.width);
  const int32_t* lst = reinterpret_cast<const int32_t*>(sel.sparse) + L * sel.width;
  const int64_t row0 = ip.qbase_sel ? (int64_t)hs * ip.qbase_sel[seq.batch] + ip.qbase_sel[b]
                                    : (int64_t)hs * TQB + ip.qbase[b];
  for (int t = lane; t < n; t += 64) {
    const int qb = lst[t];
    if (qb >= 0 && qb < nqb) atomicOr(&sel.kvbm[(row0 + qb) * sel.kv_words + (kb >> 5)], 1u << (kb & 31));
  }
}

// Also clears the column counters of the transpose (zero_n entries of col_cnt
// and col_fill, 0 without it) with a grid-stride loop: the next launches
// count into them.
__global__ __launch_bounds__(256) void k_row_count(SeqArgs seq, SelArgs sel, IndexPtrs ip, int64_t rbar,
                                                   int words, int cmax, int64_t zero_n) {
  extern __shared__ uint32_t smem_bm[];
  const int wv = threadIdx.x >> 6, lane = lane_id();
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < zero_n; i += (int64_t)gridDim.x * 256) {
    ip.col_cnt[i] = 0;
    ip.col_fill[i] = 0;
  }
  uint32_t* bm = smem_bm + wv * words;
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  const int R = ip.hdr[H_R], TQB = ip.hdr[H_TQB];
  const int nbits = row_bitmap(bm, seq, sel, ip, r < rbar ? (int)r : R, R, TQB);
  int cnt = 0;
  for (int w = lane; w < ((nbits + 31) >> 5); w += 64) cnt += __popc(bm[w]);
  cnt = wave_sum_i(cnt);
  if (lane == 0 && r < rbar) {
    ip.row_cnt[r] = cnt;
    ip.key0[r] = r < R ? cmax - cnt : cmax + 1;
    ip.val0[r] = (int)r;
  }
}

// With count_cols, also counts each visited block into its column of the
// transpose (col_cnt, cleared by k_row_count).
__global__ __launch_bounds__(256) void k_row_fill(SeqArgs seq, SelArgs sel, IndexPtrs ip, int64_t rbar, int words,
                                                  int count_cols) {
  extern __shared__ uint32_t smem_bm[];
  const int wv = threadIdx.x >> 6, lane = lane_id();
  uint32_t* bm = smem_bm + wv * words;
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  const int R = ip.hdr[H_R], TQB = ip.hdr[H_TQB];
  const int nbits = row_bitmap(bm, seq, sel, ip, r < rbar ? (int)r : R, R, TQB);
  if (r >= R) return;
  int cbase = -1;  // column of KV block 0 of this row's sequence and head
  if (count_cols) {
    const int hs = (int)r / TQB;
    const int b = ip.qb_seq[(int)r - hs * TQB];
    cbase = hs * ip.hdr[H_TKB] + ip.kbase[b];
  }
  const int nwords = (nbits + 31) >> 5;
  int pos = ip.row_ptr[r];
  for (int c = 0; c < nwords; c += 64) {
    const int w = c + lane;
    uint32_t word = w < nwords ? bm[w] : 0u;
    const int pc = __popc(word);
    const int inc = wave_incl_scan(pc);
    int o = pos + inc - pc;
    while (word) {
      const int bit = __ffs(word) - 1;
      ip.cols[o++] = w * 32 + bit;
      if (cbase >= 0) atomicAdd(&ip.col_cnt[cbase + w * 32 + bit], 1);
      word &= word - 1;
    }
    pos += __shfl(inc, 63, 64);
  }
}

// ------------------------------------------------------------ row masks --
// Row tiles: the 128-bit row mask of every CSR entry of tile row r (one wave
// per row, LDS: the position of each KV block in the row's list, then the
// masks): the rows of each selection q-block of the tile are set in the masks
// of the blocks it visits.
__global__ __launch_bounds__(64) void k_tile_masks(SeqArgs seq, SelArgs sel, IndexPtrs ip, int64_t rbar,
                                                   int nkb_max) {
  extern __shared__ uint32_t smem_tm[];
  int* pos = reinterpret_cast<int*>(smem_tm);  // [nkb_max]
  uint32_t* msk = smem_tm + nkb_max;           // [nkb_max][4]
  const int lane = lane_id();
  const int64_t r = blockIdx.x;
  const int R = ip.hdr[H_R], TQB = ip.hdr[H_TQB];
  if (r >= R || r >= rbar) return;
  const TileRow w = tile_row(seq, ip, (int)r, TQB);
  const int e0 = ip.row_ptr[r], n = ip.row_ptr[r + 1] - e0;
  for (int e = lane; e < n; e += 64) {
    pos[ip.cols[e0 + e]] = e;
#pragma unroll
    for (int x = 0; x < 4; ++x) msk[4 * e + x] = 0u;
  }
  __syncthreads();
  // (every block a selection q-block visits is in the row's list: the list is
  // the union of exactly these visits)
  tile_members_visit(seq, sel, ip, w.hs, w.b, w.m0, w.nm, w.sq, w.skv, [&](int j, int kb) {
    const int row0 = j * seq.sel_bx;
    const uint32_t bits = seq.sel_bx >= 32 ? 0xffffffffu : ((1u << seq.sel_bx) - 1u) << (row0 & 31);
    atomicOr(&msk[4 * pos[kb] + (row0 >> 5)], bits);
  });
  __syncthreads();
  for (int x = lane; x < 4 * n; x += 64) ip.row_mask[(int64_t)e0 * 4 + x] = msk[x];
}

// Row tiles: each CSC entry takes the row mask of its (tile, block) CSR entry,
// found by binary search in the tile's ascending list (one wave per column).
__global__ __launch_bounds__(256) void k_col_masks(IndexPtrs ip, int64_t cbar) {
  const int wv = threadIdx.x >> 6, lane = lane_id();
  const int64_t c = (int64_t)blockIdx.x * 4 + wv;
  const int C = ip.hdr[H_C], TQB = ip.hdr[H_TQB], TKB = ip.hdr[H_TKB];
  if (c >= C || c >= cbar) return;
  const int hs = (int)(c / TKB), kg = (int)(c % TKB);
  const int b = ip.kb_seq[kg];
  const int kb = kg - ip.kbase[b];
  for (int o = ip.col_ptr[c] + lane; o < ip.col_ptr[c + 1]; o += 64) {
    const int r = hs * TQB + ip.qbase[b] + ip.qrows[o];
    int lo = ip.row_ptr[r], hi = ip.row_ptr[r + 1];  // cols[lo] <= kb < cols[hi] holds throughout
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ip.cols[mid] <= kb)
        lo = mid;
      else
        hi = mid;
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) ip.col_mask[(int64_t)o * 4 + x] = ip.row_mask[(int64_t)lo * 4 + x];
  }
}

// --------------------------------------------------------- exclusive scan --
// out[0..n) = exclusive prefix sums of in[0..n), out[n] = total; also copies
// the total to *total_out when given.  One block of 1024 threads; in and out
// may be the same array.
__device__ void scan_excl(const int32_t* in, int32_t* out, int64_t n, int32_t* total_out) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int64_t base = 0; base < n; base += 4096) {
    int v[4];
    int s = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = base + tid * 4 + e;
      v[e] = i < n ? in[i] : 0;
      s += v[e];
    }
    int tot;
    const int inc = block_incl_scan<1024>(s, wsum, tot);
    int run = carry + inc - s;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = base + tid * 4 + e;
      if (i < n) out[i] = run;
      run += v[e];
    }
    carry += tot;
  }
  if (tid == 0) {
    out[n] = carry;
    if (total_out) *total_out = carry;
  }
}

__global__ __launch_bounds__(1024) void k_scan_excl(const int32_t* in, int32_t* out, int64_t n, int32_t* total_out) {
  scan_excl(in, out, n, total_out);
}
// The same for two independent arrays in one launch.
__global__ __launch_bounds__(1024) void k_scan_excl2(int32_t* a, int64_t na, int32_t* b, int64_t nb) {
  scan_excl(a, a, na, nullptr);
  __syncthreads();
  scan_excl(b, b, nb, nullptr);
}

// ---------------------------------------------------- stable radix sort ----
// LSD radix sort on 8-bit digits of non-negative keys; each pass is stable,
// so equal keys keep their input (id) order.
__global__ __launch_bounds__(256) void k_radix_hist(const int32_t* key, int64_t n, int shift, int32_t* hist,
                                                    int nblocks) {
  __shared__ int h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 256 + tid;
  if (i < n) atomicAdd(&h[(key[i] >> shift) & 255], 1);
  __syncthreads();
  hist[(int64_t)tid * nblocks + blockIdx.x] = h[tid];
}

__global__ __launch_bounds__(256) void k_radix_scatter(const int32_t* key_in, const int32_t* val_in, int64_t n,
                                                       int shift, const int32_t* hist_scan, int nblocks,
                                                       int32_t* key_out, int32_t* val_out) {
  __shared__ int cnt[4][256];
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  for (int e = tid; e < 1024; e += 256) cnt[e >> 8][e & 255] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 256 + tid;
  const bool valid = i < n;
  int key = 0, val = 0, d = 0;
  if (valid) {
    key = key_in[i];
    val = val_in[i];
    d = (key >> shift) & 255;
  }
  uint64_t eq = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const uint64_t m = __ballot((d >> bit) & 1);
    eq &= ((d >> bit) & 1) ? m : ~m;
  }
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  const int rank_w = __popcll(eq & lt);
  const bool leader = valid && ((eq >> lane) == 1ull);
  if (leader) cnt[wv][d] = __popcll(eq);
  __syncthreads();
  if (valid) {
    int r = rank_w;
    for (int w = 0; w < wv; ++w) r += cnt[w][d];
    const int dst = hist_scan[(int64_t)d * nblocks + blockIdx.x] + r;
    if (key_out) key_out[dst] = key;
    val_out[dst] = val;
  }
}

// Both single-pass sorts of the index (rows, dK/dV items) in one launch per
// step: blocks [0, nba) take sort A, the rest sort B.
struct SortSeg {
  const int32_t* key;
  const int32_t* val;
  int64_t n;
  int32_t* hist;  // [256 * nb + 1]
  int nb;
  int32_t* dst;
};

__global__ __launch_bounds__(256) void k_radix_hist2(SortSeg a, SortSeg b) {
  const bool in_a = (int)blockIdx.x < a.nb;
  const SortSeg& g = in_a ? a : b;
  const int blk = in_a ? (int)blockIdx.x : (int)blockIdx.x - a.nb;
  __shared__ int h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blk * 256 + tid;
  if (i < g.n) atomicAdd(&h[g.key[i] & 255], 1);
  __syncthreads();
  g.hist[(int64_t)tid * g.nb + blk] = h[tid];
}

__global__ __launch_bounds__(256) void k_radix_scatter2(SortSeg a, SortSeg b) {
  const bool in_a = (int)blockIdx.x < a.nb;
  const SortSeg& g = in_a ? a : b;
  const int blk = in_a ? (int)blockIdx.x : (int)blockIdx.x - a.nb;
  __shared__ int cnt[4][256];
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  for (int e = tid; e < 1024; e += 256) cnt[e >> 8][e & 255] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blk * 256 + tid;
  const bool valid = i < g.n;
  int val = 0, d = 0;
  if (valid) {
    val = g.val[i];
    d = g.key[i] & 255;
  }
  uint64_t eq = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const uint64_t m = __ballot((d >> bit) & 1);
    eq &= ((d >> bit) & 1) ? m : ~m;
  }
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  const int rank_w = __popcll(eq & lt);
  const bool leader = valid && ((eq >> lane) == 1ull);
  if (leader) cnt[wv][d] = __popcll(eq);
  __syncthreads();
  if (valid) {
    int r = rank_w;
    for (int w = 0; w < wv; ++w) r += cnt[w][d];
    g.dst[g.hist[(int64_t)d * g.nb + blk] + r] = val;
  }
}

// ------------------------------------------------------------- transpose --
__device__ __forceinline__ void row_coords(const IndexPtrs& ip, int r, int TQB, int& hs, int& b, int& qb) {
  hs = r / TQB;
  const int qg = r - hs * TQB;
  b = ip.qb_seq[qg];
  qb = qg - ip.qbase[b];
}

__global__ __launch_bounds__(256) void k_col_fill(IndexPtrs ip, int64_t rbar) {
  const int wv = threadIdx.x >> 6, lane = lane_id();
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  const int R = ip.hdr[H_R], TQB = ip.hdr[H_TQB], TKB = ip.hdr[H_TKB];
  if (r >= R || r >= rbar) return;
  int hs, b, qb;
  row_coords(ip, (int)r, TQB, hs, b, qb);
  const int base = hs * TKB + ip.kbase[b];
  for (int e = ip.row_ptr[r] + lane; e < ip.row_ptr[r + 1]; e += 64) {
    const int c = base + ip.cols[e];
    const int slot = atomicAdd(&ip.col_fill[c], 1);
    ip.qrows[ip.col_ptr[c] + slot] = qb;
  }
}

// Puts each column's q-block list in ascending order (one wave per column).
// With kv_key set (one sparse head per KV head, so dK/dV item i is column i),
// also writes the items' sort keys: kvkey_max - load, kvkey_max + 1 past the
// last item.
__global__ __launch_bounds__(256) void k_col_sort(IndexPtrs ip, int64_t cbar, int words, int bx, int32_t* kv_key,
                                                  int32_t* kv_val, int kvkey_max) {
  extern __shared__ uint32_t smem_bm[];
  const int wv = threadIdx.x >> 6, lane = lane_id();
  uint32_t* bm = smem_bm + wv * words;
  const int64_t c = (int64_t)blockIdx.x * 4 + wv;
  const int C = ip.hdr[H_C], TKB = ip.hdr[H_TKB];
  int nqb = 0, p0 = 0, p1 = 0;
  if (c < C && c < cbar) {
    const int kg = (int)(c % TKB);
    const int b = ip.kb_seq[kg];
    nqb = cdiv(ip.sq[b], bx);
    p0 = ip.col_ptr[c];
    p1 = ip.col_ptr[c + 1];
  }
  if (kv_key && c < cbar && lane == 0) {
    kv_key[c] = c < C ? kvkey_max - (p1 - p0) : kvkey_max + 1;
    kv_val[c] = (int)c;
  }
  const int nwords = (nqb + 31) >> 5;
  for (int w = lane; w < nwords; w += 64) bm[w] = 0;
  __syncthreads();
  for (int e = p0 + lane; e < p1; e += 64) {
    const int qb = ip.qrows[e];
    atomicOr(&bm[qb >> 5], 1u << (qb & 31));
  }
  __syncthreads();
  int pos = p0;
  for (int cc = 0; cc < nwords; cc += 64) {
    const int w = cc + lane;
    uint32_t word = w < nwords ? bm[w] : 0u;
    const int pc = __popc(word);
    const int inc = wave_incl_scan(pc);
    int o = pos + inc - pc;
    while (word) {
      const int bit = __ffs(word) - 1;
      ip.qrows[o++] = w * 32 + bit;
      word &= word - 1;
    }
    pos += __shfl(inc, 63, 64);
  }
}

// Sort keys of the dK/dV items: item i = g * TKB + kg, load = number of
// (sparse head of group g, q-block) pairs that reach KV block kg.
__global__ __launch_bounds__(256) void k_kv_keys(IndexPtrs ip, int64_t kvbar, int hs_total, int n2, int group,
                                                 int kvkey_max, int32_t* kv_key, int32_t* kv_val) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= kvbar) return;
  const int TKB = ip.hdr[H_TKB];
  const int items = n2 * TKB;
  int key = kvkey_max + 1;
  if (i < items) {
    const int g = (int)(i / TKB), kg = (int)(i % TKB);
    int load = 0;
    if (hs_total == n2) {
      load = ip.col_cnt[g * TKB + kg];
    } else {
      for (int h = g * group; h < (g + 1) * group; ++h) load += ip.col_cnt[h * TKB + kg];
    }
    key = kvkey_max - load;
  }
  kv_key[i] = key;
  kv_val[i] = (int)i;
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

int radix_passes(int64_t maxkey) {
  int bits = 0;
  while ((maxkey >> bits) != 0) ++bits;
  return bits <= 8 ? 1 : (bits + 7) / 8;
}

// Sorts (key, val)[0..n) (key1 / val1 hold the intermediate passes) and
// writes the values in key order to `dst`.
hipError_t radix_sort(const IndexPtrs& ip, const int32_t* key, const int32_t* val, int64_t n, int64_t maxkey,
                      int32_t* dst, hipStream_t st) {
  const int nb = (int)blocks_for(n, 256);
  const int passes = radix_passes(maxkey);
  const int32_t *ki = key, *vi = val;
  int32_t *ko = ip.key1, *vo = ip.val1;
  int32_t *ko2 = ip.key0, *vo2 = ip.val0;
  for (int p = 0; p < passes; ++p) {
    const bool last = p == passes - 1;
    k_radix_hist<<<nb, 256, 0, st>>>(ki, n, 8 * p, ip.hist, nb);
    k_scan_excl<<<1, 1024, 0, st>>>(ip.hist, ip.hist, (int64_t)nb * 256, nullptr);
    k_radix_scatter<<<nb, 256, 0, st>>>(ki, vi, n, 8 * p, ip.hist, nb, last ? nullptr : ko, last ? dst : vo);
    ki = ko;
    vi = vo;
    int32_t* t = ko; ko = ko2; ko2 = t;
    t = vo; vo = vo2; vo2 = t;
  }
  return hipGetLastError();
}


// Value check of BSA_FLAG_CHECK_VALUES: one workgroup walks the sequences
// (and, paged, every block_table entry that a pass would read) and writes the
// CHK_* bits of the failed checks to hdr[H_CHECK].  Every array is read only
// inside the extent the descriptor gives it, whatever the values: a page
// count taken from seqused_kv is clamped to [0, max_pages] first.
__global__ __launch_bounds__(1024) void k_check_values(CheckArgs c, int32_t* hdr) {
  __shared__ uint32_t bits;
  if (threadIdx.x == 0) bits = 0u;
  __syncthreads();
  uint32_t m = 0u;
  if (threadIdx.x == 0) {
    if (c.cu_q[0] != 0 || c.cu_q[c.batch] != c.total_q) m |= CHK_CU_Q_ENDS;
    if (c.cu_kv && (c.cu_kv[0] != 0 || c.cu_kv[c.batch] > c.total_kv)) m |= CHK_CU_KV_ENDS;
  }
  for (int b = threadIdx.x; b < c.batch; b += blockDim.x) {
    const int64_t sq = c.cu_q[b + 1] - c.cu_q[b];
    if (sq < 0) m |= CHK_CU_Q_ORDER;
    else if (sq > c.max_sq) m |= CHK_SQ_LONG;
    if (c.cu_kv) {
      const int64_t skv = c.cu_kv[b + 1] - c.cu_kv[b];
      if (skv < 0) m |= CHK_CU_KV_ORDER;
      else if (skv > c.max_skv) m |= CHK_SKV_LONG;
    } else {
      const int32_t used = c.seqused_kv[b];
      if (used < 0 || used > c.max_skv) m |= CHK_SKV_LONG;
    }
  }
  if (c.block_table) {
    const int64_t n = (int64_t)c.batch * c.max_pages;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
      const int b = (int)(i / c.max_pages), pg = (int)(i - (int64_t)b * c.max_pages);
      const int64_t cap = (int64_t)c.max_pages * c.page_size;
      const int64_t used = c.seqused_kv[b] < 0 ? 0 : (c.seqused_kv[b] > cap ? cap : (int64_t)c.seqused_kv[b]);
      if (pg < (used + c.page_size - 1) / c.page_size) {
        const int32_t id = c.block_table[i];
        if (id < 0 || id >= c.total_kv) m |= CHK_PAGE;
      }
    }
  }
  if (m) atomicOr(&bits, m);
  __syncthreads();
  if (threadIdx.x == 0) hdr[H_CHECK] = (int32_t)bits;
}

}  // namespace

namespace {

// Sort keys of the chunked dispatch order: work entry i gets the head chunk
// of its row (rows past the last one sort last), so a stable sort groups the
// longest-first order by chunk.
__global__ __launch_bounds__(256) void k_chunk_keys(IndexPtrs ip, int64_t rbar, int chunk, int nchunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rbar) return;
  const int R = ip.hdr[H_R], TQB = ip.hdr[H_TQB];
  const int r = ip.work[i];
  ip.key0[i] = i < R ? (r / TQB) / chunk : nchunks;
  ip.val0[i] = r;
}

// Launches: setup, row counts (+ clearing the column counters), row scan,
// row fill (+ column counts), then either both work lists at the end with one
// shared hist / scan / scatter launch each (when both sort in one radix pass)
// or each list with its own passes.
hipError_t index_lists(const SeqArgs& seq, const SelArgs& sel, const Bounds& bd, const IndexPtrs& ip, int n2,
                       int group, bool with_csc, hipStream_t st) {
  const bool merged = with_csc && radix_passes((int64_t)bd.cmax + 1) == 1 &&
                      radix_passes((int64_t)bd.kvkey_max + 1) == 1;
  const bool kv = kv_lists(sel.kind);
  const int64_t kv_n = kv ? (int64_t)sel.hs * bd.qbar_sel * sel.kv_words : 0;
  const unsigned clear_blocks = kv ? (unsigned)std::min<int64_t>(blocks_for(kv_n, 256), 1024) : 0;
  k_setup<<<1 + clear_blocks, 256, 0, st>>>(seq, ip, sel.hs, n2, sel.kvbm, kv_n);
  if (kv) {
    const int64_t nlists = (int64_t)sel.hs * sel.rows * (sel.kind == SP_KV_B ? seq.batch : 1);
    if (nlists > 0) k_kv_scatter<<<blocks_for(nlists, 4), 256, 0, st>>>(seq, sel, ip, nlists);
  }
  const int words = (bd.nkb_max + 31) / 32 > 0 ? (bd.nkb_max + 31) / 32 : 1;
  const size_t lds = 4 * (size_t)words * 4;
  const unsigned rgrid = blocks_for(bd.rbar, 4);
  k_row_count<<<rgrid, 256, lds, st>>>(seq, sel, ip, bd.rbar, words, bd.cmax, with_csc ? bd.cbar : 0);
  k_scan_excl<<<1, 1024, 0, st>>>(ip.row_cnt, ip.row_ptr, bd.rbar, ip.hdr + H_NNZ);
  k_row_fill<<<rgrid, 256, lds, st>>>(seq, sel, ip, bd.rbar, words, with_csc ? 1 : 0);
  if (ip.row_mask) {
    const int nkb = std::max(bd.nkb_max, 1);
    k_tile_masks<<<(unsigned)bd.rbar, 64, (size_t)nkb * 20, st>>>(seq, sel, ip, bd.rbar, nkb);
  }
  hipError_t e = hipSuccess;
  if (!merged) {
    e = radix_sort(ip, ip.key0, ip.val0, bd.rbar, (int64_t)bd.cmax + 1, ip.work, st);
    if (e != hipSuccess || !with_csc) return e;
  }
  // dK/dV item keys: key1 / val1 when merged (key0 / val0 still hold the row
  // keys), else key0 / val0 (the row sort is done)
  int32_t* kv_key = merged ? ip.key1 : ip.key0;
  int32_t* kv_val = merged ? ip.val1 : ip.val0;
  const bool direct = sel.hs == n2;
  k_scan_excl<<<1, 1024, 0, st>>>(ip.col_cnt, ip.col_ptr, bd.cbar, nullptr);
  k_col_fill<<<rgrid, 256, 0, st>>>(ip, bd.rbar);
  const int qwords = (bd.nqb_max + 31) / 32 > 0 ? (bd.nqb_max + 31) / 32 : 1;
  k_col_sort<<<blocks_for(bd.cbar, 4), 256, 4 * (size_t)qwords * 4, st>>>(
      ip, bd.cbar, qwords, seq.bx, direct ? kv_key : nullptr, kv_val, bd.kvkey_max);
  if (!direct)
    k_kv_keys<<<blocks_for(bd.kvbar, 256), 256, 0, st>>>(ip, bd.kvbar, sel.hs, n2, group, bd.kvkey_max, kv_key,
                                                         kv_val);
  if (ip.col_mask) k_col_masks<<<blocks_for(bd.cbar, 4), 256, 0, st>>>(ip, bd.cbar);
  if (!merged) return radix_sort(ip, kv_key, kv_val, bd.kvbar, (int64_t)bd.kvkey_max + 1, ip.work_kv, st);
  const int nba = (int)blocks_for(bd.rbar, 256), nbb = (int)blocks_for(bd.kvbar, 256);
  const SortSeg sa{ip.key0, ip.val0, bd.rbar, ip.hist, nba, ip.work};
  const SortSeg sb{ip.key1, ip.val1, bd.kvbar, ip.hist + 256 * (int64_t)nba + 1, nbb, ip.work_kv};
  k_radix_hist2<<<nba + nbb, 256, 0, st>>>(sa, sb);
  k_scan_excl2<<<1, 1024, 0, st>>>(sa.hist, 256 * (int64_t)nba, sb.hist, 256 * (int64_t)nbb);
  k_radix_scatter2<<<nba + nbb, 256, 0, st>>>(sa, sb);
  return hipGetLastError();
}

}  // namespace

// The block index, then, when the Q-major passes run in head chunks, their
// dispatch order work_q: work stably sorted by head chunk (key0 / val0 and
// the sort scratch are free once the lists are built).
hipError_t launch_index(const SeqArgs& seq, const SelArgs& sel, const Bounds& bd, const IndexPtrs& ip, int n2,
                        int group, bool with_csc, hipStream_t st) {
  hipError_t e = index_lists(seq, sel, bd, ip, n2, group, with_csc, st);
  if (e != hipSuccess || bd.q_chunk_heads >= sel.hs) return e;
  const int nchunks = (sel.hs + bd.q_chunk_heads - 1) / bd.q_chunk_heads;
  k_chunk_keys<<<blocks_for(bd.rbar, 256), 256, 0, st>>>(ip, bd.rbar, bd.q_chunk_heads, nchunks);
  return radix_sort(ip, ip.key0, ip.val0, bd.rbar, nchunks, ip.work_q, st);
}

hipError_t launch_check_values(const CheckArgs& c, int32_t* hdr, hipStream_t st) {
  k_check_values<<<1, 1024, 0, st>>>(c, hdr);
  return hipGetLastError();
}

}  // namespace bsa
