// Pieces shared by the forward and backward attention kernels: work-item
// decoding, key-tile staging (global -> registers -> LDS) and the walk over a
// row's selected KV blocks in 64-key sub-tiles.
#pragma once

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

constexpr int KT = 64;   // keys per sub-tile of the Q-major kernels
constexpr int QT = 128;  // query rows per Q-major work item (4 waves x 32)

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  xcd_item maps dispatch index `bid` to a work item so that every XCD
// takes runs of 2^seg consecutive items from the longest-first order --
// neighbouring q-blocks (or KV blocks) of one head, which share most of the
// tiles they read -- while the order across XCDs stays longest-first at a
// granularity of 8 * 2^seg items.  Grids are padded to a multiple of
// 8 * 2^seg; items past the end exit.
__device__ __forceinline__ int64_t xcd_item(int64_t bid, int seg) {
  const int64_t x = bid % NUM_XCD, k = bid / NUM_XCD;
  return (((k >> seg) * NUM_XCD + x) << seg) + (k & ((1 << seg) - 1));
}

// A Q-major work item: a slice of at most 128 rows of one q-block of one
// q-head (block_x is a multiple of 64: ceil(block_x / 128) slices).
struct QItem {
  int r;        // CSR row
  int h, g;     // q-head, kv-head
  int b, qb;    // sequence, local q-block
  int64_t q0;   // first token row of sequence b
  int sq, skv;  // lengths
  int row_lo;   // first local query row of the item
  int nrows;    // valid query rows in the item
};

// item = (slot * heads_per_row + j) * slices + slice; slot indexes the
// longest-first row order.  Returns false past the last item and for a slice
// that starts past the sequence end (nothing to do).
__device__ __forceinline__ bool decode_qitem(int64_t item, const int32_t* hdr, const int32_t* work,
                                             const int32_t* qb_seq, const int32_t* qbase, const SeqArgs& seq,
                                             int heads_per_row, int group, QItem& it) {
  const int R = ldu(hdr, H_R);
  const int slices = (seq.bx + QT - 1) / QT;
  if (item >= (int64_t)R * heads_per_row * slices) return false;
  const int64_t ritem = item / slices;
  const int slice = (int)(item - ritem * slices);
  const int slot = (int)(ritem / heads_per_row);
  const int jh = (int)(ritem - (int64_t)slot * heads_per_row);
  it.r = ldu(work, slot);
  const int TQB = ldu(hdr, H_TQB);
  const int hs = it.r / TQB;
  const int qg = it.r - hs * TQB;
  it.h = heads_per_row == 1 ? hs : hs * group + jh;
  it.g = it.h / group;
  it.b = ldu(qb_seq, qg);
  it.qb = qg - ldu(qbase, it.b);
  it.q0 = ldu(seq.cu_q, it.b);
  it.sq = (int)(ldu(seq.cu_q, it.b + 1) - it.q0);
  it.skv = seq.seqused_kv ? ldu(seq.seqused_kv, it.b) : (int)(ldu(seq.cu_kv, it.b + 1) - ldu(seq.cu_kv, it.b));
  it.row_lo = it.qb * seq.bx + slice * QT;
  it.nrows = min(min(QT, seq.bx - slice * QT), it.sq - it.row_lo);
  return it.nrows > 0;
}

// s_waitcnt on the vector-memory counter only: wait until at most N of this
// wave's vector memory operations (loads, and loads into LDS) are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | (N & 0xF) | ((N >> 4) << 14));
}

// LDS byte address of a pointer into __shared__ memory, and a 64-bit value
// made wave-uniform (readfirstlane returns int: each half is taken as
// unsigned before widening).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

// One wave-wide global -> LDS copy: lane l fetches SIZE (4 or 16) bytes from
// sbase + voff (sbase the wave-uniform global byte address, voff the lane's
// byte offset) and they land at LDS byte m0 + SIZE l.  Issued as inline asm
// on purpose: when the compiler sees a load that writes LDS it treats it as
// an access to two memory kinds whose completion order it cannot track, and
// from then on waits for every outstanding vector-memory and LDS operation
// (vmcnt(0) / lgkmcnt(0)) before any LDS read -- which would drain the next
// stage's prefetch in the middle of the current stage.  The kernels
// synchronise these copies themselves: wait_vmcnt for the issuing wave, then
// a workgroup barrier before any wave reads the stage.  M0 holds the LDS base
// (no other code in these kernels uses M0); one wait state separates its
// write from the copy.
template <int SIZE>
__device__ __forceinline__ void dma_raw(uint64_t sbase, uint32_t voff, uint32_t m0) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (SIZE == 16) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
                 : "memory", "m0");
  } else {
    static_assert(SIZE == 4, "4- or 16-byte copies");
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
                 : "memory", "m0");
  }
#pragma clang diagnostic pop
}

template <int SIZE>
__device__ __forceinline__ void dma_to_lds(const void* gbase, uint32_t off, const void* lds) {
  dma_raw<SIZE>(uniform_u64((uint64_t)(uintptr_t)gbase), off, __builtin_amdgcn_readfirstlane(lds_addr(lds)));
}

// Direct global -> LDS staging (global_load_lds_dwordx4) of a ROWS x D tile
// with layout L, rows row_stride elements apart in global memory.  Lane l of
// a wave instruction writes LDS bytes base + 16 l (checked on the hardware),
// so instruction i fills 16-byte slots 64 i .. 64 i + 63 of the tile; each
// lane fetches the global chunk that the layout puts in its slot (pad slots
// fetch a harmless chunk).  The tile's NINST instructions are spread over the
// 4 waves, PER_WAVE each.  The lanes' byte offsets of a full tile are fixed
// for a work item and kept in registers, so a copy costs no vector ALU work;
// in a partial tile (rows at or past `nvalid`, the last tile of a sequence)
// those rows are fetched from row nvalid - 1 (finite data the kernel then
// masks), so no lane reads outside the tensor.
template <class L, int D, int ROWS>
struct DmaTile {
  static constexpr int SPR = L::ROW_BYTES / 16;  // 16-byte slots per row
  static constexpr int NINST = ROWS * SPR / 64;
  static constexpr int PER_WAVE = NINST / 4;
  static_assert((ROWS * SPR) % 64 == 0 && NINST % 4 == 0, "tile must split evenly over 4 waves");
  int wv, stride;
  uint32_t voff[PER_WAVE];
  __device__ __forceinline__ void slot(int j, int& r, int& c) const {
    const int sl = 64 * (wv + 4 * j) + lane_id();
    r = sl / SPR;
    const int cc = sl % SPR;
    int chunk;
    if constexpr (L::LINEAR) {
      chunk = cc < L::CH ? cc : 0;
    } else {
      chunk = cc ^ L::swz(r);
    }
    c = 8 * chunk;
  }
  // the copying waves are waves 0..3 of the workgroup, or of a 4-wave group of it
  __device__ __forceinline__ void init(int row_stride) {
    wv = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3);
    stride = row_stride;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      int r, c;
      slot(j, r, c);
      voff[j] = 2u * (uint32_t)(r * stride + c);
    }
  }
  // gbase: element pointer of tile row 0, column 0 (wave-uniform)
  __device__ __forceinline__ void issue(char* lds_tile, const uint16_t* gbase, int nvalid) const {
    const uint64_t sb = uniform_u64((uint64_t)(uintptr_t)gbase);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_tile)) + 1024u * wv;
    if (nvalid >= ROWS) {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) dma_raw<16>(sb, voff[j], m0 + 4096u * j);
    } else {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        int r, c;
        slot(j, r, c);
        dma_raw<16>(sb, 2u * (uint32_t)(min(r, nvalid - 1) * stride + c), m0 + 4096u * j);
      }
    }
  }
};

// The same direct staging for an XorTile<D> of ROWS rows by a workgroup of NW
// waves.  Wave w's instruction j fills slots 64 (w + NW j) .. + 63, i.e. rows
// r0 + RSTEP j of the lane; the XOR pattern repeats every PERIOD instructions,
// so a full tile needs PERIOD lane offsets, the rest of instruction j's
// offset (RSTEP j rows) being added to the wave-uniform base.
template <int D, int ROWS, int NW>
struct DmaXor {
  using L = XorTile<D>;
  static constexpr int SPR = D / 8;
  static constexpr int NINST = ROWS * SPR / 64;
  static constexpr int PER_WAVE = NINST / NW;
  static constexpr int RSTEP = 64 * NW / SPR;
  static constexpr int PERIOD = RSTEP % 16 == 0 ? 1 : RSTEP % 8 == 0 ? 2 : RSTEP % 4 == 0 ? 4 : 16;
  static_assert(64 % SPR == 0 && NINST % NW == 0, "tile must split evenly over the waves");
  int wv, stride;
  uint32_t vb[PERIOD];
  __device__ __forceinline__ int r0() const { return 64 * wv / SPR + lane_id() / SPR; }
  __device__ __forceinline__ int col(int p) const { return 8 * ((lane_id() % SPR) ^ L::swz(r0() + RSTEP * p)); }
  // the copying waves are waves 0 .. NW-1 of the workgroup, or of an NW-wave group of it
  __device__ __forceinline__ void init(int row_stride) {
    wv = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) % NW);
    stride = row_stride;
#pragma unroll
    for (int p = 0; p < PERIOD; ++p) vb[p] = 2u * (uint32_t)(r0() * stride + col(p));
  }
  // instructions J0 .. J1 - 1 of this wave's share (all by default)
  template <int J0 = 0, int J1 = PER_WAVE>
  __device__ __forceinline__ void issue(char* lds_tile, const uint16_t* gbase, int nvalid) const {
    const uint64_t sb = uniform_u64((uint64_t)(uintptr_t)gbase);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_tile)) + 1024u * wv;
    if (nvalid >= ROWS) {
#pragma unroll
      for (int j = J0; j < J1; ++j)
        dma_raw<16>(sb + 2ull * RSTEP * j * (uint64_t)stride, vb[j % PERIOD], m0 + 1024u * NW * j);
    } else {
#pragma unroll
      for (int j = J0; j < J1; ++j) {
        const int r = min(r0() + RSTEP * j, nvalid - 1);
        dma_raw<16>(sb, 2u * (uint32_t)(r * stride + col(j % PERIOD)), m0 + 1024u * NW * j);
      }
    }
  }
};

// Waits for every scalar (and LDS) load in flight and keeps the scheduler from
// moving loads across this point.  Called after a loop's index-list reads so
// that no scalar load -- whose results may return out of order and would force
// full LDS waits -- is outstanding while the MFMA pipeline streams LDS reads.
__device__ __forceinline__ void settle_scalar_loads() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt unconstrained
  __builtin_amdgcn_sched_barrier(0);
}

// The lane index computed on the spot (v_mbcnt), in an asm the compiler may
// not hoist: inside a loop that runs at the register limit, a lane index kept
// live across the loop gets spilled, and the wait for its reload would also
// wait for the tile copies issued just before.
__device__ __forceinline__ int lane_id_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// One fp32 per row of a 64-row tile, loaded by one wave into LDS (lane l ->
// bytes 4 l); rows at or past nvalid repeat row nvalid - 1.
__device__ __forceinline__ void dma_rows_f32(float* lds, const float* g, int stride, int nvalid) {
  const int r = min(lane_id_here(), nvalid - 1);
  dma_to_lds<4>(g, 4u * (uint32_t)(r * stride), lds);
}

// Walk over the T-key sub-tiles of a CSR row: blocks cols[e0..e1), keeping
// sub-tiles whose first key is below `kend` (the key bound of the item: Skv,
// or its last row's window end + 1) and that end above `kstart` (its first
// row's window start).  The row's block list is held in a VGPR (lane l holds
// entry base + l), so handing out a sub-tile is a lane read instead of a
// scalar memory round trip on the critical path of the tile copies.  Rows of
// more than 64 entries reload the register per 64 entries and wait for that
// load on the spot (rare), which leaves the compiler no pending load of it to
// wait for elsewhere -- such a wait would also drain the tile copies in
// flight.
//
// When block_y is a multiple of T each block is cut into block_y / T
// sub-tiles.  Otherwise (block_y a multiple of 16) the walk hands out the
// T-aligned windows of keys that meet a selected block, each window once,
// with `gmask` naming its 16-key groups that lie in selected blocks (bit g:
// keys 16 g .. 16 g + 15 of the window); the kernels mask the other groups.
// Several small blocks then share one window's MFMAs, and a window never
// crosses a T-aligned page boundary.
template <int T = KT>
struct RegTileWalk {
  static constexpr uint32_t FULL = (1u << (T / 16)) - 1u;
  const int32_t* cols;
  int e, e1, base, s, nsub, by, kend;
  bool grouped;
  int wk;          // grouped: first key of the next window
  uint32_t gmask;  // 16-key groups of the last sub-tile handed out that are selected
  int ent;         // not grouped: the list entry (CSR position) of the last sub-tile handed out
  int colv;
  // The caller waits for the initial load (any vmcnt wait covering it) before
  // the first take<false>(); take<true>() reads its entries with scalar loads
  // instead, for a first sub-tile issued before that wait.
  __device__ __forceinline__ void init(const int32_t* c, int e0, int e_end, int by_, int kend_, int kstart = 0) {
    cols = c;
    e1 = e_end;
    // the list is ascending: drop trailing blocks that start at or past kend
    // (only a slice of a q-block taller than 128 rows can end before the
    // q-block's window end, so this loop rarely runs)
    while (e1 > e0 && ldu(c, e1 - 1) * by_ >= kend_) --e1;
    // and leading blocks that end below kstart (band masks only)
    while (e0 < e1 && (ldu(c, e0) + 1) * by_ <= kstart) ++e0;
    e = e0;
    base = e0;
    s = 0;
    by = by_;
    nsub = by_ / T;
    kend = kend_;
    grouped = by_ % T != 0;
    gmask = FULL;
    wk = 0;
    if (e0 < e1) {
      const int k0 = max(kstart, ldu(c, e0) * by_);
      if (grouped) {
        wk = k0 & ~(T - 1);
        if (wk >= kend_) e = e1;
      } else if (kstart > 0) {
        s = (k0 - ldu(c, e0) * by_) / T;  // first sub-tile of the first block that reaches kstart
      }
    }
    colv = e0 + lane_id() < e_end ? c[e0 + lane_id()] : 0;
  }
  __device__ __forceinline__ bool valid() const { return e < e1; }
  template <bool SCALAR>
  __device__ __forceinline__ int entry(int ee) {
    if constexpr (SCALAR) {
      return ldu(cols, ee);
    } else {
      if (__builtin_expect(ee - base >= 64, 0)) {
        base += 64;
        colv = base + lane_id() < e1 ? cols[base + lane_id()] : 0;
        wait_vmcnt<0>();
        pin(colv);
      }
      return __builtin_amdgcn_readlane(colv, ee - base);
    }
  }
  // first key of the current sub-tile (and its gmask); advances to the next one
  template <bool SCALAR = false>
  __device__ __forceinline__ int take() {
    if (!grouped) {
      const int key = entry<SCALAR>(e) * by + s * T;
      ent = e;
      ++s;
      if (s >= nsub || key + T >= kend) {
        ++e;
        s = 0;
      }
      return key;
    }
    const int key0 = wk;
    uint32_t m = 0;
    while (e < e1) {  // the blocks that meet window [key0, key0 + T)
      const int bs = entry<SCALAR>(e) * by, be = bs + by;
      if (bs >= key0 + T) break;
      const int glo = (max(bs, key0) - key0) >> 4, ghi = (min(be, key0 + T) - key0) >> 4;
      m |= ((1u << ghi) - 1u) & ~((1u << glo) - 1u);
      if (be > key0 + T) break;  // the block goes on in the next window
      ++e;
    }
    gmask = m;
    if (e < e1) {  // the next window: the next one, or the next block's first
      wk = max(key0 + T, (entry<SCALAR>(e) * by) & ~(T - 1));
      if (wk >= kend) e = e1;
    }
    return key0;
  }
};

// Element offsets of key tiles of KV head g of sequence b: packed rows
// (cu_kv[b] + key) * N2 + g, computed from a per-item base with no memory
// access, or through the page table (block_table[b, key / page_size], key %
// page_size) for paged caches.
template <bool PAGED>
struct KvAddr {
  int64_t row0, step;
  const int32_t* block_table;
  int b, g, n2, d, page_size, max_pages;
  int64_t page_stride;
  __device__ __forceinline__ void init(const SeqArgs& sq, const int32_t* bt, int b_, int g_, int n2_, int d_,
                                       int page_size_, int max_pages_, int64_t page_stride_) {
    block_table = bt;
    b = b_;
    g = g_;
    n2 = n2_;
    d = d_;
    page_size = page_size_;
    max_pages = max_pages_;
    page_stride = page_stride_;
    step = (int64_t)n2_ * d_;
    row0 = PAGED ? 0 : (ldu(sq.cu_kv, b_) * n2_ + g_) * (int64_t)d_;
  }
  __device__ __forceinline__ int64_t off(int key0) const {
    if constexpr (PAGED)
      return ((int64_t)ldu(block_table, (int64_t)b * max_pages + key0 / page_size)) * page_stride +
             ((int64_t)(key0 % page_size) * n2 + g) * d;
    else
      return row0 + key0 * step;
  }
};

// Packs 8 consecutive fp32 accumulator values (elements base .. base+7 of an
// MFMA C fragment) into a 16-bit MFMA operand.
template <typename MF>
__device__ __forceinline__ u32x4_t pack8(const f32x16_t& x, int base) {
  u32x4_t r;
  r.x = MF::pack(x[base + 0], x[base + 1]);
  r.y = MF::pack(x[base + 2], x[base + 3]);
  r.z = MF::pack(x[base + 4], x[base + 5]);
  r.w = MF::pack(x[base + 6], x[base + 7]);
  return r;
}

// Per-lane LDS byte offsets of the two MFMA operand read patterns of a
// row-major tile with layout L, for reads whose first row is a multiple of 16:
//  * rd(kk): rows row0 + lane % 32, columns 16 kk + 8 (lane / 32) .. + 7 (an
//    A or B operand over D, ds_read_b128); add row0 * ROW_BYTES.
//  * tr(mt, h): the transposed read -- source lane s of each 16-lane group
//    points at row k0 + 4 (lane / 32) + s / 4 + 8 h, columns 32 mt + 16 ((lane
//    / 16) % 2) + 4 (s % 4) .. + 3, so lane l receives rows k0 + 4 (l / 32) +
//    8 h + {0..3} of column 32 mt + l % 32.  Add k0 * ROW_BYTES.  The two
//    reads h = 0, 1 form an A operand whose 8 k-slots match a C fragment
//    packed by pack8(x, 8 (kc % 2)) for the 16-row chunk k0 = 16 kc.
// Linear layouts keep one base per pattern (the rest are immediates); the
// XOR layout keeps every offset.
template <class L, int D, bool LIN = L::LINEAR>
struct Operands;

template <class L, int D>
struct Operands<L, D, true> {
  int rb, tb;
  __device__ __forceinline__ void init() {
    const int lane = lane_id(), s16 = lane & 15;
    rb = L::chunk_off(lane & 31, lane >> 5);
    tb = L::col_off(4 * (lane >> 5) + (s16 >> 2), 16 * ((lane >> 4) & 1) + 4 * (s16 & 3));
  }
  __device__ __forceinline__ int rd(int kk) const { return rb + 32 * kk; }
  __device__ __forceinline__ int tr(int mt, int h) const { return tb + 64 * mt + 8 * h * L::ROW_BYTES; }
};

template <class L, int D>
struct Operands<L, D, false> {
  int rd_[D / 16];
  int tr_[D / 32][2];
  __device__ __forceinline__ void init() {
    const int lane = lane_id(), s16 = lane & 15;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) rd_[kk] = L::chunk_off(lane & 31, 2 * kk + (lane >> 5));
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        tr_[mt][h] = L::col_off(4 * (lane >> 5) + (s16 >> 2) + 8 * h,
                                32 * mt + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3));
  }
  __device__ __forceinline__ int rd(int kk) const { return rd_[kk]; }
  __device__ __forceinline__ int tr(int mt, int h) const { return tr_[mt][h]; }
};

// Compact per-lane offsets of the same two read patterns for an XorTile<D>
// (3 registers instead of D/16 + D/16): the XOR permutation only moves the
// chunk bits that kk (resp. mt) select, so the row-major read of step kk is
// rb ^ 32 kk and the transposed read of feature tile mt, half h is
// tb[h] ^ 64 mt (checked for every lane, step and tile at D = 64 and 128).
// Each read then costs one XOR; refresh() keeps the compiler from hoisting
// the XORs (one register per step) out of a loop.
template <int D>
struct XorOperands {
  using L = XorTile<D>;
  int rb, tb0, tb1;
  __device__ __forceinline__ void init() {
    const int lane = lane_id(), s16 = lane & 15;
    rb = L::chunk_off(lane & 31, lane >> 5);
    const int c0 = 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
    tb0 = L::col_off(4 * (lane >> 5) + (s16 >> 2), c0);
    tb1 = L::col_off(4 * (lane >> 5) + (s16 >> 2) + 8, c0);
  }
  __device__ __forceinline__ void refresh() {
    pin(rb);
    pin(tb0);
    pin(tb1);
  }
  __device__ __forceinline__ int rd(int kk) const { return rb ^ (32 * kk); }
  __device__ __forceinline__ int tr(int mt, int h) const { return (h ? tb1 : tb0) ^ (64 * mt); }
};

// A/B operand (rows row0 + lane % 32) via ds_read_b128.
template <class L, class OF>
__device__ __forceinline__ u32x4_t read_operand_of(const char* lds, const OF& of, int row0, int kk) {
  return lds_read16(lds + row0 * L::ROW_BYTES, of.rd(kk));
}
template <class L, int D>
__device__ __forceinline__ u32x4_t read_operand(const char* lds, const Operands<L, D>& of, int row0, int kk) {
  return read_operand_of<L>(lds, of, row0, kk);
}
template <int D>
__device__ __forceinline__ u32x4_t read_operand(const char* lds, const XorOperands<D>& of, int row0, int kk) {
  return read_operand_of<XorTile<D>>(lds, of, row0, kk);
}
// A operand of the transposed tile for the 16-row chunk k0 = 16 kc, columns 32 mt ..
template <class L, class OF>
__device__ __forceinline__ u32x4_t read_tr_operand_of(const char* lds, const OF& of, int k0, int mt) {
  const char* base = lds + k0 * L::ROW_BYTES;
  const u32x2_t lo = lds_read_tr(base, of.tr(mt, 0));
  const u32x2_t hi = lds_read_tr(base, of.tr(mt, 1));
  u32x4_t r;
  r.x = lo.x;
  r.y = lo.y;
  r.z = hi.x;
  r.w = hi.y;
  return r;
}
template <class L, int D>
__device__ __forceinline__ u32x4_t read_tr_operand(const char* lds, const Operands<L, D>& of, int k0, int mt) {
  return read_tr_operand_of<L>(lds, of, k0, mt);
}
template <int D>
__device__ __forceinline__ u32x4_t read_tr_operand(const char* lds, const XorOperands<D>& of, int k0, int mt) {
  return read_tr_operand_of<XorTile<D>>(lds, of, k0, mt);
}

// Runs N MFMA steps whose A (or B) operands come from LDS: step i's operand
// is read by read(i) LOOK steps before mfma(i, operand) consumes it, and the
// order is pinned with scheduling barriers, so each MFMA finds its operand
// already loaded instead of waiting out the LDS latency.
template <int N, int LOOK, class ReadF, class MfmaF>
__device__ __forceinline__ void mfma_pipeline(ReadF read, MfmaF mfma) {
  u32x4_t ring[LOOK];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < LOOK; ++i) ring[i] = read(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const u32x4_t a = ring[i % LOOK];
    if (i + LOOK < N) ring[i % LOOK] = read(i + LOOK);
    mfma(i, a);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Stores a [32 x 32] C fragment holding X^T (rows = feature d, columns =
// token) as 16-bit values: lane l owns token column l % 32 and writes
// features d0 + 8 i + 4 (l / 32) .. + 3 for i < 4 as 8-byte pieces.
template <typename MF>
__device__ __forceinline__ void store_cols(uint16_t* row_ptr, int d0, const f32x16_t& x, float mul) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x2_t v;
    v.x = MF::pack(x[4 * i + 0] * mul, x[4 * i + 1] * mul);
    v.y = MF::pack(x[4 * i + 2] * mul, x[4 * i + 3] * mul);
    *reinterpret_cast<u32x2_t*>(row_ptr + d0 + 8 * i + 4 * (lane >> 5)) = v;
  }
}

}  // namespace bsa
