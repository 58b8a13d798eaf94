// Pieces shared by the forward and backward attention kernels: work-item
// decoding, key-tile staging (global -> registers -> LDS) and the walk over a
// row's selected KV blocks in 64-key sub-tiles.
#pragma once

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

constexpr int KT = 64;   // keys per sub-tile of the Q-major kernels
constexpr int QT = 128;  // query rows per Q-major work item (4 waves x 32)

// A Q-major work item: one q-block of one q-head.
struct QItem {
  int r;        // CSR row
  int h, g;     // q-head, kv-head
  int b, qb;    // sequence, local q-block
  int64_t q0;   // first token row of sequence b
  int sq, skv;  // lengths
  int row_lo;   // first local query row of the item
  int nrows;    // valid query rows in the item
};

// item = slot * heads_per_row + j; slot indexes the longest-first row order.
__device__ __forceinline__ bool decode_qitem(int64_t item, const int32_t* hdr, const int32_t* work,
                                             const int32_t* qb_seq, const int32_t* qbase, const SeqArgs& seq,
                                             int heads_per_row, int group, QItem& it) {
  const int R = hdr[H_R];
  if (item >= (int64_t)R * heads_per_row) return false;
  const int slot = (int)(item / heads_per_row);
  const int jh = (int)(item - (int64_t)slot * heads_per_row);
  it.r = work[slot];
  const int TQB = hdr[H_TQB];
  const int hs = it.r / TQB;
  const int qg = it.r - hs * TQB;
  it.h = heads_per_row == 1 ? hs : hs * group + jh;
  it.g = it.h / group;
  it.b = qb_seq[qg];
  it.qb = qg - qbase[it.b];
  it.q0 = seq.cu_q[it.b];
  it.sq = (int)(seq.cu_q[it.b + 1] - it.q0);
  it.skv = seq.seqused_kv ? seq.seqused_kv[it.b] : (int)(seq.cu_kv[it.b + 1] - seq.cu_kv[it.b]);
  it.row_lo = it.qb * QT;
  it.nrows = min(QT, it.sq - it.row_lo);
  return true;
}

__device__ __forceinline__ KvAddr make_kv_addr(const SeqArgs& seq, const int32_t* block_table, int b, int g,
                                               int n2, int D, int page_size, int max_pages,
                                               int64_t page_stride) {
  KvAddr ka;
  ka.block_table = block_table;
  ka.paged = seq.seqused_kv != nullptr;
  ka.seq_row0 = ka.paged ? 0 : seq.cu_kv[b];
  ka.bt_row = b * max_pages;
  ka.page_size = page_size;
  ka.page_stride = page_stride;
  ka.row_stride = (int64_t)n2 * D;
  ka.head_off = (int64_t)g * D;
  return ka;
}

// Staging of a [ROWS x D] 16-bit tile: 256 threads, 16 bytes each per pass.
template <int D, int ROWS>
struct Stage {
  static constexpr int CH = D / 8;
  static constexpr int RPP = 256 / CH;      // rows per pass
  static constexpr int PASSES = ROWS / RPP;
  static_assert(ROWS % RPP == 0, "tile rows must fill whole passes");
  u32x4_t r[PASSES];

  // rows whose `ok(row)` is false are zero-filled; `off(row)` is the element
  // offset of the row's column 0.
  template <typename OffF, typename OkF>
  __device__ __forceinline__ void load(const uint16_t* base, OffF off, OkF ok) {
    const int c = threadIdx.x % CH;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = p * RPP + threadIdx.x / CH;
      r[p] = ok(row) ? gload16(base + off(row) + c * 8) : zero_u4();
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int c = threadIdx.x % CH;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = p * RPP + threadIdx.x / CH;
      lds_write16(lds, Tile<D>::chunk_off(row, c), r[p]);
    }
  }
};

// Walk over the 64-key sub-tiles of a CSR row: blocks cols[e0..e1), each cut
// into by / 64 sub-tiles, keeping those whose first key is below `kend` (the
// key bound of the item: Skv, or the causal limit of its last row + 1).
struct SubTileWalk {
  const int32_t* cols;
  int e, e1, s, nsub, by, kend;
  __device__ __forceinline__ void init(const int32_t* c, int e0, int e_end, int by_, int kend_) {
    cols = c;
    e = e0;
    e1 = e_end;
    s = 0;
    by = by_;
    nsub = by_ / KT;
    kend = kend_;
  }
  __device__ __forceinline__ bool valid() const { return e < e1; }
  __device__ __forceinline__ int key() const { return cols[e] * by + s * KT; }
  __device__ __forceinline__ void next() {
    ++s;
    if (s >= nsub || cols[e] * by + s * KT >= kend) {
      ++e;
      s = 0;
    }
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

// A-operand read of a transposed 16-bit tile (rows = contraction index):
// lane l gets rows k0 + 4 (l / 32) + {0..3} and + 8 + {0..3} of column
// col0 + l % 32 -- the key/query-slot order that matches a C fragment packed
// with pack8(x, 8 * (kc % 2)) for 16-row chunk kc (k0 = 16 kc).
template <int D>
__device__ __forceinline__ u32x4_t read_tr_operand(const char* lds, int k0, int col0) {
  const int lane = lane_id();
  const int s16 = lane & 15;
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
  const int row = k0 + 4 * (lane >> 5) + (s16 >> 2);
  const u32x2_t lo = lds_read_tr(lds, Tile<D>::col_off(row, col));
  const u32x2_t hi = lds_read_tr(lds, Tile<D>::col_off(row + 8, col));
  u32x4_t r;
  r.x = lo.x;
  r.y = lo.y;
  r.z = hi.x;
  r.w = hi.y;
  return r;
}

// A/B-operand read of a row-major tile: lane l gets row row0 + l % 32,
// columns 16 kk + 8 (l / 32) .. + 7.
template <int D>
__device__ __forceinline__ u32x4_t read_operand(const char* lds, int row0, int kk) {
  const int lane = lane_id();
  return lds_read16(lds, Tile<D>::chunk_off(row0 + (lane & 31), 2 * kk + (lane >> 5)));
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
