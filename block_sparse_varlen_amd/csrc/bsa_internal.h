// Internal definitions shared by the host planner (bsa_api.cpp) and the HIP
// kernels of libbsa.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bsa {

// int32 header written at the start of the index region of the workspace.
enum HeaderSlot {
  H_TQB = 0,    // total q-blocks: sum_b ceil(Sq_b / block_x)
  H_TKB = 1,    // total kv-blocks: sum_b ceil(Skv_b / block_y)
  H_R = 2,      // rows = Hs * TQB
  H_C = 3,      // columns = Hs * TKB
  H_NNZ = 4,    // visited (row, kv-block) pairs
  H_KVITEMS = 5,// N2 * TKB
  H_CHECK = 6,  // value check word (CHK_* bits) of BSA_FLAG_CHECK_VALUES; 0 once the index is built
  H_COUNT = 16  // header size in int32 (padded)
};

// Bits of the value check word (the numbers of the public BSA_CHECK_* list).
enum CheckBit : uint32_t {
  CHK_CU_Q_ENDS = 1u,    // cu_seqlens_q[0] != 0 or cu_seqlens_q[B] != total_q
  CHK_CU_Q_ORDER = 2u,   // cu_seqlens_q decreases somewhere
  CHK_SQ_LONG = 4u,      // some Sq_b > max_seqlen_q
  CHK_CU_KV_ENDS = 8u,   // TND: cu_seqlens_kv[0] != 0 or cu_seqlens_kv[B] > total_kv
  CHK_CU_KV_ORDER = 16u, // TND: cu_seqlens_kv decreases somewhere
  CHK_SKV_LONG = 32u,    // some Skv_b > max_seqlen_kv (TND), or seqused_kv[b] outside [0, max_seqlen_kv] (paged)
  CHK_PAGE = 64u         // paged: a block_table entry of a page holding keys < seqused_kv[b] outside [0, pages)
};

// The device-resident sequence description and the extents the descriptor
// gives each array: cu_q [batch + 1], cu_kv [batch + 1] (TND), seqused_kv
// [batch] and block_table [batch, max_pages] (paged).
struct CheckArgs {
  const int64_t* cu_q;
  const int64_t* cu_kv;       // TND, else nullptr
  const int32_t* seqused_kv;  // paged, else nullptr
  const int32_t* block_table; // paged, else nullptr
  int32_t batch, max_sq, max_skv, page_size, max_pages;
  int64_t total_q, total_kv;  // total_kv: rows (TND) or pages (paged)
};

enum SparseKind { SP_NONE = 0, SP_MASK = 1, SP_SABI = 2, SP_IDX = 3, SP_IDX_B = 4, SP_KV = 5, SP_KV_B = 6 };
__host__ __device__ inline bool kv_lists(int kind) { return kind == SP_KV || kind == SP_KV_B; }

// Row tiles: q-blocks of at most ROW_TILE_MAX_BX rows that divide ROW_TILE
// are grouped into ROW_TILE-row tiles (see SeqArgs), when block_y is a
// multiple of 64 and a row of the index has at most ROW_TILE_MAX_KB blocks.
constexpr int ROW_TILE = 128;
constexpr int ROW_TILE_MAX_BX = 32;
constexpr int ROW_TILE_MAX_KB = 2048;

// Attention work items are handed to the 8 XCDs in runs of 2^xseg
// consecutive items (xcd_item in bsa_attn.h; xseg is a launch argument);
// grids are padded to whole rounds of 8 runs.
constexpr int NUM_XCD = 8;

// Host-known upper bounds that size every workspace region.
struct Bounds {
  int64_t qbar;      // >= total q-blocks
  int64_t kbar;      // >= total kv-blocks
  int64_t rbar;      // Hs * qbar
  int64_t cbar;      // Hs * kbar
  int64_t nnzbar;    // rbar * cmax
  int64_t kvbar;     // N2 * kbar
  int32_t nqb_max;   // ceil(max_seqlen_q / bx)
  int32_t nkb_max;   // ceil(max_seqlen_kv / by)
  int32_t cmax;      // largest possible visited count of a row
  int64_t qbar_sel;  // >= total selection q-blocks (block_x rows each; = qbar without row tiles)
  int32_t kvkey_max; // largest possible key of a dK/dV item
  int32_t q_chunk_heads;  // sparse heads per dispatch chunk of the Q-major passes (>= Hs: one chunk)
};

// Byte offsets of the workspace regions (all 256-byte aligned).
struct Layout {
  size_t hdr, sq, skv, qbase, kbase, qb_seq, kb_seq;
  size_t row_cnt, row_ptr, cols, key0, val0, key1, val1, hist, work, work_q, kvbm;
  size_t col_cnt, col_ptr, col_fill, qrows, kvkey0, kvval0, kvkey1, kvval1, kvhist, work_kv;
  size_t ndl, lse2, dq_acc;
  size_t qbase_sel, row_mask, col_mask;  // row tiles only (0 otherwise)
  size_t index_end;  // bytes used by the index products
  size_t total;      // bytes needed in all
};

// Everything a kernel needs to interpret sequences and the selection.
struct SeqArgs {
  const int64_t* cu_q;
  const int64_t* cu_kv;       // TND keys, or nullptr when paged
  const int32_t* seqused_kv;  // paged keys, or nullptr
  int32_t batch;
  // bx: query rows per q-block of the index and of the kernels' work items.
  // sel_bx: rows per q-block of the caller's selection (block_x).  They differ
  // only with row tiles: q-blocks of at most 32 rows that divide 128 are
  // grouped into tiles of bx = 128 rows, each visiting the union of its
  // q-blocks' visited sets, with per-row masks (row_tiles below).
  int32_t bx, sel_bx, by;
  // Token window of the causal and band masks: key j is allowed for query i
  // when i + (Skv - Sq) + win_lo <= j <= i + (Skv - Sq) + win_hi (no window:
  // masked = 0).  Causal: win_lo = -WIN_INF, win_hi = 0; band: -preTokens,
  // nextTokens, both clamped to [-WIN_INF, WIN_INF].
  int32_t masked;
  int32_t win_lo, win_hi;
};
// Any window edge at or beyond this many tokens acts as unbounded (sequence
// lengths stay below 2^28, so i + (Skv - Sq) + win never overflows int32).
constexpr int32_t WIN_INF = 1 << 30;
// Kernel variant of the token window: 0 none, 1 an upper end only (causal, or
// a band with unbounded preTokens), 2 both ends.
inline int window_mode(const SeqArgs& s) { return !s.masked ? 0 : s.win_lo <= -WIN_INF ? 1 : 2; }

struct SelArgs {
  const void* sparse;
  const int32_t* count;
  int32_t kind;
  int32_t hs;      // Hs
  int32_t rows;    // selection tensor row dimension
  int32_t width;   // W
  // per-KV-block lists: the rows' visited-block bitmaps the lists are first
  // scattered into ([rows of the index][kv_words] words), else nullptr
  uint32_t* kvbm;
  int32_t kv_words;
};

struct IndexPtrs {
  int32_t* hdr;
  int32_t* sq;       // [B]
  int32_t* skv;      // [B]
  int32_t* qbase;    // [B+1]
  int32_t* kbase;    // [B+1]
  int32_t* qb_seq;   // [qbar]
  int32_t* kb_seq;   // [kbar]
  int32_t* row_cnt;  // [rbar]
  int32_t* row_ptr;  // [rbar+1]
  int32_t* cols;     // [nnzbar]
  int32_t* key0; int32_t* val0; int32_t* key1; int32_t* val1;  // [max(rbar, kvbar)]
  int32_t* hist;     // [256 * (ceil(rbar/256) + ceil(kvbar/256)) + 2]
  int32_t* work;     // [rbar]
  int32_t* work_q;   // [rbar] work grouped by head chunk (the Q-major dispatch order when chunked)
  int32_t* col_cnt;  // [cbar]
  int32_t* col_ptr;  // [cbar+1]
  int32_t* col_fill; // [cbar]
  int32_t* qrows;    // [nnzbar]
  int32_t* work_kv;  // [kvbar]
  // row tiles only (nullptr otherwise):
  int32_t* qbase_sel;   // [B+1] first global selection q-block of each sequence
  uint32_t* row_mask;   // [nnzbar][4] per CSR entry: bit i of the 128-bit mask = row i of the tile
                        //   lies in a q-block that visits the entry's block
  uint32_t* col_mask;   // [nnzbar][4] the same per CSC entry
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  SeqArgs seq;
  const int32_t* block_table;
  const int32_t* hdr;
  const int32_t* qb_seq;
  const int32_t* qbase;
  const int32_t* row_ptr;
  const int32_t* cols;
  const int32_t* work;
  const uint32_t* row_mask;  // row tiles with a selection: [nnz][4] per CSR entry, else nullptr
  int32_t n1, n2, group;   // N1, N2, G = N1/N2
  int32_t heads_per_row;   // G when the selection is shared by a GQA group, else 1
  int32_t page_size, max_pages;
  int64_t page_stride;     // elements
  float sigma;             // fp32 scale
  float sigma_log2e;       // scale * log2(e)
  int32_t xseg;            // log2 of the run of consecutive items each XCD takes
};

struct BwdPreArgs {
  const void* out;
  const void* dout;
  const float* lse;
  float* ndl;   // -rowsum(dO o O)
  float* lse2;  // lse * log2(e)
  float* dq_acc;  // fp32 dQ accumulator [T_q, N1, D] to clear (atomic dQ), or nullptr
  int64_t rows; // T_q * N1
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* lse2;  // lse * log2(e)
  const float* ndl;  // -rowsum(dO o O)
  void* dq;
  void* dk;
  void* dv;
  float* dq_acc;  // atomic dQ: fp32 [T_q, N1, D] accumulator of dS K (unscaled), else nullptr
  SeqArgs seq;
  const int32_t* hdr;
  const int32_t* qb_seq;
  const int32_t* kb_seq;
  const int32_t* qbase;
  const int32_t* kbase;
  const int32_t* row_ptr;
  const int32_t* cols;
  const int32_t* work;
  const int32_t* col_ptr;
  const int32_t* qrows;
  const int32_t* work_kv;
  const uint32_t* row_mask;    // row tiles with a selection: [nnz][4] per CSR entry, else nullptr
  const uint32_t* col_mask;    // the same per CSC entry
  const int32_t* block_table;  // paged K/V (and dK/dV): [B, max_pages]
  int32_t page_size, max_pages;
  int64_t page_stride;     // elements
  int32_t n1, n2, group, heads_per_row, hs;
  int32_t sub_tiles;       // ceil(block_y / 128): dK/dV tiles per KV block (the last one may be partial)
  float sigma;
  float sigma_log2e;
  int32_t xseg_q, xseg_kv;  // log2 of the XCD runs of the dQ and the dK/dV launches
};

// ---- launchers (defined in the .hip files) ----
hipError_t launch_index(const SeqArgs& seq, const SelArgs& sel, const Bounds& bd, const IndexPtrs& ip,
                        int n2, int group, bool with_csc, hipStream_t stream);
// writes the value check word of `c` to hdr[H_CHECK]
hipError_t launch_check_values(const CheckArgs& c, int32_t* hdr, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, int dtype, int head_dim, int64_t grid, hipStream_t stream);
// e4m3 q / k / v (head dim 128), out in out_dtype
hipError_t launch_fwd_fp8(const FwdArgs& a, int out_dtype, int64_t grid, hipStream_t stream);
hipError_t launch_bwd_pre(const BwdPreArgs& a, int dtype, int head_dim, hipStream_t stream);
// with a.dq_acc set, the dK/dV kernel also adds dS K into it (atomic dQ)
hipError_t launch_bwd_dkdv(const BwdArgs& a, int dtype, int head_dim, int64_t grid, hipStream_t stream);
// dq = scale * dq_acc in dtype
hipError_t launch_dq_convert(const float* acc, void* dq, int64_t elems, float sigma, int dtype, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int dtype, int head_dim, int64_t grid, hipStream_t stream);

// Profiling hooks (bsa_api.cpp): bracket a launch with events when enabled.
void prof_begin(int kernel, hipStream_t stream);
void prof_end(int kernel, hipStream_t stream);

}  // namespace bsa
