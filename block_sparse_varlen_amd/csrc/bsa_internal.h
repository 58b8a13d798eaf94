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
  H_COUNT = 16  // header size in int32 (padded)
};

enum SparseKind { SP_NONE = 0, SP_MASK = 1, SP_SABI = 2, SP_IDX = 3 };

// Attention work items are handed to the 8 XCDs in runs of XCD_SEG
// consecutive items (xcd_item in bsa_attn.h); grids are padded to whole rounds.
constexpr int NUM_XCD = 8;
constexpr int XCD_SEG = 32;

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
  int32_t kvkey_max; // largest possible key of a dK/dV item
};

// Byte offsets of the workspace regions (all 256-byte aligned).
struct Layout {
  size_t hdr, sq, skv, qbase, kbase, qb_seq, kb_seq;
  size_t row_cnt, row_ptr, cols, key0, val0, key1, val1, hist, work;
  size_t col_cnt, col_ptr, col_fill, qrows, kvkey0, kvval0, kvkey1, kvval1, kvhist, work_kv;
  size_t ndl, lse2;
  size_t index_end;  // bytes used by the index products
  size_t total;      // bytes needed in all
};

// Everything a kernel needs to interpret sequences and the selection.
struct SeqArgs {
  const int64_t* cu_q;
  const int64_t* cu_kv;       // TND keys, or nullptr when paged
  const int32_t* seqused_kv;  // paged keys, or nullptr
  int32_t batch;
  int32_t bx, by;
  int32_t causal;
};

struct SelArgs {
  const void* sparse;
  const int32_t* count;
  int32_t kind;
  int32_t hs;      // Hs
  int32_t rows;    // selection tensor row dimension
  int32_t width;   // W
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
  int32_t* col_cnt;  // [cbar]
  int32_t* col_ptr;  // [cbar+1]
  int32_t* col_fill; // [cbar]
  int32_t* qrows;    // [nnzbar]
  int32_t* work_kv;  // [kvbar]
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
  int32_t n1, n2, group;   // N1, N2, G = N1/N2
  int32_t heads_per_row;   // G when the selection is shared by a GQA group, else 1
  int32_t page_size, max_pages;
  int64_t page_stride;     // elements
  float sigma;             // fp32 scale
  float sigma_log2e;       // scale * log2(e)
};

struct BwdPreArgs {
  const void* out;
  const void* dout;
  const float* lse;
  float* ndl;   // -rowsum(dO o O)
  float* lse2;  // lse * log2(e)
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
  const int32_t* block_table;  // paged K/V (and dK/dV): [B, max_pages]
  int32_t page_size, max_pages;
  int64_t page_stride;     // elements
  int32_t n1, n2, group, heads_per_row, hs;
  int32_t sub_tiles;       // block_y / 128 (dK/dV tiles per KV block)
  float sigma;
  float sigma_log2e;
};

// ---- launchers (defined in the .hip files) ----
hipError_t launch_index(const SeqArgs& seq, const SelArgs& sel, const Bounds& bd, const IndexPtrs& ip,
                        int n2, int group, bool with_csc, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, int dtype, int head_dim, int64_t grid, hipStream_t stream);
// e4m3 q / k / v (head dim 128), out in out_dtype
hipError_t launch_fwd_fp8(const FwdArgs& a, int out_dtype, int64_t grid, hipStream_t stream);
hipError_t launch_bwd_pre(const BwdPreArgs& a, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int dtype, int head_dim, int64_t grid, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int dtype, int head_dim, int64_t grid, hipStream_t stream);

// Profiling hooks (bsa_api.cpp): bracket a launch with events when enabled.
void prof_begin(int kernel, hipStream_t stream);
void prof_end(int kernel, hipStream_t stream);

}  // namespace bsa
