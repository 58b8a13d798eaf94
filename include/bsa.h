/*
 * bsa.h -- variable-length (TND-packed) block-sparse FlashAttention for
 * AMD Instinct MI355X (gfx950), C ABI of libbsa.so.
 *
 * The operation.  For every sequence b, q-head h and query row i the forward
 * pass computes softmax(scale * q_i K_sel^T) V_sel over the keys j that row i
 * may attend to, and the natural-log log-sum-exp of the scaled scores
 * (BlockSparseAttentionGrad README, "Function description", forward formula;
 * GenericBlockSparseAttention page, "Sparse attention mechanism";
 * BlitzSparseAttention page, "softmax_lse output").  The backward pass
 * returns dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO with
 * dS = P o (dO V^T - rowsum(dO o O)) (BlockSparseAttentionGrad README,
 * backward formulas).
 *
 * Key j (local to sequence b) is allowed for query i (local) when
 *   (a) block floor(j / block_y) is selected for q-block floor(i / block_x)
 *       of sparse head hs(h) (see BSA_SPARSE_*),
 *   (b) j < Skv_b, and
 *   (c) with BSA_MASK_CAUSAL, j <= i + Skv_b - Sq_b (causal mask aligned at
 *       the bottom-right corner, the FlashAttention UnpaddingScoreGradV2
 *       page's rightDownCausal, the only causal mode of its TND layout);
 *       with BSA_MASK_BAND, i + Skv_b - Sq_b - pre_tokens <= j <=
 *       i + Skv_b - Sq_b + next_tokens (the band, sparseMode 4, of the
 *       FlashAttention UnpaddingScoreGradV2 page, section 6.6, and the
 *       BlitzSparseAttention page's sparseMode limits, aligned at the same
 *       corner; preTokens / nextTokens count the earlier / later tokens the
 *       sliding window keeps, PromptFlashAttention page, attribute table).
 * A row with no allowed key gets O = 0 and lse = +inf; in the backward pass
 * its dQ is 0, and keys no row reaches get dK = dV = 0.
 *
 * A selection is a set: duplicate entries count once, entry order does not
 * matter, entries outside [0, nKB_b) are skipped, an idx count is clamped to
 * [0, W], and rows past the selection tensor's row dimension select nothing.
 * KV block indices are local to their sequence.  q-head h reads KV head
 * h / (N1 / N2).
 *
 * Two-stage use, following the pages' two-stage calls (size query, then
 * execute on a stream; GenericBlockSparseAttention page, "aclnn API"):
 *   1. bsa_get_workspace_size(): host only, checks the descriptor and returns
 *      the device workspace each call needs.
 *   2. bsa_fwd() / bsa_bwd(): enqueue all work on `stream` and return.  Each
 *      call rebuilds its block index in the workspace first (the pages
 *      require the schedule metadata to be regenerated for every call).
 *
 * Ownership.  Every pointer argument of stage 2 is caller-owned device
 * memory (except the descriptor, a host pointer).  The library never
 * allocates, frees or synchronizes (BSA_FLAG_CHECK_VALUES aside); outputs are fully overwritten (no
 * pre-zeroing needed; for paged dK/dV see bsa_bwd) and must not alias inputs
 * or the workspace; workspace
 * contents are undefined on entry and exit.  Calls on different streams with
 * different workspaces may run concurrently.  A call enqueues nothing but
 * kernel launches, so it can be captured into a HIP graph and replayed
 * (not with BSA_FLAG_CHECK_VALUES, which waits on the stream, nor while
 * bsa_profile_enable is on).
 *
 * Errors.  Status codes reuse the pages' numbers (GenericBlockSparseAttention
 * page, first-stage return codes).  Device-resident values (cu_seqlens,
 * seqused_kv, block_table entries) are not validated by default, as on the
 * pages (GenericBlockSparseAttention page, "values are not checked at tiling
 * time"): inconsistent values are undefined behaviour, except out-of-range
 * *selection* entries, which are defined as skipped.  BSA_FLAG_CHECK_VALUES
 * validates them first.
 */
#ifndef BSA_H_
#define BSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsa_status {
  BSA_OK = 0,
  BSA_ERR_PARAM_NULLPTR = 161001, /* a required pointer is NULL */
  BSA_ERR_PARAM_INVALID = 161002, /* unsupported dtype/shape/attribute, or workspace too small */
  BSA_ERR_INNER = 561103,         /* a valid combination with no compiled kernel variant */
  BSA_ERR_RUNTIME = 561000        /* a HIP launch or runtime error */
} bsa_status_t;

/* Element types.  BSA_DTYPE_FP8_E4M3 is FLOAT8_E4M3 (OCP e4m3fn: 4 exponent
 * bits, bias 7, 3 mantissa bits, no infinities, max 448) for q, k and v of a
 * forward pass: GenericBlockSparseAttention's quantType 5 (Quantisation
 * table), where the operator casts P to the same fp8 type itself and no
 * scale factors are passed; out is fp16 or bf16 (out_dtype).  Head dim 128
 * only; bsa_bwd has no fp8 variant (BSA_ERR_INNER). */
enum { BSA_DTYPE_F16 = 1, BSA_DTYPE_BF16 = 2, BSA_DTYPE_FP8_E4M3 = 3 };

/* How the per-q-block KV block selection is given (argument `sparse`). */
enum {
  /* every KV block of the sequence is selected; `sparse` is ignored */
  BSA_SPARSE_NONE = 0,
  /* uint8 [B, Hs, sparse_rows, sparse_width], nonzero = compute column kb
     (BlockSparseAttentionGrad README, blockSparseMaskOptional) */
  BSA_SPARSE_BLOCK_MASK = 1,
  /* uint16 [B, Hs, sparse_rows, sparse_width], KV block indices, 0xFFFF =
     unused slot (BlitzSparseAttention page, sabi section) */
  BSA_SPARSE_SABI_U16 = 2,
  /* int32 [Hs, sparse_rows, sparse_width] over global q-blocks (sparse_rows =
     totalQBlocks = sum_b ceil(Sq_b / block_x)), -1 = unused, plus
     `sparse_count` int32 [Hs, sparse_rows]: the first count entries are live
     (GenericBlockSparseAttention page, sparseBlockIdx / sparseBlockCount;
     layoutSparsePattern 4, or 6 with Hs = N1) */
  BSA_SPARSE_IDX_I32 = 3,
  /* The same lists with a batch axis: int32 [B, Hs, sparse_rows, sparse_width]
     over local q-blocks, count int32 [B, Hs, sparse_rows] (layoutSparsePattern
     0, or 2 with Hs = N1) */
  BSA_SPARSE_IDX_BATCH_I32 = 4,
  /* Per-KV-block lists: int32 [Hs, sparse_rows, sparse_width], row gk =
     kbase_b + kb over global KV blocks (sparse_rows = totalKBlocks = sum_b
     ceil(Skv_b / block_y)) naming the local q-blocks that chose KV block kb,
     -1 = unused, count int32 [Hs, sparse_rows] (layoutSparsePattern 5, or 7
     with Hs = N1: "each KV block lists the Q blocks that chose it").  KV block
     kb is selected for q-block qb when qb is among its list's first count
     entries. */
  BSA_SPARSE_KV_IDX_I32 = 5,
  /* Per-KV-block lists with a batch axis: int32 [B, Hs, sparse_rows,
     sparse_width] over local KV blocks, count int32 [B, Hs, sparse_rows]
     (layoutSparsePattern 1, or 3 with Hs = N1) */
  BSA_SPARSE_KV_IDX_BATCH_I32 = 6
};

/* Token masks.  BSA_MASK_BAND reads pre_tokens / next_tokens; either may be
   negative (a window that leaves out the diagonal key), and a window with
   pre_tokens + next_tokens < 0 holds no key.  Values beyond 2^30 in size act
   as unbounded: BAND with pre_tokens >= 2^30 and next_tokens = 0 is CAUSAL.
   GenericBlockSparseAttention's planned window mask (winLeft / winRight) is
   the same band. */
enum { BSA_MASK_NONE = 0, BSA_MASK_CAUSAL = 1, BSA_MASK_BAND = 2 };

/* K/V layout: packed [T_kv, N2, D] rows addressed through cu_seqlens_kv, or
   paged [pages, page_size, N2, D] through block_table + seqused_kv
   (GenericBlockSparseAttention page, "Paged Attention", PA_BBND). */
enum { BSA_KV_TND = 0, BSA_KV_PAGED = 1 };

/* Call flags (bsa_problem_t.flags).
 * BSA_FLAG_INDEX_BUILT: the workspace already holds the block index of this
 *   problem and selection, built by bsa_build_index() into it (with_csc != 0
 *   for bsa_bwd) and not overwritten since, so bsa_fwd / bsa_bwd skip
 *   rebuilding it -- GenericBlockSparseAttention's metadata operator, whose
 *   output the main operator consumes; as there, an index that does not match
 *   the call (other problem, selection or sequence lengths) is undefined
 *   behaviour.  A training step can build the index once and run both passes
 *   on it.  The workspace size rules are unchanged. */
enum { BSA_FLAG_INDEX_BUILT = 1u };
/* dQ of bsa_bwd.  By default it comes from a separate Q-block-major pass over
 * the per-q-block lists (no atomics: bit-identical results run to run).
 * BSA_FLAG_DQ_ATOMIC instead adds dS K into an fp32 accumulator inside the
 * KV-major dK/dV kernel with atomics, then scales and converts it (the
 * workspace grows by T_q * N1 * D * 4 bytes; results vary in the last bits
 * from run to run, as the FlashAttention UnpaddingScoreGradV2 page says of
 * its own default).  BSA_FLAG_DETERMINISTIC asks for bit-identical results
 * run to run and so excludes BSA_FLAG_DQ_ATOMIC (both set:
 * BSA_ERR_PARAM_INVALID).  Both flags are ignored by bsa_fwd. */
enum { BSA_FLAG_DETERMINISTIC = 2u, BSA_FLAG_DQ_ATOMIC = 4u };
/* BSA_FLAG_CHECK_VALUES: before any other device work, bsa_fwd / bsa_bwd /
 * bsa_build_index run one validator kernel over the device-resident sequence
 * description, wait for it (the stream is synchronized: not for use under
 * graph capture) and return BSA_ERR_PARAM_INVALID, with nothing else
 * enqueued, when a check fails.  The failed checks' BSA_CHECK_* bits are
 * left in header[6] of the workspace (bsa_index_view's off_header; 0 after a
 * call that passed).  Checked: cu_seqlens_q starts at 0, never decreases and
 * ends at total_q, with every Sq_b <= max_seqlen_q; TND: cu_seqlens_kv starts
 * at 0, never decreases and ends at most at total_kv, with every Skv_b <=
 * max_seqlen_kv; paged: every seqused_kv[b] in [0, max_seqlen_kv] and, in
 * bsa_fwd / bsa_bwd, every block_table entry of a page that holds keys below
 * seqused_kv[b] in [0, total_kv).  Not checked: whether sequences share a
 * page (bsa_bwd forbids it) and selection values (out-of-range entries are
 * defined as skipped).  bsa_fwd_noalloc rejects the flag. */
enum { BSA_FLAG_CHECK_VALUES = 8u };
enum {
  BSA_CHECK_CU_Q_ENDS = 1,    /* cu_seqlens_q[0] != 0 or cu_seqlens_q[B] != total_q */
  BSA_CHECK_CU_Q_ORDER = 2,   /* cu_seqlens_q decreases somewhere */
  BSA_CHECK_SQ_LONG = 4,      /* some Sq_b > max_seqlen_q */
  BSA_CHECK_CU_KV_ENDS = 8,   /* TND: cu_seqlens_kv[0] != 0 or cu_seqlens_kv[B] > total_kv */
  BSA_CHECK_CU_KV_ORDER = 16, /* TND: cu_seqlens_kv decreases somewhere */
  BSA_CHECK_SKV_LONG = 32,    /* TND: some Skv_b > max_seqlen_kv; paged: seqused_kv[b] outside [0, max_seqlen_kv] */
  BSA_CHECK_PAGE = 64         /* paged: a block_table entry that is read lies outside [0, total_kv) */
};

typedef struct bsa_problem {
  uint32_t struct_size;      /* sizeof(bsa_problem_t) */
  int32_t dtype;             /* BSA_DTYPE_*: q, k, v, dout, and out, dq, dk, dv unless out_dtype says otherwise */
  int32_t batch;             /* B >= 0 */
  int32_t num_heads_q;       /* N1 in [1, 256] */
  int32_t num_heads_kv;      /* N2 >= 1, N1 % N2 == 0, N1 / N2 <= 128 */
  int32_t head_dim;          /* D in {64, 128} */
  int64_t total_q;           /* T_q: rows of q/out/dout/dq (= cu_seqlens_q[B]) */
  int64_t total_kv;          /* T_kv rows of k/v (TND) or number of pages (paged) */
  int32_t max_seqlen_q;      /* upper bound on every Sq_b */
  int32_t max_seqlen_kv;     /* upper bound on every Skv_b */
  int32_t block_x;           /* q rows per selection block; 1 .. 4096 (work items hold up to 128 rows of one
                                q-block; q-blocks of at most 32 rows that divide 128 are grouped into
                                128-row tiles with per-row masks, see the index layout below) */
  int32_t block_y;           /* keys per selection block; multiple of 16, <= 4096 */
  int32_t sparse_kind;       /* BSA_SPARSE_* */
  int32_t sparse_heads;      /* Hs: N1 (pattern per q-head) or N2 (shared by a GQA group) */
  int32_t sparse_rows;       /* row dimension of the selection tensor (see BSA_SPARSE_*) */
  int32_t sparse_width;      /* W: columns (mask), slots (sabi), topK (per-q-block lists, <= 256) or
                                q-blocks per list (per-KV-block lists) */
  int32_t mask_type;         /* BSA_MASK_* */
  int32_t kv_layout;         /* BSA_KV_* */
  int32_t page_size;         /* paged: tokens per page, multiple of 64 */
  int32_t max_pages_per_seq; /* paged: second dimension of block_table */
  int64_t page_stride;       /* paged: elements between pages, >= page_size*N2*D, multiple of N2*D */
  double scale;              /* > 0, or 0 for 1/sqrt(D); applied rounded to fp32 */
  uint32_t flags;            /* BSA_FLAG_* bits, others must be 0 */
  int32_t out_dtype;         /* 0 (= dtype) or dtype for fp16 / bf16; F16 or BF16 with FP8_E4M3 inputs */
  int64_t pre_tokens;        /* BSA_MASK_BAND: earlier tokens the window keeps (else ignored) */
  int64_t next_tokens;       /* BSA_MASK_BAND: later tokens the window keeps (else ignored) */
} bsa_problem_t;

/* Stage 1.  Checks `p` and writes the workspace bytes bsa_fwd (`fwd_bytes`)
 * and bsa_bwd (`bwd_bytes`) need; either out-pointer may be NULL, not both.
 * Host only, no device work.  Sizes come from host-known bounds (total_q,
 * total_kv, maximum lengths, selection shape), never from device values.
 * Returns BSA_ERR_PARAM_NULLPTR, BSA_ERR_PARAM_INVALID for an unsupported
 * descriptor, BSA_ERR_INNER for a valid one with no compiled variant. */
bsa_status_t bsa_get_workspace_size(const bsa_problem_t* p, size_t* fwd_bytes, size_t* bwd_bytes);

/* Stage 2, forward.
 *   q            [T_q, N1, D]           dtype, contiguous
 *   k, v         [T_kv, N2, D] (TND) or [pages, page_size, N2, D] (paged,
 *                page axis strided by page_stride elements)
 *   cu_seqlens_q int64 [B+1], cu_seqlens_q[0] = 0, non-decreasing
 *   cu_seqlens_kv int64 [B+1] (TND; NULL when paged)
 *   seqused_kv   int32 [B] (paged: required; TND: NULL)
 *   sparse       selection tensor per p->sparse_kind (NULL for NONE)
 *   sparse_count count tensor of the list kinds (IDX*, KV_IDX*), else NULL
 *   block_table  int32 [B, max_pages_per_seq] (paged only, else NULL); only
 *                entries for pages holding keys < Skv_b are read
 *   out          [T_q, N1, D] out_dtype (dtype when out_dtype is 0)
 *   lse          float32 [T_q, N1], natural log of the scaled scores' sum
 * Returns BSA_ERR_PARAM_NULLPTR when a required pointer is NULL,
 * BSA_ERR_PARAM_INVALID when workspace_bytes is below the stage-1 value,
 * BSA_ERR_RUNTIME on a HIP error.  B == 0 or T_q == 0: BSA_OK, nothing done. */
bsa_status_t bsa_fwd(const bsa_problem_t* p, const void* q, const void* k, const void* v,
                     const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                     const int32_t* seqused_kv, const void* sparse, const int32_t* sparse_count,
                     const int32_t* block_table, void* out, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments and results as bsa_fwd without the workspace:
 * the block index is built in a device array the library owns, one per GPU
 * (BSA_NOALLOC_SCRATCH_BYTES, held until the process ends; its device address
 * is looked up once per device on the first call there, with that device
 * current).  Every call on a GPU shares that GPU's array and overwrites it:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and give undefined results; calls ordered on one stream are safe.  Returns
 * BSA_ERR_PARAM_INVALID when the problem's forward workspace
 * (bsa_get_workspace_size's fwd_bytes) exceeds the array or when
 * BSA_FLAG_INDEX_BUILT or BSA_FLAG_CHECK_VALUES is set, before any device
 * work.  Allocates nothing
 * (no hipMalloc / hipFree / allocating library call). */
#define BSA_NOALLOC_SCRATCH_BYTES (16u << 20)
bsa_status_t bsa_fwd_noalloc(const bsa_problem_t* p, const void* q, const void* k, const void* v,
                             const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                             const int32_t* seqused_kv, const void* sparse, const int32_t* sparse_count,
                             const int32_t* block_table, void* out, float* lse, void* stream);

/* Stage 2, backward.  Inputs as bsa_fwd plus `out` and `lse` from the forward
 * pass and `dout` [T_q, N1, D].  Outputs dq [T_q, N1, D], dk and dv with k's
 * shape.  In the paged layout dk / dv are written at the (page, slot) of every
 * key below seqused_kv[b] of every sequence (zeros for keys no row attends)
 * and the rest of the page pool is left as it was; two sequences must not
 * share a page (their gradients would be written, not summed).  dQ is
 * computed by a separate Q-block-major pass (deterministic run to run)
 * unless BSA_FLAG_DQ_ATOMIC is set. */
bsa_status_t bsa_bwd(const bsa_problem_t* p, const void* q, const void* k, const void* v,
                     const void* out, const void* dout, const float* lse,
                     const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                     const int32_t* seqused_kv, const void* sparse, const int32_t* sparse_count,
                     const int32_t* block_table, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, void* stream);

/* The block index the passes build (the role of GenericBlockSparseAttention's
 * metadata pre-operator: a load-balanced schedule computed before the main
 * kernel).  bsa_build_index enqueues only the index construction into the
 * workspace; bsa_index_view says where each product sits.  Layout (all int32,
 * see the field comments):
 *   header[0..7]: totalQBlocks, totalKBlocks, R = Hs*totalQBlocks rows,
 *                 C = Hs*totalKBlocks columns, nnz, N2*totalKBlocks kv items,
 *                 0 (the value check word, see BSA_FLAG_CHECK_VALUES), 0
 *   row_ptr[R+1], cols[nnz]: per row r = hs*totalQBlocks + qbase_b + qb the
 *                 ascending local KV blocks holding at least one allowed pair
 *   work[R]:      rows by visited count descending, ties by row id
 *   with_csc != 0 adds
 *   col_ptr[C+1], qrows[nnz]: per column c = hs*totalKBlocks + kbase_b + kb the
 *                 ascending local q-blocks that visit it
 *   work_kv[N2*totalKBlocks]: items g*totalKBlocks + kbase_b + kb by the number
 *                 of (sparse head of group g, q-block) pairs reaching them,
 *                 descending, ties by item id.
 * Row tiles: when block_x is at most 32 and divides 128, block_y is a
 * multiple of 64 and ceil(max_seqlen_kv / block_y) <= 2048, the index groups the selection's q-blocks into tiles of
 * tile_rows = 128 query rows (tile t of sequence b holds q-blocks
 * t*128/block_x ..), and every "q-block" above is a tile: a tile visits the
 * union of its q-blocks' visited sets, and each CSR entry (and each CSC
 * entry, with_csc) carries a 128-bit row mask, uint32 [4] (bit i%32 of word
 * i/32: row i of the tile lies in one of the tile's q-blocks that visits the
 * entry's block).  The attention kernels then take whole tiles of rows as
 * work items instead of q-blocks of block_x rows, and mask per row.
 * The workspace needed is at most bsa_get_workspace_size's fwd_bytes
 * (with_csc == 0) or bwd_bytes (with_csc != 0). */
typedef struct bsa_index_view {
  uint64_t off_header, off_row_ptr, off_cols, off_work, off_col_ptr, off_qrows, off_work_kv;
  int64_t max_rows, max_cols, max_nnz, max_kv_items;
  int32_t tile_rows;  /* query rows per q-block of the index (block_x, or 128 with row tiles) */
  int32_t reserved;
  uint64_t off_row_mask, off_col_mask;  /* row tiles: uint32 [nnz][4] per CSR / CSC entry, else 0 */
} bsa_index_view_t;

bsa_status_t bsa_index_view(const bsa_problem_t* p, int with_csc, bsa_index_view_t* view);

bsa_status_t bsa_build_index(const bsa_problem_t* p, const int64_t* cu_seqlens_q,
                             const int64_t* cu_seqlens_kv, const int32_t* seqused_kv,
                             const void* sparse, const int32_t* sparse_count, int with_csc,
                             void* workspace, size_t workspace_bytes, void* stream);

/* A static string naming `s`. */
const char* bsa_status_string(bsa_status_t s);

/* Per-kernel timing with HIP events recorded on the launch stream, for
 * measurement tools.  While enabled (nonzero) every launch of the library's
 * kernels is bracketed by events; bsa_profile_read() synchronizes on the
 * recorded events and returns, for kernel id `kernel` (BSA_KERNEL_*), the
 * number of launches and their summed duration in milliseconds since the last
 * bsa_profile_reset().  Not for use while another thread calls the library. */
enum {
  BSA_KERNEL_INDEX = 0, /* all block-index kernels together */
  BSA_KERNEL_FWD = 1,
  BSA_KERNEL_BWD_PRE = 2,
  BSA_KERNEL_BWD_DKDV = 3,
  BSA_KERNEL_BWD_DQ = 4,
  BSA_KERNEL_COUNT = 5
};
bsa_status_t bsa_profile_enable(int enable);
bsa_status_t bsa_profile_reset(void);
bsa_status_t bsa_profile_read(int kernel, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* BSA_H_ */
