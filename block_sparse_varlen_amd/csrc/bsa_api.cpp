// Host side of libbsa.so: descriptor checks, workspace planning and the
// enqueue sequence of each entry point declared in include/bsa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "../../include/bsa.h"
#include "bsa_internal.h"

using namespace bsa;

// Device scratch of bsa_fwd_noalloc: it stands in for the workspace argument
// (the block index) of callers that cannot allocate device memory.  Each GPU
// the library runs on holds its own copy for the life of the process.  In host
// code `scratch` is only a host-side handle of the symbol, never a device
// address: its address on a device comes from hipGetSymbolAddress (scratch_ptr).
static __device__ __align__(256) unsigned char scratch[BSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
bsa_status_t scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return BSA_ERR_RUNTIME;
  if (dev >= kMaxDevices) return BSA_ERR_INNER;
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&s]() { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  if (s.err != hipSuccess || !s.ptr) return BSA_ERR_RUNTIME;
  *out = s.ptr;
  return BSA_OK;
}

}  // namespace

namespace {

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
// grid sizes are padded to whole XCD rounds of 8 runs of 2^seg items (see
// xcd_item in bsa_attn.h)
int64_t xcd_grid(int64_t items, int seg) {
  const int64_t round = (int64_t)NUM_XCD << seg;
  return cdiv64(items, round) * round;
}
// XCD run lengths (log2).  Q-major launches (forward, dQ) keep runs of 32
// neighbouring q-blocks on one XCD, so they share K/V tiles in its L2, unless
// there are at most ~4 items per workgroup slot (2048 on 256 CUs at two
// workgroups each): then balance matters more than sharing and runs of 4
// spread the longest items over the XCDs.  The dK/dV items of one run share
// few Q/dO tiles, so they always take runs of 4.
int q_xseg(int64_t items) { return items <= 2048 ? 2 : 5; }
constexpr int KV_XSEG = 2;
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- checks --
bsa_status_t check_problem(const bsa_problem_t* p) {
  if (!p) return BSA_ERR_PARAM_NULLPTR;
  if (p->struct_size != sizeof(bsa_problem_t)) return BSA_ERR_PARAM_INVALID;
  if (p->dtype != BSA_DTYPE_F16 && p->dtype != BSA_DTYPE_BF16 && p->dtype != BSA_DTYPE_FP8_E4M3)
    return BSA_ERR_PARAM_INVALID;
  if (p->dtype == BSA_DTYPE_FP8_E4M3 ? (p->out_dtype != BSA_DTYPE_F16 && p->out_dtype != BSA_DTYPE_BF16)
                                     : (p->out_dtype != 0 && p->out_dtype != p->dtype))
    return BSA_ERR_PARAM_INVALID;
  if (p->head_dim != 64 && p->head_dim != 128) return BSA_ERR_PARAM_INVALID;
  if (p->batch < 0 || p->total_q < 0 || p->total_kv < 0) return BSA_ERR_PARAM_INVALID;
  if (p->max_seqlen_q < 0 || p->max_seqlen_kv < 0) return BSA_ERR_PARAM_INVALID;
  if (p->num_heads_q < 1 || p->num_heads_q > 256 || p->num_heads_kv < 1) return BSA_ERR_PARAM_INVALID;
  if (p->num_heads_q % p->num_heads_kv != 0 || p->num_heads_q / p->num_heads_kv > 128) return BSA_ERR_PARAM_INVALID;
  if (p->block_x <= 0 || p->block_y <= 0 || p->block_y % 16 != 0) return BSA_ERR_PARAM_INVALID;
  if (p->sparse_kind < BSA_SPARSE_NONE || p->sparse_kind > BSA_SPARSE_KV_IDX_BATCH_I32) return BSA_ERR_PARAM_INVALID;
  if (p->sparse_heads != p->num_heads_q && p->sparse_heads != p->num_heads_kv) return BSA_ERR_PARAM_INVALID;
  if (p->sparse_kind != BSA_SPARSE_NONE && (p->sparse_rows < 0 || p->sparse_width < 1)) return BSA_ERR_PARAM_INVALID;
  if ((p->sparse_kind == BSA_SPARSE_IDX_I32 || p->sparse_kind == BSA_SPARSE_IDX_BATCH_I32) && p->sparse_width > 256)
    return BSA_ERR_PARAM_INVALID;
  if (p->mask_type != BSA_MASK_NONE && p->mask_type != BSA_MASK_CAUSAL && p->mask_type != BSA_MASK_BAND)
    return BSA_ERR_PARAM_INVALID;
  if (p->kv_layout != BSA_KV_TND && p->kv_layout != BSA_KV_PAGED) return BSA_ERR_PARAM_INVALID;
  if (p->kv_layout == BSA_KV_PAGED) {
    const int64_t row = (int64_t)p->num_heads_kv * p->head_dim;
    if (p->page_size <= 0 || p->max_pages_per_seq < 0) return BSA_ERR_PARAM_INVALID;
    if ((int64_t)p->max_pages_per_seq * p->page_size < p->max_seqlen_kv) return BSA_ERR_PARAM_INVALID;
    if (p->page_stride < (int64_t)p->page_size * row || p->page_stride % row != 0) return BSA_ERR_PARAM_INVALID;
  }
  if (!(p->scale >= 0.0) || !std::isfinite(p->scale)) return BSA_ERR_PARAM_INVALID;
  if ((p->flags & ~(uint32_t)(BSA_FLAG_INDEX_BUILT | BSA_FLAG_DETERMINISTIC | BSA_FLAG_DQ_ATOMIC |
                             BSA_FLAG_CHECK_VALUES)) != 0)
    return BSA_ERR_PARAM_INVALID;
  if ((p->flags & BSA_FLAG_DETERMINISTIC) && (p->flags & BSA_FLAG_DQ_ATOMIC)) return BSA_ERR_PARAM_INVALID;
  // valid descriptors without a compiled variant
  if (p->block_x > 4096) return BSA_ERR_INNER;
  if (p->dtype == BSA_DTYPE_FP8_E4M3 && p->head_dim != 128) return BSA_ERR_INNER;
  if (p->block_y > 4096) return BSA_ERR_INNER;
  if (p->kv_layout == BSA_KV_PAGED && p->page_size % 64 != 0) return BSA_ERR_INNER;
  if ((int64_t)p->max_seqlen_kv > (int64_t)p->block_y * 65536 || (int64_t)p->max_seqlen_q > (int64_t)p->block_x * 65536)
    return BSA_ERR_INNER;
  return BSA_OK;
}

bsa_status_t check_bwd_variant(const bsa_problem_t* p) {
  if (p->dtype == BSA_DTYPE_FP8_E4M3) return BSA_ERR_INNER;  // forward-only quantisation
  return BSA_OK;
}

// Whether q-blocks are grouped into row tiles (SeqArgs): narrow q-blocks that
// divide the tile, a block_y the kernels walk in whole 64-key sub-tiles, and
// KV blocks few enough for the mask builder's LDS.
bool row_tiles(const bsa_problem_t* p) {
  return p->block_x <= ROW_TILE_MAX_BX && ROW_TILE % p->block_x == 0 && p->block_y % 64 == 0 &&
         cdiv64(p->max_seqlen_kv, p->block_y) <= ROW_TILE_MAX_KB;
}
// query rows per q-block of the index and of the work items
int32_t item_rows(const bsa_problem_t* p) { return row_tiles(p) ? ROW_TILE : p->block_x; }

// Sparse heads per dispatch chunk of the forward and dQ passes.  Rows whose
// K/V are read at random (sparse selections over long sequences) re-read
// them from memory many times; when the K/V of all heads exceed the 256 MiB
// last-level cache, the Q-major passes take their rows head chunk by head
// chunk (longest-first inside each chunk), the largest power-of-two number
// of heads whose K/V fit in that cache, so the re-reads hit it.  Returns
// sparse_heads (one chunk) otherwise.
int32_t q_chunk_heads(const bsa_problem_t* p) {
  constexpr int64_t kLastLevelCache = 256ll << 20;
  const int64_t tokens = p->kv_layout == BSA_KV_PAGED ? p->total_kv * p->page_size : p->total_kv;
  const int64_t elem = p->dtype == BSA_DTYPE_FP8_E4M3 ? 1 : 2;
  const int64_t per_head = tokens * p->num_heads_kv * p->head_dim * 2 * elem / std::max(p->sparse_heads, 1);
  if (per_head <= 0) return std::max(p->sparse_heads, 1);
  int64_t fit = kLastLevelCache / per_head, c = 1;
  while (c * 2 <= fit) c *= 2;
  return (int32_t)std::min<int64_t>(c, std::max(p->sparse_heads, 1));
}

Bounds make_bounds(const bsa_problem_t* p) {
  Bounds b{};
  const int64_t B = p->batch;
  const int32_t bx = item_rows(p);
  b.nqb_max = (int32_t)cdiv64(p->max_seqlen_q, bx);
  b.nkb_max = (int32_t)cdiv64(p->max_seqlen_kv, p->block_y);
  b.qbar = std::min<int64_t>(p->total_q / bx + B, B * b.nqb_max);
  b.qbar_sel = std::max<int64_t>(
      std::min<int64_t>(p->total_q / p->block_x + B, B * cdiv64(p->max_seqlen_q, p->block_x)), 1);
  if (p->kv_layout == BSA_KV_PAGED)
    b.kbar = B * b.nkb_max;
  else
    b.kbar = std::min<int64_t>(p->total_kv / p->block_y + B, B * b.nkb_max);
  b.qbar = std::max<int64_t>(b.qbar, 1);
  b.kbar = std::max<int64_t>(b.kbar, 1);
  b.rbar = (int64_t)p->sparse_heads * b.qbar;
  b.cbar = (int64_t)p->sparse_heads * b.kbar;
  const int64_t nkb = std::max<int32_t>(b.nkb_max, 1);
  // per-KV-block lists may select every KV block for one q-block, and a row
  // tile's union any block
  const bool all_kb = p->sparse_kind == BSA_SPARSE_NONE || kv_lists(p->sparse_kind) || row_tiles(p);
  b.cmax = (int32_t)(all_kb ? nkb : std::min<int64_t>(p->sparse_width, nkb));
  b.nnzbar = std::max<int64_t>(b.rbar * b.cmax, 1);
  b.kvbar = (int64_t)p->num_heads_kv * b.kbar;
  const int group = p->num_heads_q / p->num_heads_kv;
  b.kvkey_max = (p->sparse_heads == p->num_heads_q ? group : 1) * std::max<int32_t>(b.nqb_max, 1);
  b.q_chunk_heads = q_chunk_heads(p);
  return b;
}

// dQ by fp32 atomics inside the dK/dV kernel (else the separate pass)
bool dq_atomic(const bsa_problem_t* p) { return (p->flags & BSA_FLAG_DQ_ATOMIC) != 0; }

// 32-bit words of one row's visited-block bitmap
int64_t kv_words(const Bounds& b) { return std::max<int64_t>((b.nkb_max + 31) / 32, 1); }

bool bounds_fit(const Bounds& b) {
  const int64_t lim = (int64_t)1 << 30;
  return b.rbar < lim && b.cbar < lim && b.nnzbar < lim && b.kvbar < lim;
}

Layout make_layout(const bsa_problem_t* p, const Bounds& b, bool with_csc, bool with_dl) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + std::max<size_t>(bytes, 4));
    return o;
  };
  const size_t B = (size_t)p->batch;
  L.hdr = take(H_COUNT * 4);
  L.sq = take(B * 4);
  L.skv = take(B * 4);
  L.qbase = take((B + 1) * 4);
  L.kbase = take((B + 1) * 4);
  L.qb_seq = take((size_t)b.qbar * 4);
  L.kb_seq = take((size_t)b.kbar * 4);
  L.row_cnt = take((size_t)b.rbar * 4);
  L.row_ptr = take((size_t)(b.rbar + 1) * 4);
  L.cols = take((size_t)b.nnzbar * 4);
  // sized for both sorts whatever with_csc is, so the forward products sit at
  // the same offsets in the forward and the backward layout (an index built
  // for the backward pass serves a forward call too)
  const int64_t nsort = std::max<int64_t>(b.rbar, b.kvbar);
  L.key0 = take((size_t)nsort * 4);
  L.val0 = take((size_t)nsort * 4);
  L.key1 = take((size_t)nsort * 4);
  L.val1 = take((size_t)nsort * 4);
  // one radix sort's histograms, or both work lists' side by side
  L.hist = take((size_t)(256 * (cdiv64(b.rbar, 256) + cdiv64(b.kvbar, 256)) + 2) * 4);
  L.work = take((size_t)b.rbar * 4);
  L.work_q = take((size_t)b.rbar * 4);
  // per-KV-block lists are scattered into per-row bitmaps first (rows of
  // selection q-blocks)
  L.kvbm = kv_lists(p->sparse_kind) ? take((size_t)p->sparse_heads * b.qbar_sel * kv_words(b) * 4) : 0;
  if (row_tiles(p)) {
    L.qbase_sel = take((B + 1) * 4);
    L.row_mask = take((size_t)b.nnzbar * 16);
  }
  if (with_csc) {
    L.col_cnt = take((size_t)b.cbar * 4);
    L.col_ptr = take((size_t)(b.cbar + 1) * 4);
    L.col_fill = take((size_t)b.cbar * 4);
    L.qrows = take((size_t)b.nnzbar * 4);
    L.work_kv = take((size_t)b.kvbar * 4);
    if (row_tiles(p)) L.col_mask = take((size_t)b.nnzbar * 16);
  }
  L.index_end = off;
  if (with_dl) {
    L.ndl = take((size_t)p->total_q * p->num_heads_q * 4);
    L.lse2 = take((size_t)p->total_q * p->num_heads_q * 4);
    if (dq_atomic(p)) L.dq_acc = take((size_t)p->total_q * p->num_heads_q * p->head_dim * 4);
  }
  L.total = off;
  return L;
}

IndexPtrs make_ptrs(void* ws, const Layout& L, bool with_csc, bool tiles) {
  char* w = static_cast<char*>(ws);
  auto at = [&](size_t o) { return reinterpret_cast<int32_t*>(w + o); };
  IndexPtrs ip{};
  ip.hdr = at(L.hdr);
  ip.sq = at(L.sq);
  ip.skv = at(L.skv);
  ip.qbase = at(L.qbase);
  ip.kbase = at(L.kbase);
  ip.qb_seq = at(L.qb_seq);
  ip.kb_seq = at(L.kb_seq);
  ip.row_cnt = at(L.row_cnt);
  ip.row_ptr = at(L.row_ptr);
  ip.cols = at(L.cols);
  ip.key0 = at(L.key0);
  ip.val0 = at(L.val0);
  ip.key1 = at(L.key1);
  ip.val1 = at(L.val1);
  ip.hist = at(L.hist);
  ip.work = at(L.work);
  ip.work_q = at(L.work_q);
  if (with_csc) {
    ip.col_cnt = at(L.col_cnt);
    ip.col_ptr = at(L.col_ptr);
    ip.col_fill = at(L.col_fill);
    ip.qrows = at(L.qrows);
    ip.work_kv = at(L.work_kv);
  }
  if (tiles) {
    ip.qbase_sel = at(L.qbase_sel);
    ip.row_mask = reinterpret_cast<uint32_t*>(w + L.row_mask);
    if (with_csc) ip.col_mask = reinterpret_cast<uint32_t*>(w + L.col_mask);
  }
  return ip;
}

SeqArgs make_seq(const bsa_problem_t* p, const int64_t* cu_q, const int64_t* cu_kv, const int32_t* seqused) {
  SeqArgs s{};
  s.cu_q = cu_q;
  s.cu_kv = p->kv_layout == BSA_KV_PAGED ? nullptr : cu_kv;
  s.seqused_kv = p->kv_layout == BSA_KV_PAGED ? seqused : nullptr;
  s.batch = p->batch;
  s.bx = item_rows(p);
  s.sel_bx = p->block_x;
  s.by = p->block_y;
  s.masked = p->mask_type != BSA_MASK_NONE;
  auto clampw = [](int64_t x) { return (int32_t)std::max<int64_t>(-WIN_INF, std::min<int64_t>(WIN_INF, x)); };
  if (p->mask_type == BSA_MASK_BAND) {
    s.win_lo = -clampw(p->pre_tokens);
    s.win_hi = clampw(p->next_tokens);
  } else {
    s.win_lo = -WIN_INF;
    s.win_hi = 0;
  }
  return s;
}

SelArgs make_sel(const bsa_problem_t* p, const void* sparse, const int32_t* count, void* ws, const Layout& L,
                 const Bounds& b) {
  SelArgs s{};
  if (kv_lists(p->sparse_kind)) {
    s.kvbm = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + L.kvbm);
    s.kv_words = (int32_t)kv_words(b);
  }
  s.sparse = sparse;
  s.count = count;
  s.kind = p->sparse_kind;
  s.hs = p->sparse_heads;
  s.rows = p->sparse_kind == BSA_SPARSE_NONE ? 0 : p->sparse_rows;
  s.width = p->sparse_kind == BSA_SPARSE_NONE ? 0 : p->sparse_width;
  return s;
}

float sigma_of(const bsa_problem_t* p) {
  const double s = p->scale != 0.0 ? p->scale : 1.0 / std::sqrt((double)p->head_dim);
  return (float)s;
}

bsa_status_t check_index_ptrs(const bsa_problem_t* p, const int64_t* cu_q, const int64_t* cu_kv,
                              const int32_t* seqused, const void* sparse, const int32_t* count) {
  if (!cu_q) return BSA_ERR_PARAM_NULLPTR;
  if (p->kv_layout == BSA_KV_TND && !cu_kv) return BSA_ERR_PARAM_NULLPTR;
  if (p->kv_layout == BSA_KV_PAGED && !seqused) return BSA_ERR_PARAM_NULLPTR;
  if (p->sparse_kind != BSA_SPARSE_NONE && !sparse) return BSA_ERR_PARAM_NULLPTR;
  if (p->sparse_kind >= BSA_SPARSE_IDX_I32 && !count) return BSA_ERR_PARAM_NULLPTR;
  return BSA_OK;
}

bsa_status_t from_hip(hipError_t e) { return e == hipSuccess ? BSA_OK : BSA_ERR_RUNTIME; }

// BSA_FLAG_CHECK_VALUES: checks the device-resident sequence description
// with one kernel and waits for its word (the one call path that synchronizes
// the stream), before any kernel that trusts those values is enqueued.
// block_table may be NULL (index-only calls read no page).
bsa_status_t check_values(const bsa_problem_t* p, const int64_t* cu_q, const int64_t* cu_kv,
                          const int32_t* seqused, const int32_t* block_table, int32_t* hdr, hipStream_t s) {
  const bool paged = p->kv_layout == BSA_KV_PAGED;
  CheckArgs c{};
  c.cu_q = cu_q;
  c.cu_kv = paged ? nullptr : cu_kv;
  c.seqused_kv = paged ? seqused : nullptr;
  c.block_table = paged ? block_table : nullptr;
  c.batch = p->batch;
  c.max_sq = p->max_seqlen_q;
  c.max_skv = p->max_seqlen_kv;
  c.page_size = paged ? p->page_size : 0;
  c.max_pages = paged ? p->max_pages_per_seq : 0;
  c.total_q = p->total_q;
  c.total_kv = p->total_kv;
  if (launch_check_values(c, hdr, s) != hipSuccess) return BSA_ERR_RUNTIME;
  int32_t word = -1;
  if (hipMemcpyAsync(&word, hdr + H_CHECK, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess)
    return BSA_ERR_RUNTIME;
  if (hipStreamSynchronize(s) != hipSuccess) return BSA_ERR_RUNTIME;
  return word == 0 ? BSA_OK : BSA_ERR_PARAM_INVALID;
}

// ------------------------------------------------------------- profiling --
struct ProfRec {
  int kernel;
  hipEvent_t start, stop;
};
struct ProfState {
  std::mutex mu;
  bool enabled = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  int64_t launches[BSA_KERNEL_COUNT] = {};
  double total_ms[BSA_KERNEL_COUNT] = {};
  hipEvent_t pending_start[BSA_KERNEL_COUNT] = {};
};
ProfState& prof() {
  static ProfState s;
  return s;
}
hipEvent_t prof_event(ProfState& s) {
  if (!s.pool.empty()) {
    hipEvent_t e = s.pool.back();
    s.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
void prof_drain(ProfState& s) {
  for (auto& r : s.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      s.launches[r.kernel] += 1;
      s.total_ms[r.kernel] += ms;
    }
    s.pool.push_back(r.start);
    s.pool.push_back(r.stop);
  }
  s.recs.clear();
}

bsa_status_t fwd_impl(const bsa_problem_t* p, const void* q, const void* k, const void* v, const int64_t* cu_q,
                     const int64_t* cu_kv, const int32_t* seqused, const void* sparse, const int32_t* count,
                     const int32_t* block_table, void* out, float* lse, void* workspace, size_t ws_bytes,
                     void* stream) {
  bsa_status_t st = check_problem(p);
  if (st != BSA_OK) return st;
  const Bounds b = make_bounds(p);
  if (!bounds_fit(b)) return BSA_ERR_PARAM_INVALID;
  const Layout L = make_layout(p, b, false, false);
  if (p->batch == 0 || p->total_q == 0) return BSA_OK;
  if (!q || !out || !lse) return BSA_ERR_PARAM_NULLPTR;
  if (p->total_kv > 0 && (!k || !v)) return BSA_ERR_PARAM_NULLPTR;
  st = check_index_ptrs(p, cu_q, cu_kv, seqused, sparse, count);
  if (st != BSA_OK) return st;
  if (p->kv_layout == BSA_KV_PAGED && !block_table) return BSA_ERR_PARAM_NULLPTR;
  if (!workspace) return BSA_ERR_PARAM_NULLPTR;
  if (ws_bytes < L.total) return BSA_ERR_PARAM_INVALID;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const IndexPtrs ip = make_ptrs(workspace, L, false, row_tiles(p));
  if (p->flags & BSA_FLAG_CHECK_VALUES) {
    st = check_values(p, cu_q, cu_kv, seqused, block_table, ip.hdr, s);
    if (st != BSA_OK) return st;
  }
  const int group = p->num_heads_q / p->num_heads_kv;
  const SeqArgs seq = make_seq(p, cu_q, cu_kv, seqused);
  hipError_t e = hipSuccess;
  if (!(p->flags & BSA_FLAG_INDEX_BUILT)) {
    prof_begin(BSA_KERNEL_INDEX, s);
    e = launch_index(seq, make_sel(p, sparse, count, workspace, L, b), b, ip, p->num_heads_kv, group, false, s);
    prof_end(BSA_KERNEL_INDEX, s);
    if (e != hipSuccess) return BSA_ERR_RUNTIME;
  }

  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.seq = seq;
  a.block_table = block_table;
  a.hdr = ip.hdr;
  a.qb_seq = ip.qb_seq;
  a.qbase = ip.qbase;
  a.row_ptr = ip.row_ptr;
  a.cols = ip.cols;
  a.work = b.q_chunk_heads < p->sparse_heads ? ip.work_q : ip.work;
  // row tiles without a selection need no row masks: a row's token window
  // already removes every block its own q-block does not visit
  a.row_mask = p->sparse_kind != BSA_SPARSE_NONE ? ip.row_mask : nullptr;
  a.n1 = p->num_heads_q;
  a.n2 = p->num_heads_kv;
  a.group = group;
  a.heads_per_row = p->sparse_heads == p->num_heads_q ? 1 : group;
  a.page_size = p->kv_layout == BSA_KV_PAGED ? p->page_size : 0;
  a.max_pages = p->kv_layout == BSA_KV_PAGED ? p->max_pages_per_seq : 0;
  a.page_stride = p->kv_layout == BSA_KV_PAGED ? p->page_stride : 0;
  a.sigma = sigma_of(p);
  a.sigma_log2e = a.sigma * 1.4426950408889634f;
  const int64_t items = b.rbar * a.heads_per_row * cdiv64(item_rows(p), 128);
  a.xseg = q_xseg(items);
  prof_begin(BSA_KERNEL_FWD, s);
  const int64_t grid = xcd_grid(items, a.xseg);
  e = p->dtype == BSA_DTYPE_FP8_E4M3 ? launch_fwd_fp8(a, p->out_dtype, grid, s)
                                     : launch_fwd(a, p->dtype, p->head_dim, grid, s);
  prof_end(BSA_KERNEL_FWD, s);
  return from_hip(e);
}

}  // namespace

namespace bsa {
void prof_begin(int kernel, hipStream_t st) {
  ProfState& s = prof();
  if (!s.enabled) return;
  std::lock_guard<std::mutex> g(s.mu);
  hipEvent_t e = prof_event(s);
  if (e && hipEventRecord(e, st) == hipSuccess) s.pending_start[kernel] = e;
}
void prof_end(int kernel, hipStream_t st) {
  ProfState& s = prof();
  if (!s.enabled) return;
  std::lock_guard<std::mutex> g(s.mu);
  hipEvent_t b = s.pending_start[kernel];
  if (!b) return;
  s.pending_start[kernel] = nullptr;
  hipEvent_t e = prof_event(s);
  if (e && hipEventRecord(e, st) == hipSuccess) s.recs.push_back({kernel, b, e});
}
}  // namespace bsa

extern "C" {

const char* bsa_status_string(bsa_status_t s) {
  switch (s) {
    case BSA_OK: return "BSA_OK";
    case BSA_ERR_PARAM_NULLPTR: return "BSA_ERR_PARAM_NULLPTR: a required pointer is NULL";
    case BSA_ERR_PARAM_INVALID: return "BSA_ERR_PARAM_INVALID: unsupported descriptor or workspace too small";
    case BSA_ERR_INNER: return "BSA_ERR_INNER: no compiled kernel variant for this descriptor";
    case BSA_ERR_RUNTIME: return "BSA_ERR_RUNTIME: HIP launch or runtime error";
  }
  return "unknown bsa_status_t";
}

bsa_status_t bsa_get_workspace_size(const bsa_problem_t* p, size_t* fwd_bytes, size_t* bwd_bytes) {
  if (!p || (!fwd_bytes && !bwd_bytes)) return BSA_ERR_PARAM_NULLPTR;
  bsa_status_t st = check_problem(p);
  if (st != BSA_OK) return st;
  const Bounds b = make_bounds(p);
  if (!bounds_fit(b)) return BSA_ERR_PARAM_INVALID;
  if (bwd_bytes) {
    st = check_bwd_variant(p);
    if (st != BSA_OK) return st;
    *bwd_bytes = make_layout(p, b, true, true).total;
  }
  if (fwd_bytes) *fwd_bytes = make_layout(p, b, false, false).total;
  return BSA_OK;
}

bsa_status_t bsa_index_view(const bsa_problem_t* p, int with_csc, bsa_index_view_t* v) {
  if (!p || !v) return BSA_ERR_PARAM_NULLPTR;
  const bsa_status_t st = check_problem(p);
  if (st != BSA_OK) return st;
  const Bounds b = make_bounds(p);
  if (!bounds_fit(b)) return BSA_ERR_PARAM_INVALID;
  const Layout L = make_layout(p, b, with_csc != 0, false);
  v->off_header = L.hdr;
  v->off_row_ptr = L.row_ptr;
  v->off_cols = L.cols;
  v->off_work = L.work;
  v->off_col_ptr = with_csc ? L.col_ptr : 0;
  v->off_qrows = with_csc ? L.qrows : 0;
  v->off_work_kv = with_csc ? L.work_kv : 0;
  v->max_rows = b.rbar;
  v->max_cols = with_csc ? b.cbar : 0;
  v->max_nnz = b.nnzbar;
  v->max_kv_items = with_csc ? b.kvbar : 0;
  v->tile_rows = item_rows(p);
  v->reserved = 0;
  v->off_row_mask = row_tiles(p) ? L.row_mask : 0;
  v->off_col_mask = row_tiles(p) && with_csc ? L.col_mask : 0;
  return BSA_OK;
}

bsa_status_t bsa_build_index(const bsa_problem_t* p, const int64_t* cu_q, const int64_t* cu_kv,
                             const int32_t* seqused, const void* sparse, const int32_t* count, int with_csc,
                             void* workspace, size_t ws_bytes, void* stream) {
  bsa_status_t st = check_problem(p);
  if (st != BSA_OK) return st;
  const Bounds b = make_bounds(p);
  if (!bounds_fit(b)) return BSA_ERR_PARAM_INVALID;
  const Layout L = make_layout(p, b, with_csc != 0, false);
  if (p->batch == 0) return BSA_OK;
  st = check_index_ptrs(p, cu_q, cu_kv, seqused, sparse, count);
  if (st != BSA_OK) return st;
  if (!workspace) return BSA_ERR_PARAM_NULLPTR;
  if (ws_bytes < L.total) return BSA_ERR_PARAM_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const IndexPtrs ip = make_ptrs(workspace, L, with_csc != 0, row_tiles(p));
  if (p->flags & BSA_FLAG_CHECK_VALUES) {
    st = check_values(p, cu_q, cu_kv, seqused, nullptr, ip.hdr, s);
    if (st != BSA_OK) return st;
  }
  prof_begin(BSA_KERNEL_INDEX, s);
  const hipError_t e = launch_index(make_seq(p, cu_q, cu_kv, seqused), make_sel(p, sparse, count, workspace, L, b), b, ip,
                                    p->num_heads_kv, p->num_heads_q / p->num_heads_kv, with_csc != 0, s);
  prof_end(BSA_KERNEL_INDEX, s);
  return from_hip(e);
}

bsa_status_t bsa_fwd(const bsa_problem_t* p, const void* q, const void* k, const void* v, const int64_t* cu_q,
                     const int64_t* cu_kv, const int32_t* seqused, const void* sparse, const int32_t* count,
                     const int32_t* block_table, void* out, float* lse, void* workspace, size_t ws_bytes,
                     void* stream) {
  return fwd_impl(p, q, k, v, cu_q, cu_kv, seqused, sparse, count, block_table, out, lse, workspace, ws_bytes,
                  stream);
}

bsa_status_t bsa_fwd_noalloc(const bsa_problem_t* p, const void* q, const void* k, const void* v,
                             const int64_t* cu_q, const int64_t* cu_kv, const int32_t* seqused, const void* sparse,
                             const int32_t* count, const int32_t* block_table, void* out, float* lse,
                             void* stream) {
  bsa_status_t st = check_problem(p);
  if (st != BSA_OK) return st;
  // the index of this entry point lives in the library's scratch array, so a
  // prebuilt one cannot be handed in
  if (p->flags & BSA_FLAG_INDEX_BUILT) return BSA_ERR_PARAM_INVALID;
  // nor can it wait for a value check (its callers may be capturing a graph)
  if (p->flags & BSA_FLAG_CHECK_VALUES) return BSA_ERR_PARAM_INVALID;
  const Bounds b = make_bounds(p);
  if (!bounds_fit(b)) return BSA_ERR_PARAM_INVALID;
  const size_t need = make_layout(p, b, false, false).total;
  if (need > (size_t)BSA_NOALLOC_SCRATCH_BYTES) return BSA_ERR_PARAM_INVALID;
  if (p->batch == 0 || p->total_q == 0) return BSA_OK;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != BSA_OK) return st;
  return fwd_impl(p, q, k, v, cu_q, cu_kv, seqused, sparse, count, block_table, out, lse, ws,
                  (size_t)BSA_NOALLOC_SCRATCH_BYTES, stream);
}

bsa_status_t bsa_bwd(const bsa_problem_t* p, const void* q, const void* k, const void* v, const void* out,
                     const void* dout, const float* lse, const int64_t* cu_q, const int64_t* cu_kv,
                     const int32_t* seqused, const void* sparse, const int32_t* count, const int32_t* block_table,
                     void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes, void* stream) {
  bsa_status_t st = check_problem(p);
  if (st != BSA_OK) return st;
  st = check_bwd_variant(p);
  if (st != BSA_OK) return st;
  const Bounds b = make_bounds(p);
  if (!bounds_fit(b)) return BSA_ERR_PARAM_INVALID;
  const Layout L = make_layout(p, b, true, true);
  if (p->batch == 0 || (p->total_q == 0 && p->total_kv == 0)) return BSA_OK;
  if (p->total_q > 0 && (!q || !out || !dout || !lse || !dq)) return BSA_ERR_PARAM_NULLPTR;
  if (p->total_kv > 0 && (!k || !v || !dk || !dv)) return BSA_ERR_PARAM_NULLPTR;
  st = check_index_ptrs(p, cu_q, cu_kv, seqused, sparse, count);
  if (st != BSA_OK) return st;
  if (p->kv_layout == BSA_KV_PAGED && !block_table) return BSA_ERR_PARAM_NULLPTR;
  if (!workspace) return BSA_ERR_PARAM_NULLPTR;
  if (ws_bytes < L.total) return BSA_ERR_PARAM_INVALID;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const IndexPtrs ip = make_ptrs(workspace, L, true, row_tiles(p));
  if (p->flags & BSA_FLAG_CHECK_VALUES) {
    st = check_values(p, cu_q, cu_kv, seqused, block_table, ip.hdr, s);
    if (st != BSA_OK) return st;
  }
  const int group = p->num_heads_q / p->num_heads_kv;
  const SeqArgs seq = make_seq(p, cu_q, cu_kv, seqused);
  hipError_t e = hipSuccess;
  if (!(p->flags & BSA_FLAG_INDEX_BUILT)) {
    prof_begin(BSA_KERNEL_INDEX, s);
    e = launch_index(seq, make_sel(p, sparse, count, workspace, L, b), b, ip, p->num_heads_kv, group, true, s);
    prof_end(BSA_KERNEL_INDEX, s);
    if (e != hipSuccess) return BSA_ERR_RUNTIME;
  }

  float* ndl = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.ndl);
  float* lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lse2);
  float* acc = dq_atomic(p) ? reinterpret_cast<float*>(static_cast<char*>(workspace) + L.dq_acc) : nullptr;
  // (the atomic dQ accumulator is cleared by k_bwd_pre, a kernel rather than
  // a memset, so the call can be captured in a HIP graph)
  BwdPreArgs pa{out, dout, lse, ndl, lse2, acc, p->total_q * p->num_heads_q};
  prof_begin(BSA_KERNEL_BWD_PRE, s);
  e = launch_bwd_pre(pa, p->dtype, p->head_dim, s);
  prof_end(BSA_KERNEL_BWD_PRE, s);
  if (e != hipSuccess) return BSA_ERR_RUNTIME;

  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.lse2 = lse2;
  a.ndl = ndl;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dq_acc = acc;
  a.seq = seq;
  a.hdr = ip.hdr;
  a.qb_seq = ip.qb_seq;
  a.kb_seq = ip.kb_seq;
  a.qbase = ip.qbase;
  a.kbase = ip.kbase;
  a.row_ptr = ip.row_ptr;
  a.cols = ip.cols;
  a.work = b.q_chunk_heads < p->sparse_heads ? ip.work_q : ip.work;  // the dQ pass's row order
  a.col_ptr = ip.col_ptr;
  a.qrows = ip.qrows;
  a.work_kv = ip.work_kv;
  a.row_mask = p->sparse_kind != BSA_SPARSE_NONE ? ip.row_mask : nullptr;
  a.col_mask = p->sparse_kind != BSA_SPARSE_NONE ? ip.col_mask : nullptr;
  a.block_table = block_table;
  a.page_size = p->kv_layout == BSA_KV_PAGED ? p->page_size : 0;
  a.max_pages = p->kv_layout == BSA_KV_PAGED ? p->max_pages_per_seq : 0;
  a.page_stride = p->kv_layout == BSA_KV_PAGED ? p->page_stride : 0;
  a.n1 = p->num_heads_q;
  a.n2 = p->num_heads_kv;
  a.group = group;
  a.heads_per_row = p->sparse_heads == p->num_heads_q ? 1 : group;
  a.hs = p->sparse_heads;
  a.sub_tiles = (p->block_y + 127) / 128;
  a.sigma = sigma_of(p);
  a.sigma_log2e = a.sigma * 1.4426950408889634f;
  const int64_t q_items = b.rbar * a.heads_per_row * cdiv64(item_rows(p), 128);
  const int64_t kv_items = b.kvbar * a.sub_tiles;
  a.xseg_q = q_xseg(q_items);
  a.xseg_kv = KV_XSEG;
  if (p->total_kv > 0) {
    prof_begin(BSA_KERNEL_BWD_DKDV, s);
    e = launch_bwd_dkdv(a, p->dtype, p->head_dim, xcd_grid(kv_items, a.xseg_kv), s);
    prof_end(BSA_KERNEL_BWD_DKDV, s);
    if (e != hipSuccess) return BSA_ERR_RUNTIME;
  }
  if (p->total_q > 0) {
    prof_begin(BSA_KERNEL_BWD_DQ, s);
    if (acc)
      e = launch_dq_convert(acc, dq, p->total_q * p->num_heads_q * p->head_dim, a.sigma, p->dtype, s);
    else
      e = launch_bwd_dq(a, p->dtype, p->head_dim, xcd_grid(q_items, a.xseg_q), s);
    prof_end(BSA_KERNEL_BWD_DQ, s);
  }
  return from_hip(e);
}

bsa_status_t bsa_profile_enable(int enable) {
  ProfState& s = prof();
  std::lock_guard<std::mutex> g(s.mu);
  s.enabled = enable != 0;
  return BSA_OK;
}

bsa_status_t bsa_profile_reset(void) {
  ProfState& s = prof();
  std::lock_guard<std::mutex> g(s.mu);
  prof_drain(s);
  for (int i = 0; i < BSA_KERNEL_COUNT; ++i) {
    s.launches[i] = 0;
    s.total_ms[i] = 0.0;
  }
  return BSA_OK;
}

bsa_status_t bsa_profile_read(int kernel, int64_t* launches, double* total_ms) {
  if (!launches || !total_ms) return BSA_ERR_PARAM_NULLPTR;
  if (kernel < 0 || kernel >= BSA_KERNEL_COUNT) return BSA_ERR_PARAM_INVALID;
  ProfState& s = prof();
  std::lock_guard<std::mutex> g(s.mu);
  prof_drain(s);
  *launches = s.launches[kernel];
  *total_ms = s.total_ms[kernel];
  return BSA_OK;
}

}  // extern "C"
