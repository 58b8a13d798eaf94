// Forward block-sparse varlen attention on gfx950.
//
// Computes O = softmax(scale * Q K_sel^T, mask) V_sel and lse over only the
// KV blocks each q-block selects (BlockSparseAttentionGrad README, forward
// formula; GenericBlockSparseAttention page, "Sparse attention mechanism"),
// with an fp32 online softmax and rescale (the pages' softmaxPrecision 0
// path) and the log-sum-exp produced in the same pass (BlitzSparseAttention
// page, "softmax_lse output").
//
// One workgroup (4 waves) per work item = one 128-row q-block of one q-head,
// taken longest-first from the index preprocessor's order.  Wave w owns query
// rows 32w .. 32w+31 and keeps its Q rows in registers.  The kernel walks the
// item's selected KV blocks in 64-key sub-tiles: K and V are staged through
// registers into double-buffered LDS (16-byte global loads, the next
// sub-tile's loads in flight while the current one is computed), then each
// wave computes
//   S^T = K Q^T           (MFMA 32x32x16, K read row-major from LDS)
//   online softmax        (each lane owns one query row: in-register max/sum,
//                          one cross-half exchange)
//   O^T += V^T P^T        (MFMA, V^T read with LDS transpose loads, P^T taken
//                          straight from the S^T accumulator registers)
// so no score ever leaves registers and the rescale by exp(m_old - m_new) is
// a per-lane multiply.
#include "bsa_attn.h"

namespace bsa {
namespace {

template <typename MF, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void k_fwd(FwdArgs a) {
  constexpr int TILE = KT * D * 2;  // bytes of one K or V sub-tile
  constexpr int NMT = D / 32;       // 32-row feature tiles of O^T
  constexpr int NKK = D / 16;       // contraction steps over D
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE];

  QItem it;
  if (!decode_qitem(blockIdx.x, a.hdr, a.work, a.qb_seq, a.qbase, a.seq, a.heads_per_row, a.group, it)) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int my_local = wv * 32 + (lane & 31);  // row within the item
  const int my_row = it.row_lo + my_local;     // row within the sequence
  const bool row_ok = my_local < it.nrows;
  const int qoff = it.skv - it.sq;             // causal: key j allowed for row i when j <= i + qoff
  int kend = it.skv;
  if (CAUSAL) kend = min(kend, it.row_lo + it.nrows - 1 + qoff + 1);

  // Q^T operand (B of S^T = K Q^T): lane holds row my_row, d = 16 kk + 8 (lane / 32) .. + 7
  const int64_t qstride = (int64_t)a.n1 * D;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (it.q0 + my_row) * qstride + (int64_t)it.h * D +
                       8 * (lane >> 5);
  u32x4_t qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = row_ok ? gload16(qp + 16 * kk) : zero_u4();

  const KvAddr ka = make_kv_addr(a.seq, a.block_table, it.b, it.g, a.n2, D, a.page_size, a.max_pages, a.page_stride);
  const uint16_t* kbase_p = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* vbase_p = reinterpret_cast<const uint16_t*>(a.v);

  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = zero16();
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.sigma_log2e;

  Stage<D, KT> sk, sv;
  SubTileWalk wk;
  wk.init(a.cols, a.row_ptr[it.r], a.row_ptr[it.r + 1], a.seq.by, kend);
  auto load = [&](int key0) {
    auto off = [&](int row) { return ka.offset(key0 + row); };
    auto ok = [&](int row) { return key0 + row < it.skv; };
    sk.load(kbase_p, off, ok);
    sv.load(vbase_p, off, ok);
  };
  if (wk.valid()) load(wk.key());
  int buf = 0;
  while (wk.valid()) {
    const int key0 = wk.key();
    char* kl = smem + buf * 2 * TILE;
    char* vl = kl + TILE;
    sk.store(kl);
    sv.store(vl);
    __syncthreads();
    wk.next();
    if (wk.valid()) load(wk.key());

    // ---- S^T = K Q^T for keys key0 .. key0+63 (two 32-key tiles) ----
    f32x16_t s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = zero16();
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) s[t] = MF::mfma(read_operand<D>(kl, 32 * t, kk), qf[kk], s[t]);
    }
    // ---- masks: keys past Skv, causal limit ----
    const bool edge = key0 + KT > it.skv || (CAUSAL && key0 + KT - 1 > it.row_lo + wv * 32 + qoff);
    if (edge) {
      const int lim = CAUSAL ? min(it.skv - 1, my_row + qoff) : it.skv - 1;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * t + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (key > lim) s[t][i] = -INFINITY;
        }
    }
    // ---- online softmax (row = this lane's column) ----
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
    mx = fmaxf(mx, wave_xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new * c2;
    const float alpha = fast_exp2(m_run * c2 - m_use);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[t][i], c2, -m_use));
        s[t][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[mt][i] *= alpha;
    // ---- O^T += V^T P^T ----
    u32x4_t pb[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) pb[kc] = pack8<MF>(s[kc >> 1], 8 * (kc & 1));
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) o[mt] = MF::mfma(read_tr_operand<D>(vl, 16 * kc, 32 * mt), pb[kc], o[mt]);
    buf ^= 1;
  }

  // ---- epilogue: O = O^T / l, lse = scale * m + ln l ----
  const float l_tot = l_run + wave_xor32(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (it.q0 + my_row) * qstride + (int64_t)it.h * D;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) store_cols<MF>(op, 32 * mt, o[mt], inv);
    if (lane < 32) {
      a.lse[(it.q0 + my_row) * a.n1 + it.h] =
          l_tot > 0.f ? m_run * a.sigma + fast_log2(l_tot) * 0.69314718055994531f : INFINITY;
    }
  }
}

template <typename MF, int D>
hipError_t launch_t(const FwdArgs& a, int64_t grid, hipStream_t st) {
  if (a.seq.causal)
    k_fwd<MF, D, true><<<(unsigned)grid, 256, 0, st>>>(a);
  else
    k_fwd<MF, D, false><<<(unsigned)grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int dtype, int head_dim, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  const bool bf = dtype == 2;
  if (head_dim == 128) return bf ? launch_t<BF16, 128>(a, grid, st) : launch_t<F16, 128>(a, grid, st);
  return bf ? launch_t<BF16, 64>(a, grid, st) : launch_t<F16, 64>(a, grid, st);
}

}  // namespace bsa
