// Forward block-sparse varlen attention on gfx950.
//
// Computes O = softmax(scale * Q K_sel^T, mask) V_sel and lse over only the
// KV blocks each q-block selects (BlockSparseAttentionGrad README, forward
// formula; GenericBlockSparseAttention page, "Sparse attention mechanism"),
// with an fp32 online softmax and rescale (the pages' softmaxPrecision 0
// path) and the log-sum-exp produced in the same pass (BlitzSparseAttention
// page, "softmax_lse output").
//
// One workgroup (4 waves) per work item = up to 128 rows of one q-block of
// one q-head, taken longest-first from the index preprocessor's order.  Wave w
// owns query rows 32w .. 32w+31 and keeps its Q rows in registers.  The kernel
// walks the item's selected KV blocks in 64-key sub-tiles: K and V are copied
// straight from global memory into double-buffered LDS (direct-to-LDS loads,
// the next sub-tile's copies in flight while the current one is computed),
// then each wave computes
//   S^T = K Q^T           (MFMA 32x32x16, K read row-major from LDS)
//   online softmax        (each lane owns one query row: in-register max/sum,
//                          one cross-half exchange)
//   O^T += V^T P^T        (MFMA, V^T read with LDS transpose loads, P^T taken
//                          straight from the S^T accumulator registers)
// so no score ever leaves registers and the rescale by exp(m_old - m_new) is
// a per-lane multiply.
#include <type_traits>

#include "bsa_attn.h"

namespace bsa {
namespace {

// Softmax rescale threshold (log2 units): the running maximum used for the
// exponentials is only moved when a row's new maximum exceeds it by more than
// this, so exp2 arguments stay <= RESCALE_LOG2 (P <= 256) and the O^T rescale
// is skipped for most sub-tiles.  Any reference maximum gives the same O and
// lse; only the rounding differs.
constexpr float RESCALE_LOG2 = 8.f;

template <typename MF, int D, int WMODE, bool PAGED>
__global__ __launch_bounds__(256, 2) void k_fwd(FwdArgs a) {
  // K is read row-major only (XOR-permuted chunks), V transposed only (rows
  // padded by 64 bytes): both layouts keep their read pattern conflict free
  // and both split into whole direct-to-LDS load instructions per wave.
  using KL = XorTile<D>;
  using VL = PadTile<D, 64>;
  constexpr int KTILE = KL::template bytes<KT>();
  constexpr int VTILE = VL::template bytes<KT>();
  constexpr int STAGE = KTILE + VTILE;
  constexpr int NMT = D / 32;  // 32-row feature tiles of O^T
  constexpr int NKK = D / 16;  // contraction steps over D
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  QItem it;
  if (!decode_qitem(xcd_item(blockIdx.x, a.xseg), a.hdr, a.work, a.qb_seq, a.qbase, a.seq, a.heads_per_row, a.group,
                   it))
    return;
  const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int my_local = wv * 32 + (lane & 31);  // row within the item
  const int my_row = it.row_lo + my_local;     // row within the sequence
  const bool row_ok = my_local < it.nrows;
  // a wave whose 32 rows all lie past the item's rows (short q-blocks, the
  // sequence end) only helps with the copies and the barriers
  const bool wave_active = wv * 32 < it.nrows;
  // with a token window (causal or band mask) key j is allowed for row i when
  // i + qoff + win_lo <= j <= i + qoff + win_hi; WMODE 1 has no lower end
  // (causal, or a band with unbounded preTokens), WMODE 2 has both
  constexpr bool WIN = WMODE != 0, LO = WMODE == 2;
  const int qoff = it.skv - it.sq;
  const int win_lo = a.seq.win_lo, win_hi = a.seq.win_hi;
  int kend = it.skv, kstart = 0;
  if (WIN) {
    kend = min(kend, it.row_lo + it.nrows - 1 + qoff + win_hi + 1);
    if (LO) kstart = max(0, it.row_lo + qoff + win_lo);
  }

  // Q^T operand (B of S^T = K Q^T): lane holds row my_row, d = 16 kk + 8 (lane / 32) .. + 7
  const int64_t qstride = (int64_t)a.n1 * D;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (it.q0 + my_row) * qstride + (int64_t)it.h * D +
                       8 * (lane >> 5);
  u32x4_t qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = row_ok ? gload16(qp + 16 * kk) : zero_u4();

  const uint16_t* kbase_p = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* vbase_p = reinterpret_cast<const uint16_t*>(a.v);

  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = zero16();
  float m_run = -INFINITY;  // reference maximum of this lane's row (raw scores)
  float l_run = 0.f;        // this lane's partial row sum relative to m_run
  const float c2 = a.sigma_log2e;
  const float thresh = RESCALE_LOG2 / c2;

  DmaTile<KL, D, KT> kdma;
  DmaTile<VL, D, KT> vdma;
  kdma.init(a.n2 * D);
  vdma.init(a.n2 * D);
  Operands<KL, D> ofk;
  Operands<VL, D> ofv;
  ofk.init();
  ofv.init();
  // `ld` walks the sub-tiles and loads each one a step before it is computed
  // (LDS double buffer); key_next is the first key of the last one issued
  RegTileWalk<> ld;
  ld.init(a.cols, ldu(a.row_ptr, it.r), ldu(a.row_ptr, it.r + 1), a.seq.by, kend, kstart);
  KvAddr<PAGED> kva;
  kva.init(a.seq, a.block_table, it.b, it.g, a.n2, D, a.page_size, a.max_pages, a.page_stride);
  int key_next = 0;
  uint32_t gm_next = 0xFu;  // selected 16-key groups of that sub-tile
  // row tiles: this wave's 32 rows' bits of that sub-tile's row mask
  uint32_t rm_next = 0xFFFFFFFFu;
  // the first sub-tile goes out before the block list register has landed
  auto issue = [&](int stage, auto first) {
    char* st = smem + stage * STAGE;
    const int key0 = ld.template take<decltype(first)::value>();
    key_next = key0;
    gm_next = ld.gmask;
    if (a.row_mask) rm_next = ldu(a.row_mask, (int64_t)ld.ent * 4 + wv);
    const int64_t off = kva.off(key0);
    kdma.issue(st, kbase_p + off, it.skv - key0);
    vdma.issue(st + KTILE, vbase_p + off, it.skv - key0);
  };
  bool more = ld.valid();
  if (more) issue(0, std::true_type{});
  int stage = 0;
  while (more) {
    const int key0 = key_next;     // the sub-tile computed in this step
    const uint32_t gm = gm_next;   // its 16-key groups in selected blocks
    const uint32_t rm = rm_next;   // its row mask bits of this wave's rows
    wait_vmcnt<0>();               // this wave's loads of the current sub-tile landed
    __builtin_amdgcn_s_barrier();  // everyone's did, and the other buffer is free
    more = ld.valid();
    if (more) issue(stage ^ 1, std::false_type{});
    settle_scalar_loads();
    const int rw0 = it.row_lo + wv * 32 + qoff;  // this wave's first row, shifted to its diagonal key
    // a wave leaves out sub-tiles that no row of it may attend: all keys past
    // its last row's window end or before its first row's window start (their
    // scores would all be masked, so nothing changes), and with row tiles the
    // blocks no row of it selects
    if (!wave_active || rm == 0u || (WIN && key0 > rw0 + 31 + win_hi) || (LO && key0 + KT - 1 < rw0 + win_lo)) {
      stage ^= 1;
      continue;
    }
    const char* kl = smem + stage * STAGE;
    const char* vl = kl + KTILE;

    // ---- S^T = K Q^T for keys key0 .. key0+63 (two 32-key tiles) ----
    f32x16_t s[2];
    s[0] = zero16();
    s[1] = zero16();
    // step i: kk = i / 2, key tile t = i % 2
    mfma_pipeline<2 * NKK, 4>([&](int i) { return read_operand(kl, ofk, 32 * (i & 1), i >> 1); },
                              [&](int i, const u32x4_t& op) { s[i & 1] = MF::mfma(op, qf[i >> 1], s[i & 1]); });
    // ---- masks: keys past Skv, outside the rows' windows (edge sub-tiles only) ----
    const bool edge = key0 + KT > it.skv || gm != 0xFu || rm != 0xFFFFFFFFu ||
                      (WIN && key0 + KT - 1 > rw0 + win_hi) || (LO && key0 < rw0 + 31 + win_lo);
    if (edge) {
      const int lim = WIN ? min(it.skv - 1, my_row + qoff + win_hi) : it.skv - 1;
      const int lo = LO ? my_row + qoff + win_lo : 0;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * t + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (key > lim || (LO && key < lo)) s[t][i] = -INFINITY;
        }
      if (gm != 0xFu) {  // 16-key groups outside the selected blocks (block_y not a multiple of 64)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!((gm >> (2 * t + (i >> 3))) & 1u)) s[t][i] = -INFINITY;
      }
      if (!((rm >> (lane & 31)) & 1u)) {  // row tiles: this row's q-block does not visit the block
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[t][i] = -INFINITY;
      }
    }
    // ---- online softmax (row = this lane's column) ----
    const float mx = half_max(max32(s[0], s[1]));
    // move the reference maximum only when it is exceeded by more than the threshold
    const bool upd = mx > m_run + thresh || (m_run == -INFINITY && mx > -INFINITY);
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float m_new = upd ? mx : m_run;
      const float alpha = upd ? fast_exp2((m_run - m_new) * c2) : 1.f;  // m_run = -inf -> 0
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[mt][i] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run * c2;
    float ps[4];  // independent partial sums (short dependency chains)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[t][i], c2, -m_use));
        s[t][i] = p;
        if (t == 0 && i < 4)
          ps[i] = p;
        else
          ps[i & 3] += p;
      }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // ---- O^T += V^T P^T ----
    u32x4_t pb[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) pb[kc] = pack8<MF>(s[kc >> 1], 8 * (kc & 1));
    // step i: kc = i / NMT, mt = i % NMT
    mfma_pipeline<4 * NMT, 4>([&](int i) { return read_tr_operand(vl, ofv, 16 * (i / NMT), i % NMT); },
                              [&](int i, const u32x4_t& op) { o[i % NMT] = MF::mfma(op, pb[i / NMT], o[i % NMT]); });
    stage ^= 1;
  }

  // ---- epilogue: O = O^T / l, lse = scale * m + ln l ----
  // The two half-waves share m_run (the maximum is exchanged before use), so
  // their partial sums add directly.
  const float l_tot = half_sum(l_run);
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

template <typename MF, int D, bool PAGED>
hipError_t launch_t(const FwdArgs& a, int64_t grid, hipStream_t st) {
  switch (window_mode(a.seq)) {
    case 0: k_fwd<MF, D, 0, PAGED><<<(unsigned)grid, 256, 0, st>>>(a); break;
    case 1: k_fwd<MF, D, 1, PAGED><<<(unsigned)grid, 256, 0, st>>>(a); break;
    default: k_fwd<MF, D, 2, PAGED><<<(unsigned)grid, 256, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

template <typename MF, int D>
hipError_t launch_p(const FwdArgs& a, int64_t grid, hipStream_t st) {
  return a.seq.seqused_kv ? launch_t<MF, D, true>(a, grid, st) : launch_t<MF, D, false>(a, grid, st);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int dtype, int head_dim, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  const bool bf = dtype == 2;
  if (head_dim == 128) return bf ? launch_p<BF16, 128>(a, grid, st) : launch_p<F16, 128>(a, grid, st);
  return bf ? launch_p<BF16, 64>(a, grid, st) : launch_p<F16, 64>(a, grid, st);
}

}  // namespace bsa
