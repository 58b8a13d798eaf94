// Backward block-sparse varlen attention on gfx950 (BlockSparseAttentionGrad
// README, backward formulas):
//   softmax_grad D_i = rowsum(dO o O)             -> k_bwd_pre
//   P = exp(scale * Q K^T - lse), dP = dO V^T, dS = P o (dP - D)
//   dV = P^T dO,  dK = scale * dS^T Q             -> k_bwd_dkdv (KV-major)
//   dQ = scale * dS K                             -> k_bwd_dq   (Q-major)
// The softmax is not recomputed: P comes from the forward pass's lse, as the
// FlashAttention UnpaddingScoreGradV2 page describes its backward consuming
// the forward's softmax statistics.
//
// dK/dV are owner-computed: one workgroup per 128-key tile of one KV head,
// looping over the q-heads of its GQA group and the q-blocks that selected
// the tile (the transposed, per-KV-block index lists).  dQ comes either from
// a separate Q-block-major pass over the forward's per-q-block lists (no
// atomics, deterministic run to run), or from the dK/dV kernel itself, which
// adds each stage's dS K into an fp32 accumulator with atomics that a last
// kernel scales and converts (the order of the additions, and so the last
// bits, vary from run to run).
#include <type_traits>

#include "bsa_attn.h"

namespace bsa {
namespace {

constexpr float LOG2E = 1.4426950408889634f;

// ------------------------------------------------------------- D = dO.O --
// One 16-byte chunk per thread, D/8 threads per (token, head) row.  D is
// stored negated: the dP accumulators of the other two kernels start from
// -D, so their MFMAs produce dP - D directly.
template <typename MF, int D>
__global__ __launch_bounds__(256) void k_bwd_pre(BwdPreArgs a) {
  constexpr int CH = D / 8;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / CH;
  const int c = threadIdx.x % CH;
  // Every lane issues its three loads up front, unconditionally (lanes past
  // the last row read row 0), so they are in flight together instead of the
  // second waiting behind the first.
  const int64_t rr = row < a.rows ? row : 0;
  const u32x4_t o = gload16(reinterpret_cast<const uint16_t*>(a.out) + rr * D + c * 8);
  const u32x4_t d = gload16(reinterpret_cast<const uint16_t*>(a.dout) + rr * D + c * 8);
  float l = a.lse[rr];
  pin(l);
  float acc = MF::lo(o.x) * MF::lo(d.x) + MF::hi(o.x) * MF::hi(d.x) + MF::lo(o.y) * MF::lo(d.y) +
              MF::hi(o.y) * MF::hi(d.y) + MF::lo(o.z) * MF::lo(d.z) + MF::hi(o.z) * MF::hi(d.z) +
              MF::lo(o.w) * MF::lo(d.w) + MF::hi(o.w) * MF::hi(d.w);
#pragma unroll
  for (int m = CH / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < a.rows && c == 0) {
    a.ndl[row] = -acc;
    a.lse2[row] = l * LOG2E;
  }
  if (a.dq_acc && row < a.rows) {  // clear this chunk of the atomic dQ accumulator
    float4* z = reinterpret_cast<float4*>(a.dq_acc + row * D + c * 8);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// dq = scale * acc, 8 elements per thread
template <typename MF>
__global__ __launch_bounds__(256) void k_dq_convert(const float* acc, uint16_t* dq, int64_t n8, float sigma) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 x = reinterpret_cast<const float4*>(acc)[2 * i];
  const float4 y = reinterpret_cast<const float4*>(acc)[2 * i + 1];
  u32x4_t r;
  r.x = MF::pack(x.x * sigma, x.y * sigma);
  r.y = MF::pack(x.z * sigma, x.w * sigma);
  r.z = MF::pack(y.x * sigma, y.y * sigma);
  r.w = MF::pack(y.z * sigma, y.w * sigma);
  reinterpret_cast<u32x4_t*>(dq)[i] = r;
}

// -------------------------------------------------------------------- dQ --
// Same work items and key walk as the forward kernel.  Per 64-key sub-tile:
//   S^T = K Q^T, dP^T = V dO^T            (K, V row-major from LDS)
//   P^T = exp2(S^T scale log2e - lse log2e), dS^T = P^T o (dP^T - D)
//   dQ^T += K^T dS^T                       (K^T via LDS transpose loads)
// The dP^T accumulator starts from -D (a loop-invariant register tile), and
// key masks run only on sub-tiles that reach past Skv or outside a row's window.

template <typename MF, int D, int WMODE, bool PAGED>
__global__ __launch_bounds__(256, 2) void k_bwd_dq(BwdArgs a) {
  using L = XorTile<D>;  // K: read row-major (S^T) and transposed (dQ^T); V: row-major (dP^T)
  constexpr int TILE = L::template bytes<KT>();
  constexpr int STAGE = 2 * TILE;
  constexpr int NMT = D / 32;
  constexpr int NKK = D / 16;
  using Dma = DmaTile<L, D, KT>;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];  // double buffer

  QItem it;
  if (!decode_qitem(xcd_item(blockIdx.x, a.xseg_q), a.hdr, a.work, a.qb_seq, a.qbase, a.seq, a.heads_per_row,
                   a.group, it))
    return;
  const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int my_local = wv * 32 + (lane & 31);
  const int my_row = it.row_lo + my_local;
  const bool row_ok = my_local < it.nrows;
  // a wave whose 32 rows all lie past the item's rows only helps with the
  // copies and the barriers
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

  const int64_t qstride = (int64_t)a.n1 * D;
  const int64_t tok = it.q0 + my_row;
  const int64_t qoffs = tok * qstride + (int64_t)it.h * D + 8 * (lane >> 5);
  u32x4_t qf[NKK], df[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qf[kk] = row_ok ? gload16(reinterpret_cast<const uint16_t*>(a.q) + qoffs + 16 * kk) : zero_u4();
    df[kk] = row_ok ? gload16(reinterpret_cast<const uint16_t*>(a.dout) + qoffs + 16 * kk) : zero_u4();
  }
  const float lse2 = row_ok ? a.lse[tok * a.n1 + it.h] * LOG2E : INFINITY;
  // -D of this lane's row in every element: the start value of each dP^T tile
  f32x16_t ndt;
  {
    const float nd = row_ok ? a.ndl[tok * a.n1 + it.h] : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ndt[i] = nd;
  }

  const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.v);
  f32x16_t acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) acc[mt] = zero16();
  const float c2 = a.sigma_log2e;
  const int lim = WIN ? min(it.skv - 1, my_row + qoff + win_hi) : it.skv - 1;
  const int lo = LO ? my_row + qoff + win_lo : 0;

  Dma dma;
  dma.init(a.n2 * D);
  Operands<L, D> of;
  of.init();
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
    dma.issue(st, kp + off, it.skv - key0);
    dma.issue(st + TILE, vp + off, it.skv - key0);
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
    const char* vl = kl + TILE;
    const bool edge = key0 + KT > it.skv || gm != 0xFu || rm != 0xFFFFFFFFu ||
                      (WIN && key0 + KT - 1 > rw0 + win_hi) || (LO && key0 < rw0 + 31 + win_lo);
#pragma unroll
    for (int t = 0; t < 2; ++t) {  // 32-key halves of the sub-tile
      f32x16_t s = zero16(), dp = ndt;
      // step i: kk = i / 2; even = S^T (K rows), odd = dP^T (V rows)
      mfma_pipeline<2 * NKK, 4>([&](int i) { return read_operand((i & 1) ? vl : kl, of, 32 * t, i >> 1); },
                                [&](int i, const u32x4_t& op) {
                                  if (i & 1)
                                    dp = MF::mfma(op, df[i >> 1], dp);
                                  else
                                    s = MF::mfma(op, qf[i >> 1], s);
                                });
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = fast_exp2(fmaf(s[i], c2, -lse2));
      if (edge) {  // keys past Skv or outside this row's window
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * t + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (key > lim || (LO && key < lo)) s[i] = 0.f;
        }
        if (gm != 0xFu) {  // 16-key groups outside the selected blocks (block_y not a multiple of 64)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!((gm >> (2 * t + (i >> 3))) & 1u)) s[i] = 0.f;
        }
        if (!((rm >> (lane & 31)) & 1u)) {  // row tiles: this row's q-block does not visit the block
#pragma unroll
          for (int i = 0; i < 16; ++i) s[i] = 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] *= dp[i];  // dS^T = P^T o (dP^T - D)
      const u32x4_t db0 = pack8<MF>(s, 0), db1 = pack8<MF>(s, 8);
      // step i: kc = 2 t + i / NMT, mt = i % NMT
      mfma_pipeline<2 * NMT, 4>(
          [&](int i) { return read_tr_operand(kl, of, 16 * (2 * t + i / NMT), i % NMT); },
          [&](int i, const u32x4_t& op) { acc[i % NMT] = MF::mfma(op, (i < NMT) ? db0 : db1, acc[i % NMT]); });
    }
    stage ^= 1;
  }
  if (row_ok) {
    uint16_t* op = reinterpret_cast<uint16_t*>(a.dq) + tok * qstride + (int64_t)it.h * D;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) store_cols<MF>(op, 32 * mt, acc[mt], a.sigma);
  }
}

// ----------------------------------------------------------------- dK, dV --
// Work item: one 128-key tile of KV block (g, b, kb), taken by a workgroup of
// NW waves; wave w owns NT 32-key tiles (keys 32 NT w ..) and keeps their K
// and V rows in registers as the B operands of S = Q K^T and dP = dO V^T.  For
// every q-head of the group and every q-block in the tile's transposed list,
// 64-row query sub-tiles of Q, dO, lse and D are staged through
// double-buffered LDS and each wave computes, per 32-row half,
//   S, dP                (MFMA, Q / dO row-major from LDS)
//   P = exp2(S scale log2e - lse log2e), dS = P o (dP - D)
//   dV^T += dO^T P,  dK^T += Q^T dS   (Q^T / dO^T via LDS transpose loads,
//                                      P / dS straight from registers)
// Every operand read from LDS feeds the MFMAs of the wave's NT key tiles; dK
// and dV accumulate in AGPRs.
constexpr int QS = 64;  // query rows per staged sub-tile

// Walk over (q-head of the group, q-block of the tile's column list, 64-row
// part of the q-block: ceil(block_x / 64) of them, the last one short when
// block_x is not a multiple of 64), skipping parts past the sequence end or
// whose rows' windows miss the tile.
struct ColWalk {
  const int32_t* col_ptr;
  const int32_t* qrows;
  int hh, e, e1, half;
  int group, per_head, g, tkb, kg, sq, qoff, key_min, key_max, win, win_lo, win_hi, bx, halves;  // halves = ceil(bx / QS)
  __device__ __forceinline__ int col(int h) const { return (per_head ? g * group + h : g) * tkb + kg; }
  // a part is skipped when its last row's window ends below the tile's first
  // key or its first row's window starts above the tile's last key
  __device__ __forceinline__ bool ok(int qb, int hf) const {
    const int r0 = qb * bx + hf * QS;
    if (r0 >= sq) return false;
    if (win && min(min(r0 + QS, (qb + 1) * bx), sq) - 1 + qoff + win_hi < key_min) return false;
    if (win && r0 + qoff + win_lo > key_max) return false;
    return true;
  }
  __device__ __forceinline__ void open(int h) {
    const int c = col(h);
    e = ldu(col_ptr, c);
    e1 = ldu(col_ptr, c + 1);
  }
  __device__ __forceinline__ void settle() {
    while (hh < group) {
      while (e < e1) {
        const int qb = ldu(qrows, e);
        while (half < halves) {
          if (ok(qb, half)) return;
          ++half;
        }
        ++e;
        half = 0;
      }
      ++hh;
      if (hh < group) open(hh);
    }
  }
  __device__ __forceinline__ bool valid() const { return hh < group; }
  __device__ __forceinline__ void next() {
    ++half;
    settle();
  }
  __device__ __forceinline__ int row0() const { return ldu(qrows, e) * bx + half * QS; }
  // end of the current part's rows: the q-block's end or the sequence end
  __device__ __forceinline__ int row_end() const { return min((ldu(qrows, e) + 1) * bx, sq); }
};

constexpr int DKDV_KEYS = 128;  // keys per work item
constexpr int DKDV_STAGES = 2;  // LDS ring depth

// Workgroup shape of the dK/dV kernel: NW waves of NT 32-key tiles.  Two
// waves of 64 keys, two workgroups per CU (one wave per SIMD): each Q / dO
// operand read from LDS feeds two MFMAs.  Four waves of 32 keys (two waves
// per SIMD, so one wave's softmax could hide behind the other's MFMAs) need
// ~280 registers at D = 128 against the 256 a wave then gets; the spilled
// build was 22 % slower, so both head dims use the 64-key waves.
//
// With atomic dQ (DQA) the kernel also forms dQ += dS K per stage, which
// needs dS with the query rows on the lanes and K with the features on the
// lanes -- both transposed from what the dK/dV products hold -- so K and
// each half's dS go through LDS (32 + 2 x 12 KiB), and one workgroup of four
// 32-key waves takes a CU.
template <int D, bool DQA>
struct DkdvShape {
  static constexpr int NT = DQA ? 1 : 2, NW = DQA ? 4 : 2, LOOK = 4;
  static_assert(!DQA || D / 32 <= NW, "atomic dQ: one feature tile per wave");
};
// dS tile of the atomic dQ: rows = the item's 128 keys, columns = a half's
// 32 query rows, rows padded by 32 bytes (transposed reads of 4 rows x 32
// bytes land on distinct banks)
using DsTile = PadTile<32, 32>;
constexpr int DS_BYTES = DsTile::bytes<DKDV_KEYS>();

template <typename MF, int D, int WMODE, bool PAGED, bool DQA>
__global__ __launch_bounds__((64 * DkdvShape<D, DQA>::NW), 1) void k_bwd_dkdv(BwdArgs a) {
  constexpr int NT = DkdvShape<D, DQA>::NT;
  constexpr int NW = DkdvShape<D, DQA>::NW;
  constexpr int LOOK = DkdvShape<D, DQA>::LOOK;  // MFMA operands read this many steps ahead
  static_assert(32 * NT * NW == DKDV_KEYS, "a workgroup covers the 128-key tile");
  constexpr bool WIN = WMODE != 0, LO = WMODE == 2;  // token window; LO: with a lower end
  using QL = XorTile<D>;  // Q and dO: read row-major (S, dP) and transposed (dK^T, dV^T)
  constexpr int TILE = QL::template bytes<QS>();
  constexpr int STAGE = 2 * TILE + 2 * QS * 4;  // Q, dO, lse, D
  constexpr int NMT = D / 32;
  constexpr int NKK = D / 16;
  using Dma = DmaXor<D, QS, NW>;
  constexpr int KT_BYTES = DQA ? QL::template bytes<DKDV_KEYS>() : 0;  // atomic dQ: K of the item
  __shared__ __attribute__((aligned(16))) char smem[DKDV_STAGES * STAGE + (DQA ? KT_BYTES + 2 * DS_BYTES : 0)];

  const int KVI = ldu(a.hdr, H_KVITEMS);
  const int64_t flat = xcd_item(blockIdx.x, a.xseg_kv);
  const int64_t item = flat / a.sub_tiles;
  const int sub = (int)(flat - item * a.sub_tiles);
  if (item >= KVI) return;
  const int TKB = ldu(a.hdr, H_TKB);
  const int w_id = ldu(a.work_kv, item);
  const int g = w_id / TKB, kg = w_id - g * TKB;
  const int b = ldu(a.kb_seq, kg);
  const int kb = kg - ldu(a.kbase, b);
  const int64_t q0 = ldu(a.seq.cu_q, b);
  const int sq = (int)(ldu(a.seq.cu_q, b + 1) - q0);
  // Rows of this tile's keys: packed rows kv0 + key, or (page, slot) through
  // the block table (looked up per lane: a tile may span pages).
  int64_t kv0 = 0;
  int skv;
  if constexpr (PAGED) {
    skv = ldu(a.seq.seqused_kv, b);
  } else {
    kv0 = ldu(a.seq.cu_kv, b);
    skv = (int)(ldu(a.seq.cu_kv, b + 1) - kv0);
  }
  const int key_lo = kb * a.seq.by + sub * DKDV_KEYS;
  // keys of this item: the tile's part of block kb below Skv.  A block_y
  // that is not a multiple of 128 leaves the block's last tile partial: its
  // other keys (the next block's) are computed -- dK / dV columns do not mix
  // -- but never stored.
  const int kcap = min(skv, (kb + 1) * a.seq.by);
  if (key_lo >= kcap) return;
  const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // this lane's keys: column lane % 32 of the wave's 32-key tiles
  const int key_w = key_lo + 32 * NT * wv + (lane & 31);
  const int qoff = skv - sq;
  const int win_lo = a.seq.win_lo, win_hi = a.seq.win_hi;
  const int64_t kvstride = (int64_t)a.n2 * D;
  // element offset of key `key` (< skv) of this tile, head g, column 0
  auto key_row = [&](int key) -> int64_t {
    if constexpr (PAGED) {
      const int64_t page = a.block_table[(int64_t)b * a.max_pages + key / a.page_size];
      return page * a.page_stride + (int64_t)(key % a.page_size) * kvstride + (int64_t)g * D;
    } else {
      return (kv0 + key) * kvstride + (int64_t)g * D;
    }
  };
  u32x4_t kf[NT][NKK], vf[NT][NKK];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int key = key_w + 32 * n;
    const int64_t krow = (PAGED && key >= skv ? 0 : key_row(key)) + 8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      kf[n][kk] = key < skv ? gload16(reinterpret_cast<const uint16_t*>(a.k) + krow + 16 * kk) : zero_u4();
      vf[n][kk] = key < skv ? gload16(reinterpret_cast<const uint16_t*>(a.v) + krow + 16 * kk) : zero_u4();
    }
  }
  char* const kt = smem + DKDV_STAGES * STAGE;  // atomic dQ: K rows of the item's keys
  char* const dsbuf = kt + KT_BYTES;             // atomic dQ: two dS tiles
  Operands<DsTile, 32> dsof;
  if constexpr (DQA) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      lds_write16(kt, QL::chunk_off(32 * NT * wv + (lane & 31), 2 * kk + (lane >> 5)), kf[0][kk]);
    dsof.init();
    __syncthreads();
  }
  f32x16_t dk[NT][NMT], dv[NT][NMT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      dk[n][mt] = zero16();
      dv[n][mt] = zero16();
    }
  const float c2 = a.sigma_log2e;
  const int qstride = a.n1 * D;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* dop = reinterpret_cast<const uint16_t*>(a.dout);

  // `ld` walks the (head, q-block, half) sequence and loads each tile a step
  // before it is computed; r0_next is the first row of the last one issued.
  ColWalk ld;
  ld.col_ptr = a.col_ptr;
  ld.qrows = a.qrows;
  ld.group = a.group;
  ld.per_head = a.hs == a.n1;
  ld.g = g;
  ld.tkb = TKB;
  ld.kg = kg;
  ld.sq = sq;
  ld.qoff = qoff;
  ld.key_min = key_lo;
  ld.key_max = min(key_lo + DKDV_KEYS, kcap) - 1;
  ld.win = WIN;  // (win_lo is -WIN_INF without a lower end, so ok() needs no mode)
  ld.win_lo = a.seq.win_lo;
  ld.win_hi = a.seq.win_hi;
  ld.bx = a.seq.bx;
  ld.halves = (a.seq.bx + QS - 1) / QS;
  ld.hh = 0;
  ld.half = 0;
  ld.open(0);
  ld.settle();
  int r0_next = 0, rend_next = 0, hh_next = 0;
  uint64_t cm_next = ~0ull;  // row tiles: mask bits of that tile's 64 rows (CSC entry, half)

  Dma dma;
  dma.init(qstride);
  XorOperands<D> of;
  of.init();
  auto issue = [&](int stage) {
    char* st = smem + stage * STAGE;
    const int h = g * a.group + ld.hh;
    const int r0 = ld.row0();
    r0_next = r0;
    rend_next = ld.row_end();
    hh_next = ld.hh;
    if (a.col_mask) {
      const int64_t mo = (int64_t)ld.e * 4 + 2 * ld.half;
      cm_next = (uint64_t)ldu(a.col_mask, mo) | ((uint64_t)ldu(a.col_mask, mo + 1) << 32);
    }
    const int nvalid = sq - r0;
    const int64_t off = (q0 + r0) * (int64_t)qstride + (int64_t)h * D;
    dma.issue(st, qp + off, nvalid);
    dma.issue(st + TILE, dop + off, nvalid);
    float* stat = reinterpret_cast<float*>(st + 2 * TILE);
    // lse (wave 0) and -D (wave 1) of the tile's rows
    if (wv < 2) dma_rows_f32(stat + wv * QS, (wv == 0 ? a.lse2 : a.ndl) + (q0 + r0) * a.n1 + h, a.n1, nvalid);
    ld.next();
  };

  bool more = ld.valid();
  if (more) issue(0);
  int stage = 0;
  while (more) {
    const int r0 = r0_next;            // the tile computed in this step
    const int nrows = rend_next - r0;  // its rows inside the q-block and the sequence (may exceed QS)
    const int hh_cur = hh_next;        // its q-head within the group
    const uint64_t cm = cm_next;       // row tiles: its rows' mask bits
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // every wave's loads landed; the other stage is no longer read
    more = ld.valid();
    if (more) issue(stage ^ 1);
    settle_scalar_loads();
    of.refresh();
    char* ql = smem + stage * STAGE;
    char* dl_ = ql + TILE;
    const float* lsel = reinterpret_cast<const float*>(ql + 2 * TILE);
    const float* ndll = lsel + QS;

    // Rows past the q-block or sequence end, or keys outside some row's
    // window, need masks; every other tile takes the mask-free path.
    // (atomic dQ also masks the keys of a partial tile past the block end:
    // their dS would reach dQ)
    const bool masked = nrows < QS || (WIN && key_lo + DKDV_KEYS - 1 > r0 + qoff + win_hi) ||
                        (LO && key_lo < r0 + QS - 1 + qoff + win_lo) || (DQA && key_lo + DKDV_KEYS > kcap) ||
                        cm != ~0ull;
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // 32-row halves of the tile
      // dP starts from -D of each element's row, so the MFMAs leave dP - D
      f32x16_t s[NT], dp[NT];
      {
        f32x16_t ndt;
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const u32x4_t d4 = *reinterpret_cast<const u32x4_t*>(ndll + 32 * h + 8 * ig + 4 * (lane >> 5));
#pragma unroll
          for (int j = 0; j < 4; ++j) ndt[4 * ig + j] = __uint_as_float(d4[j]);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          s[n] = zero16();
          dp[n] = ndt;
        }
      }
      // S, dP of rows 32 h .. + 31: each Q / dO operand read feeds the NT key tiles
      mfma_pipeline<2 * NKK, LOOK>([&](int i) { return read_operand((i & 1) ? dl_ : ql, of, 32 * h, i >> 1); },
                                [&](int i, const u32x4_t& op) {
#pragma unroll
                                  for (int n = 0; n < NT; ++n) {
                                    if (i & 1)
                                      dp[n] = MF::mfma(op, vf[n][i >> 1], dp[n]);
                                    else
                                      s[n] = MF::mfma(op, kf[n][i >> 1], s[n]);
                                  }
                                });
      // P = exp2(S scale log2e - lse log2e), dS = P o (dP - D)
      u32x4_t pb[NT][2], db[NT][2];
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int rl = 32 * h + 8 * ig + 4 * (lane >> 5);  // first of 4 consecutive query rows
        const u32x4_t l4 = *reinterpret_cast<const u32x4_t*>(lsel + rl);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * ig + j;
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const float p = fast_exp2(fmaf(s[n][i], c2, -__uint_as_float(l4[j])));
            s[n][i] = p;
            dp[n][i] *= p;
          }
        }
      }
      if (masked) {  // edge tiles only: P = dS = 0 past the sequence end or outside the window
        // row tiles: bit 8 (i / 4) + i % 4 of lm is the mask bit of element i's row
        const uint32_t lm = (uint32_t)(cm >> (32 * h)) >> (4 * (lane >> 5));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rl = 32 * h + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const int kd = key_w + 32 * n - (r0 + rl + qoff);  // key minus the row's diagonal key
            if ((WIN && kd > win_hi) || (LO && kd < win_lo) || rl >= nrows || (DQA && key_w + 32 * n >= kcap) ||
                !((lm >> (8 * (i >> 2) + (i & 3))) & 1u)) {
              s[n][i] = 0.f;
              dp[n][i] = 0.f;
            }
          }
        }
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        pb[n][0] = pack8<MF>(s[n], 0);
        pb[n][1] = pack8<MF>(s[n], 8);
        db[n][0] = pack8<MF>(dp[n], 0);
        db[n][1] = pack8<MF>(dp[n], 8);
      }
      // dV^T += dO^T P, dK^T += Q^T dS over the 16-row chunks 2 h, 2 h + 1;
      // each transposed operand read feeds the NT key tiles
      mfma_pipeline<4 * NMT, LOOK>(
          [&](int i) { return read_tr_operand((i & 1) ? ql : dl_, of, 16 * (2 * h + i / (2 * NMT)), (i >> 1) % NMT); },
          [&](int i, const u32x4_t& op) {
            const int c = i / (2 * NMT);
            const int mt = (i >> 1) % NMT;
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              if (i & 1)
                MF::mfma_acc(dk[n][mt], op, db[n][c]);
              else
                MF::mfma_acc(dv[n][mt], op, pb[n][c]);
            }
          });
      if constexpr (DQA) {
        // dS of this wave's keys into the half's LDS tile [key][query row]:
        // db[0][c] holds rows 16 c + 4 (lane / 32) + 0..3 and + 8 + 0..3
        char* dsb = dsbuf + h * DS_BYTES;
        const int krow = 32 * wv + (lane & 31);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          u32x2_t lo2, hi2;
          lo2.x = db[0][c].x;
          lo2.y = db[0][c].y;
          hi2.x = db[0][c].z;
          hi2.y = db[0][c].w;
          *reinterpret_cast<u32x2_t*>(dsb + DsTile::col_off(krow, 16 * c + 4 * (lane >> 5))) = lo2;
          *reinterpret_cast<u32x2_t*>(dsb + DsTile::col_off(krow, 16 * c + 8 + 4 * (lane >> 5))) = hi2;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the writes landed
        __builtin_amdgcn_s_barrier();        // every wave's keys are in
        // dQ (32 rows x 32 features 32 wv ..) += dS (rows x 128 keys) K (keys x features)
        // wave wv takes feature tile wv (D = 64 has two: waves 2, 3 only
        // take part in the barriers); all 16 operands are read first
        // (registers are plentiful at one workgroup per CU)
        if (wv < NMT) {
          u32x4_t opa[DKDV_KEYS / 16], opb[DKDV_KEYS / 16];
#pragma unroll
          for (int i = 0; i < DKDV_KEYS / 16; ++i) {
            opa[i] = read_tr_operand(dsb, dsof, 16 * i, 0);  // dS: lanes = query rows, k = keys
            opb[i] = read_tr_operand(kt, of, 16 * i, wv);    // K: lanes = features, k = keys
          }
          f32x16_t qa = zero16();
#pragma unroll
          for (int i = 0; i < DKDV_KEYS / 16; ++i) qa = MF::mfma(opa[i], opb[i], qa);
          const int hq = g * a.group + hh_cur;
          float* qrow = a.dq_acc + ((q0 + r0) * (int64_t)a.n1 + hq) * D + 32 * wv + (lane & 31);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int rl = 32 * h + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (rl < nrows) unsafeAtomicAdd(qrow + (int64_t)rl * a.n1 * D, qa[i]);
          }
        }
      }
    }
    stage ^= 1;
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    mfma_acc_done(dk[n]);
    mfma_acc_done(dv[n]);
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int key = key_w + 32 * n;
    if (key < kcap) {
      const int64_t orow = key_row(key);
      uint16_t* dkp = reinterpret_cast<uint16_t*>(a.dk) + orow;
      uint16_t* dvp = reinterpret_cast<uint16_t*>(a.dv) + orow;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        store_cols<MF>(dkp, 32 * mt, dk[n][mt], a.sigma);
        store_cols<MF>(dvp, 32 * mt, dv[n][mt], 1.f);
      }
    }
  }
}

template <typename MF, int D, bool PAGED>
hipError_t launch_dq_p(const BwdArgs& a, int64_t grid, hipStream_t st) {
  switch (window_mode(a.seq)) {
    case 0: k_bwd_dq<MF, D, 0, PAGED><<<(unsigned)grid, 256, 0, st>>>(a); break;
    case 1: k_bwd_dq<MF, D, 1, PAGED><<<(unsigned)grid, 256, 0, st>>>(a); break;
    default: k_bwd_dq<MF, D, 2, PAGED><<<(unsigned)grid, 256, 0, st>>>(a); break;
  }
  return hipGetLastError();
}
template <typename MF, int D>
hipError_t launch_dq_t(const BwdArgs& a, int64_t grid, hipStream_t st) {
  return a.seq.seqused_kv ? launch_dq_p<MF, D, true>(a, grid, st) : launch_dq_p<MF, D, false>(a, grid, st);
}
template <typename MF, int D, bool PAGED, bool DQA>
hipError_t launch_dkdv_q(const BwdArgs& a, int64_t grid, hipStream_t st) {
  constexpr unsigned threads = 64 * DkdvShape<D, DQA>::NW;
  switch (window_mode(a.seq)) {
    case 0: k_bwd_dkdv<MF, D, 0, PAGED, DQA><<<(unsigned)grid, threads, 0, st>>>(a); break;
    case 1: k_bwd_dkdv<MF, D, 1, PAGED, DQA><<<(unsigned)grid, threads, 0, st>>>(a); break;
    default: k_bwd_dkdv<MF, D, 2, PAGED, DQA><<<(unsigned)grid, threads, 0, st>>>(a); break;
  }
  return hipGetLastError();
}
template <typename MF, int D, bool PAGED>
hipError_t launch_dkdv_p(const BwdArgs& a, int64_t grid, hipStream_t st) {
  if (a.dq_acc) return launch_dkdv_q<MF, D, PAGED, true>(a, grid, st);
  return launch_dkdv_q<MF, D, PAGED, false>(a, grid, st);
}
template <typename MF, int D>
hipError_t launch_dkdv_t(const BwdArgs& a, int64_t grid, hipStream_t st) {
  return a.seq.seqused_kv ? launch_dkdv_p<MF, D, true>(a, grid, st) : launch_dkdv_p<MF, D, false>(a, grid, st);
}
}  // namespace

hipError_t launch_bwd_pre(const BwdPreArgs& a, int dtype, int head_dim, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  const int64_t threads = a.rows * (head_dim / 8);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (dtype == 2) {
    if (head_dim == 128) k_bwd_pre<BF16, 128><<<grid, 256, 0, st>>>(a);
    else k_bwd_pre<BF16, 64><<<grid, 256, 0, st>>>(a);
  } else {
    if (head_dim == 128) k_bwd_pre<F16, 128><<<grid, 256, 0, st>>>(a);
    else k_bwd_pre<F16, 64><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_dq_convert(const float* acc, void* dq, int64_t elems, float sigma, int dtype, hipStream_t st) {
  const int64_t n8 = elems / 8;
  if (n8 <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((n8 + 255) / 256);
  if (dtype == 2)
    k_dq_convert<BF16><<<grid, 256, 0, st>>>(acc, reinterpret_cast<uint16_t*>(dq), n8, sigma);
  else
    k_dq_convert<F16><<<grid, 256, 0, st>>>(acc, reinterpret_cast<uint16_t*>(dq), n8, sigma);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int dtype, int head_dim, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  const bool bf = dtype == 2;
  if (head_dim == 128) return bf ? launch_dq_t<BF16, 128>(a, grid, st) : launch_dq_t<F16, 128>(a, grid, st);
  return bf ? launch_dq_t<BF16, 64>(a, grid, st) : launch_dq_t<F16, 64>(a, grid, st);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int dtype, int head_dim, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  const bool bf = dtype == 2;
  if (head_dim == 128) return bf ? launch_dkdv_t<BF16, 128>(a, grid, st) : launch_dkdv_t<F16, 128>(a, grid, st);
  return bf ? launch_dkdv_t<BF16, 64>(a, grid, st) : launch_dkdv_t<F16, 64>(a, grid, st);
}

}  // namespace bsa
