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
// the tile (the transposed, per-KV-block index lists).  dQ is a separate
// Q-block-major pass over the forward's per-q-block lists, so no output is
// accumulated with atomics and results are deterministic run to run.
#include "bsa_attn.h"

namespace bsa {
namespace {

constexpr float LOG2E = 1.4426950408889634f;

// ------------------------------------------------------------- D = dO.O --
// One 16-byte chunk per thread, D/8 threads per (token, head) row.
template <typename MF, int D>
__global__ __launch_bounds__(256) void k_bwd_pre(BwdPreArgs a) {
  constexpr int CH = D / 8;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / CH;
  const int c = threadIdx.x % CH;
  float acc = 0.f;
  if (row < a.rows) {
    const u32x4_t o = gload16(reinterpret_cast<const uint16_t*>(a.out) + row * D + c * 8);
    const u32x4_t d = gload16(reinterpret_cast<const uint16_t*>(a.dout) + row * D + c * 8);
    acc = MF::lo(o.x) * MF::lo(d.x) + MF::hi(o.x) * MF::hi(d.x) + MF::lo(o.y) * MF::lo(d.y) +
          MF::hi(o.y) * MF::hi(d.y) + MF::lo(o.z) * MF::lo(d.z) + MF::hi(o.z) * MF::hi(d.z) +
          MF::lo(o.w) * MF::lo(d.w) + MF::hi(o.w) * MF::hi(d.w);
  }
#pragma unroll
  for (int m = CH / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < a.rows && c == 0) a.dl[row] = acc;
}

// -------------------------------------------------------------------- dQ --
// Same work items and key walk as the forward kernel.  Per 64-key sub-tile:
//   S^T = K Q^T, dP^T = V dO^T            (K, V row-major from LDS)
//   P^T = exp2(S^T scale log2e - lse log2e), dS^T = P^T o (dP^T - D)
//   dQ^T += K^T dS^T                       (K^T via LDS transpose loads)
template <typename MF, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void k_bwd_dq(BwdArgs a) {
  constexpr int TILE = KT * D * 2;
  constexpr int NMT = D / 32;
  constexpr int NKK = D / 16;
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE];

  QItem it;
  if (!decode_qitem(blockIdx.x, a.hdr, a.work, a.qb_seq, a.qbase, a.seq, a.heads_per_row, a.group, it)) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int my_local = wv * 32 + (lane & 31);
  const int my_row = it.row_lo + my_local;
  const bool row_ok = my_local < it.nrows;
  const int qoff = it.skv - it.sq;
  int kend = it.skv;
  if (CAUSAL) kend = min(kend, it.row_lo + it.nrows - 1 + qoff + 1);

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
  const float dl = row_ok ? a.dl[tok * a.n1 + it.h] : 0.f;

  const KvAddr ka = make_kv_addr(a.seq, nullptr, it.b, it.g, a.n2, D, 0, 0, 0);
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.v);

  f32x16_t acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) acc[mt] = zero16();
  const float c2 = a.sigma_log2e;

  Stage<D, KT> sk, sv;
  SubTileWalk wk;
  wk.init(a.cols, a.row_ptr[it.r], a.row_ptr[it.r + 1], a.seq.by, kend);
  auto load = [&](int key0) {
    auto off = [&](int row) { return ka.offset(key0 + row); };
    auto ok = [&](int row) { return key0 + row < it.skv; };
    sk.load(kp, off, ok);
    sv.load(vp, off, ok);
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

    f32x16_t s[2], dp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = zero16();
      dp[t] = zero16();
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s[t] = MF::mfma(read_operand<D>(kl, 32 * t, kk), qf[kk], s[t]);
        dp[t] = MF::mfma(read_operand<D>(vl, 32 * t, kk), df[kk], dp[t]);
      }
    }
    const int lim = CAUSAL ? min(it.skv - 1, my_row + qoff) : it.skv - 1;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + 32 * t + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        float p = fast_exp2(fmaf(s[t][i], c2, -lse2));
        if (key > lim) p = 0.f;
        s[t][i] = p * (dp[t][i] - dl);  // dS^T
      }
    u32x4_t db[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) db[kc] = pack8<MF>(s[kc >> 1], 8 * (kc & 1));
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) acc[mt] = MF::mfma(read_tr_operand<D>(kl, 16 * kc, 32 * mt), db[kc], acc[mt]);
    buf ^= 1;
  }
  if (row_ok) {
    uint16_t* op = reinterpret_cast<uint16_t*>(a.dq) + tok * qstride + (int64_t)it.h * D;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) store_cols<MF>(op, 32 * mt, acc[mt], a.sigma);
  }
}

// ----------------------------------------------------------------- dK, dV --
// Work item: one 128-key tile of KV block (g, b, kb); wave w owns keys
// 32w .. 32w+31 and keeps its K and V rows in registers as the B operands of
// S = Q K^T and dP = dO V^T.  For every q-head of the group and every q-block
// in the tile's transposed list, 64-row query sub-tiles of Q, dO, lse and D
// are staged through double-buffered LDS and each wave computes
//   S, dP                (MFMA, Q / dO row-major from LDS)
//   P = exp2(S scale log2e - lse log2e), dS = P o (dP - D)
//   dV^T += dO^T P,  dK^T += Q^T dS   (Q^T / dO^T via LDS transpose loads,
//                                      P / dS straight from registers)
constexpr int QS = 64;  // query rows per staged sub-tile

template <typename MF, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void k_bwd_dkdv(BwdArgs a) {
  constexpr int TILE = QS * D * 2;
  constexpr int NMT = D / 32;
  constexpr int NKK = D / 16;
  constexpr int BUF = 2 * TILE + 2 * QS * 4;  // Q, dO, lse*log2e, D
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

  const int KVI = a.hdr[H_KVITEMS];
  const int64_t item = blockIdx.x / a.sub_tiles;
  const int sub = blockIdx.x - (int)item * a.sub_tiles;
  if (item >= KVI) return;
  const int TKB = a.hdr[H_TKB];
  const int w_id = a.work_kv[item];
  const int g = w_id / TKB, kg = w_id - g * TKB;
  const int b = a.kb_seq[kg];
  const int kb = kg - a.kbase[b];
  const int64_t q0 = a.seq.cu_q[b];
  const int sq = (int)(a.seq.cu_q[b + 1] - q0);
  const int skv = (int)(a.seq.cu_kv[b + 1] - a.seq.cu_kv[b]);
  const int key_lo = kb * a.seq.by + sub * 128;
  if (key_lo >= skv) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int my_key = key_lo + wv * 32 + (lane & 31);
  const bool key_ok = my_key < skv;
  const int qoff = skv - sq;
  const int64_t kvstride = (int64_t)a.n2 * D;
  const int64_t krow = (a.seq.cu_kv[b] + my_key) * kvstride + (int64_t)g * D + 8 * (lane >> 5);
  u32x4_t kf[NKK], vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    kf[kk] = key_ok ? gload16(reinterpret_cast<const uint16_t*>(a.k) + krow + 16 * kk) : zero_u4();
    vf[kk] = key_ok ? gload16(reinterpret_cast<const uint16_t*>(a.v) + krow + 16 * kk) : zero_u4();
  }
  f32x16_t dk[NMT], dv[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    dk[mt] = zero16();
    dv[mt] = zero16();
  }
  const float c2 = a.sigma_log2e;
  const int64_t qstride = (int64_t)a.n1 * D;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* dop = reinterpret_cast<const uint16_t*>(a.dout);
  // smallest key of this workgroup's tile: q rows whose causal limit is below
  // it contribute nothing
  const int wg_key_min = key_lo;

  // Walk: heads h of group g, q-blocks of column c(h), 64-row halves.
  struct Walk {
    int hh, e, e1, half;
  } wk;
  const int ncols_heads = a.hs == a.n1 ? a.group : 1;  // distinct columns in the group
  auto col_of = [&](int hh) { return (a.hs == a.n1 ? g * a.group + hh : g) * TKB + kg; };
  auto sub_ok = [&](int qb, int half) {
    const int r0 = qb * 128 + half * QS;
    if (r0 >= sq) return false;
    if (CAUSAL) {
      const int rlast = min(r0 + QS, sq) - 1;
      if (rlast + qoff < wg_key_min) return false;
    }
    return true;
  };
  // advance to the first valid (head, entry, half) at or after the current one
  auto settle = [&]() {
    while (wk.hh < a.group) {
      while (wk.e < wk.e1) {
        const int qb = a.qrows[wk.e];
        while (wk.half < 2) {
          if (sub_ok(qb, wk.half)) return;
          ++wk.half;
        }
        ++wk.e;
        wk.half = 0;
      }
      ++wk.hh;
      if (wk.hh < a.group) {
        const int c = col_of(ncols_heads == 1 ? 0 : wk.hh);
        wk.e = a.col_ptr[c];
        wk.e1 = a.col_ptr[c + 1];
      }
    }
  };
  {
    const int c = col_of(0);
    wk.hh = 0;
    wk.e = a.col_ptr[c];
    wk.e1 = a.col_ptr[c + 1];
    wk.half = 0;
  }
  settle();
  auto advance = [&]() {
    ++wk.half;
    settle();
  };

  Stage<D, QS> sq_, sd_;
  float st_lse = 0.f, st_dl = 0.f;
  int cur_r0 = 0, cur_h = 0;
  auto load = [&]() {
    const int h = g * a.group + wk.hh;
    const int r0 = a.qrows[wk.e] * 128 + wk.half * QS;
    auto off = [&](int row) { return (q0 + r0 + row) * qstride + (int64_t)h * D; };
    auto ok = [&](int row) { return r0 + row < sq; };
    sq_.load(qp, off, ok);
    sd_.load(dop, off, ok);
    const int t = threadIdx.x;
    if (t < 2 * QS) {
      const int row = t & (QS - 1);
      const bool rok = r0 + row < sq;
      const int64_t idx = (q0 + r0 + row) * a.n1 + h;
      if (t < QS)
        st_lse = rok ? a.lse[idx] * LOG2E : INFINITY;
      else
        st_dl = rok ? a.dl[idx] : 0.f;
    }
    cur_r0 = r0;
    cur_h = h;
  };

  int buf = 0;
  int ld_r0 = 0;
  if (wk.hh < a.group) {
    load();
    ld_r0 = cur_r0;
  }
  while (wk.hh < a.group) {
    const int r0 = ld_r0;
    char* ql = smem + buf * BUF;
    char* dl_ = ql + TILE;
    float* lsel = reinterpret_cast<float*>(ql + 2 * TILE);
    float* dll = lsel + QS;
    sq_.store(ql);
    sd_.store(dl_);
    if (threadIdx.x < QS)
      lsel[threadIdx.x] = st_lse;
    else if (threadIdx.x < 2 * QS)
      dll[threadIdx.x - QS] = st_dl;
    __syncthreads();
    advance();
    if (wk.hh < a.group) {
      load();
      ld_r0 = cur_r0;
    }

    // S[qrow, key], dP[qrow, key] for 64 query rows (two 32-row tiles)
    f32x16_t s[2], dp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = zero16();
      dp[t] = zero16();
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s[t] = MF::mfma(read_operand<D>(ql, 32 * t, kk), kf[kk], s[t]);
        dp[t] = MF::mfma(read_operand<D>(dl_, 32 * t, kk), vf[kk], dp[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int rl = 32 * t + 8 * ig + 4 * (lane >> 5);  // first of 4 consecutive query rows
        const u32x4_t l4 = *reinterpret_cast<const u32x4_t*>(lsel + rl);
        const u32x4_t d4 = *reinterpret_cast<const u32x4_t*>(dll + rl);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * ig + j;
          float p = fast_exp2(fmaf(s[t][i], c2, -__uint_as_float(l4[j])));
          if (CAUSAL && my_key > r0 + rl + j + qoff) p = 0.f;
          s[t][i] = p;
          dp[t][i] = p * (dp[t][i] - __uint_as_float(d4[j]));
        }
      }
    u32x4_t pb[4], sb[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      pb[kc] = pack8<MF>(s[kc >> 1], 8 * (kc & 1));
      sb[kc] = pack8<MF>(dp[kc >> 1], 8 * (kc & 1));
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        dv[mt] = MF::mfma(read_tr_operand<D>(dl_, 16 * kc, 32 * mt), pb[kc], dv[mt]);
        dk[mt] = MF::mfma(read_tr_operand<D>(ql, 16 * kc, 32 * mt), sb[kc], dk[mt]);
      }
    buf ^= 1;
  }
  (void)cur_h;
  if (key_ok) {
    const int64_t orow = (a.seq.cu_kv[b] + my_key) * kvstride + (int64_t)g * D;
    uint16_t* dkp = reinterpret_cast<uint16_t*>(a.dk) + orow;
    uint16_t* dvp = reinterpret_cast<uint16_t*>(a.dv) + orow;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      store_cols<MF>(dkp, 32 * mt, dk[mt], a.sigma);
      store_cols<MF>(dvp, 32 * mt, dv[mt], 1.f);
    }
  }
}

template <typename MF, int D>
hipError_t launch_dq_t(const BwdArgs& a, int64_t grid, hipStream_t st) {
  if (a.seq.causal)
    k_bwd_dq<MF, D, true><<<(unsigned)grid, 256, 0, st>>>(a);
  else
    k_bwd_dq<MF, D, false><<<(unsigned)grid, 256, 0, st>>>(a);
  return hipGetLastError();
}
template <typename MF, int D>
hipError_t launch_dkdv_t(const BwdArgs& a, int64_t grid, hipStream_t st) {
  if (a.seq.causal)
    k_bwd_dkdv<MF, D, true><<<(unsigned)grid, 256, 0, st>>>(a);
  else
    k_bwd_dkdv<MF, D, false><<<(unsigned)grid, 256, 0, st>>>(a);
  return hipGetLastError();
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
