// Forward block-sparse varlen attention with FLOAT8_E4M3 q, k, v on gfx950:
// GenericBlockSparseAttention's quantType 5 (Quantisation table): Q, K, V are
// e4m3 with no scale factors and the operator casts P to e4m3 itself before
// the PV product; the output is fp16 or bf16.
//
// Same work items, sub-tile walk, staging and online softmax as k_fwd (fp32
// softmax, the reference maximum moved only when exceeded by more than 8 in
// log2 units, so every P is at most 256 and fits e4m3's range of 448).  The
// two contractions run on v_mfma_f32_32x32x64_f8f6f4 with both operands e4m3.
//
// Operand layout of that MFMA (checked on the hardware with an in-bounds
// probe): lane l supplies row (A) or column (B) l % 32 and 32 bytes of the
// contraction, and byte j of lane l meets byte j of the other operand's lane
// in the same half (l / 32).  Any assignment of the 64 contraction indices to
// (half h, byte j) therefore works when both operands use it:
//  * S^T = K Q^T, per 32-key tile t and 64-feature step kk:
//      d = 64 kk + 32 h + j (two 16-byte pieces of a K row / Q row);
//  * O^T += V^T P^T, per 32-feature tile mt, the whole 64-key sub-tile:
//      key = 32 h + j.
// P^T (B) comes from the S^T accumulators, where lane l holds query l % 32
// and keys 32 t + 8 a + 4 (l / 32) + b (a, b < 4).  Each run of 4 keys is
// packed into one register (v_cvt_pk_fp8_f32, round to nearest even), and
// v_permlane32_swap between the tiles' registers gives lane l the keys
// 32 (l / 32) + 0 .. 31 of its query in order.  V^T (A) is read from the
// row-major V tile with ds_read_b64_tr_b8: within a 16-lane group, lanes 2 r
// and 2 r + 1 address the two 8-byte halves of a 16-byte piece of key row r,
// and lane q receives byte q of each of the 8 rows -- one feature, 8 keys.
//
// Tiles of 64 rows x 128 bytes use the XOR layout of a 64-column 16-bit tile
// (same byte geometry), and the copies and key addressing count in 16-bit
// units: every fp8 offset they form is even.
#include <type_traits>

#include "bsa_attn.h"

namespace bsa {
namespace {

constexpr float RESCALE_LOG2_F8 = 8.f;  // P <= 2^8 = 256 < 448

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;

__device__ __forceinline__ f32x16_t mfma_f8(const v8i_t& a, const v8i_t& b, const f32x16_t& c) {
  // format selectors 0 / 0: both operands FLOAT8_E4M3; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// four fp32 values -> one register of e4m3 bytes, first value in byte 0
__device__ __forceinline__ int pack4_f8(float x0, float x1, float x2, float x3) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, r, true);
}

// Three workgroups per CU (three waves per SIMD: 168 registers each, 32 KiB
// of LDS per workgroup); two measured 7 % slower.
template <typename OUT, int WMODE, bool PAGED>
__global__ __launch_bounds__(256, 3) void k_fwd_fp8(FwdArgs a) {
  constexpr int D = 128;         // features (bytes per row)
  using L = XorTile<64>;         // 128-byte rows, 8 XOR-permuted 16-byte chunks
  constexpr int TILE = L::template bytes<KT>();  // 8 KiB
  constexpr int STAGE = 2 * TILE;                // K, V
  constexpr int NMT = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  QItem it;
  if (!decode_qitem(xcd_item(blockIdx.x, a.xseg), a.hdr, a.work, a.qb_seq, a.qbase, a.seq, a.heads_per_row, a.group,
                   it))
    return;
  const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;                    // lane half
  const int my_local = wv * 32 + (lane & 31);  // row within the item
  const int my_row = it.row_lo + my_local;     // row within the sequence
  const bool row_ok = my_local < it.nrows;
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

  // Q^T operand (B of S^T): lane holds its row's bytes 64 kk + 32 h .. + 31
  const int64_t qstride = (int64_t)a.n1 * D;  // bytes
  const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.q) + (it.q0 + my_row) * qstride + (int64_t)it.h * D + 32 * hl;
  v8i_t qf[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const u32x4_t lo = row_ok ? gload16(qp + 64 * kk) : zero_u4();
    const u32x4_t hi = row_ok ? gload16(qp + 64 * kk + 16) : zero_u4();
    qf[kk] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }

  // LDS offsets.  K (A of S^T): row lane % 32 (+ 32 for tile 1, same XOR),
  // chunks 4 kk + 2 h and + 1.  V^T (A of O^T) by transposed reads: group
  // g = lane / 16, q = lane % 16; read t of feature tile mt points at key row
  // 32 (g / 2) + 8 t + q / 2, chunk 2 mt + g % 2, byte 8 (q % 2).
  int koff[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int p = 0; p < 2; ++p) koff[kk][p] = L::chunk_off(lane & 31, 4 * kk + 2 * hl + p);
  const int g16 = lane >> 4, q16 = lane & 15;
  int voff[NMT][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 32 * (g16 >> 1) + 8 * t + (q16 >> 1);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) voff[mt][t] = L::chunk_off(row, 2 * mt + (g16 & 1)) + 8 * (q16 & 1);
  }

  const uint16_t* kbase_p = reinterpret_cast<const uint16_t*>(a.k);  // 16-bit units
  const uint16_t* vbase_p = reinterpret_cast<const uint16_t*>(a.v);

  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c2 = a.sigma_log2e;
  const float thresh = RESCALE_LOG2_F8 / c2;

  DmaTile<L, 64, KT> kdma, vdma;
  kdma.init(a.n2 * (D / 2));
  vdma.init(a.n2 * (D / 2));
  RegTileWalk<> ld;
  ld.init(a.cols, ldu(a.row_ptr, it.r), ldu(a.row_ptr, it.r + 1), a.seq.by, kend, kstart);
  KvAddr<PAGED> kva;
  kva.init(a.seq, a.block_table, it.b, it.g, a.n2, D / 2, a.page_size, a.max_pages, a.page_stride / 2);
  int key_next = 0;
  uint32_t gm_next = 0xFu;  // selected 16-key groups of that sub-tile
  // row tiles: this wave's 32 rows' bits of that sub-tile's row mask
  uint32_t rm_next = 0xFFFFFFFFu;
  auto issue = [&](int stage, auto first) {
    char* st = smem + stage * STAGE;
    const int key0 = ld.template take<decltype(first)::value>();
    key_next = key0;
    gm_next = ld.gmask;
    if (a.row_mask) rm_next = ldu(a.row_mask, (int64_t)ld.ent * 4 + wv);
    const int64_t off = kva.off(key0);
    kdma.issue(st, kbase_p + off, it.skv - key0);
    vdma.issue(st + TILE, vbase_p + off, it.skv - key0);
  };
  bool more = ld.valid();
  if (more) issue(0, std::true_type{});
  int stage = 0;
  while (more) {
    const int key0 = key_next;
    const uint32_t gm = gm_next;   // its 16-key groups in selected blocks
    const uint32_t rm = rm_next;   // its row mask bits of this wave's rows
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
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
    const char* vl = kl + TILE;

    // ---- S^T = K Q^T for keys key0 .. key0+63 (two 32-key tiles) ----
    f32x16_t s[2];
    {
      v8i_t kop[2][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4_t lo = lds_read16(kl + 4096 * t, koff[kk][0]);
          const u32x4_t hi = lds_read16(kl + 4096 * t, koff[kk][1]);
          kop[kk][t] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      s[0] = mfma_f8(kop[0][0], qf[0], zero16());
      s[1] = mfma_f8(kop[0][1], qf[0], zero16());
      s[0] = mfma_f8(kop[1][0], qf[1], s[0]);
      s[1] = mfma_f8(kop[1][1], qf[1], s[1]);
    }
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
          const int key = key0 + 32 * t + 8 * (i >> 2) + 4 * hl + (i & 3);
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
    const bool upd = mx > m_run + thresh || (m_run == -INFINITY && mx > -INFINITY);
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float m_new = upd ? mx : m_run;
      const float alpha = upd ? fast_exp2((m_run - m_new) * c2) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[mt][i] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run * c2;
    float ps[4];
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
    // ---- P^T operand: e4m3, keys 32 h + 0 .. 31 of this lane's query ----
    v8i_t pb;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int p0 = pack4_f8(s[0][4 * g], s[0][4 * g + 1], s[0][4 * g + 2], s[0][4 * g + 3]);
      const int p1 = pack4_f8(s[1][4 * g], s[1][4 * g + 1], s[1][4 * g + 2], s[1][4 * g + 3]);
      const auto r = __builtin_amdgcn_permlane32_swap((unsigned)p0, (unsigned)p1, false, false);
      pb[2 * g] = (int)r[0];
      pb[2 * g + 1] = (int)r[1];
    }
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      v8i_t vop;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v2i_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(vl + voff[mt][t]));
        vop[2 * t] = r.x;
        vop[2 * t + 1] = r.y;
      }
      o[mt] = mfma_f8(vop, pb, o[mt]);
    }
    stage ^= 1;
  }

  // ---- epilogue: O = O^T / l, lse = scale * m + ln l ----
  const float l_tot = half_sum(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (it.q0 + my_row) * (int64_t)a.n1 * D + (int64_t)it.h * D;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) store_cols<OUT>(op, 32 * mt, o[mt], inv);
    if (lane < 32) {
      a.lse[(it.q0 + my_row) * a.n1 + it.h] =
          l_tot > 0.f ? m_run * a.sigma + fast_log2(l_tot) * 0.69314718055994531f : INFINITY;
    }
  }
}

template <typename OUT, bool PAGED>
hipError_t launch_t(const FwdArgs& a, int64_t grid, hipStream_t st) {
  switch (window_mode(a.seq)) {
    case 0: k_fwd_fp8<OUT, 0, PAGED><<<(unsigned)grid, 256, 0, st>>>(a); break;
    case 1: k_fwd_fp8<OUT, 1, PAGED><<<(unsigned)grid, 256, 0, st>>>(a); break;
    default: k_fwd_fp8<OUT, 2, PAGED><<<(unsigned)grid, 256, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

template <typename OUT>
hipError_t launch_p(const FwdArgs& a, int64_t grid, hipStream_t st) {
  return a.seq.seqused_kv ? launch_t<OUT, true>(a, grid, st) : launch_t<OUT, false>(a, grid, st);
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdArgs& a, int out_dtype, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  return out_dtype == 2 ? launch_p<BF16>(a, grid, st) : launch_p<F16>(a, grid, st);
}

}  // namespace bsa
