// Device helpers for the gfx950 kernels: MFMA operand types, fp32 -> 16-bit
// packing, LDS tile addressing and wave-level utilities.
//
// MFMA v_mfma_f32_32x32x16_{bf16,f16} lane layout (wave64), checked on the
// hardware:
//   A (32 x 16, M x K): lane l holds row l % 32, k = 8 * (l / 32) + j, j < 8
//   B (16 x 32, K x N): lane l holds col l % 32, k = 8 * (l / 32) + j
//   C (32 x 32):        lane l, element i holds row 8 * (i / 4) + 4 * (l / 32)
//                       + i % 4 of column l % 32
// ds_read_b64_tr_b16: within each 16-lane group, lane i returns element i % 4
// of the 8-byte rows addressed by source lanes i / 4 + 4 j (j < 4).  With
// source lane s pointing at row r0 + s / 4, columns c0 + 4 (s % 4) .. + 3 of a
// row-major 16-bit matrix, lane i receives rows r0 .. r0 + 3 of column c0 + i:
// a transposed operand read straight from a row-major LDS tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

struct BF16 {
  typedef bf16x8_t v8;
  static __device__ __forceinline__ f32x16_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
  // acc += A B with acc held in accumulation registers (AGPRs); see mfma_acc_done.
  static __device__ __forceinline__ void mfma_acc(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  }
  // Two fp32 values rounded to nearest-even bf16, packed lo | hi << 16.
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2_t r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float lo(uint32_t x) { return __uint_as_float(x << 16); }
  static __device__ __forceinline__ float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
};

struct F16 {
  typedef f16x8_t v8;
  static __device__ __forceinline__ f32x16_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void mfma_acc(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2_t r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float lo(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
  }
};

// mfma_acc pins a long-lived accumulator to the AGPRs, leaving the VGPRs to
// the operands and to the MFMA results the softmax works on.  The compiler cannot see that the asm is an
// MFMA, so it inserts none of the MFMA wait states; two are covered by hand:
//  * a VALU write of an operand register (the compiler may stage an operand
//    through a copy right before the asm) needs 2 wait states before the
//    MFMA reads it: each asm MFMA starts with s_nop 1, which issues while the
//    matrix pipe is still busy with the previous MFMA;
//  * before the results are read back, mfma_acc_done waits
//    out the MFMA latency (XDL result -> VALU read needs at most 19 wait
//    states on CDNA3/4), tied to each accumulator so that no read is
//    scheduled ahead of the wait.
template <int N>
__device__ __forceinline__ void mfma_acc_done(f32x16_t (&acc)[N]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0]));
#pragma unroll
  for (int i = 1; i < N; ++i) asm volatile("" : "+a"(acc[i]));
}

// Pins the computation of x to this point of the instruction stream: the
// compiler must have x in a VGPR here and may not sink its producers past it
// (used to keep independent VALU work interleaved with MFMA runs).
template <class T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ---------------------------------------------------------------------------
// Row-major LDS tiles of 16-bit elements with D columns.  Two layouts:
//
// XorTile: rows of 2D bytes whose 16-byte chunks are XOR-permuted by row % 16.
//   ds_read_b128 is served 16 lanes at a time; 16 consecutive rows reading the
//   same logical chunk land on 16 distinct 16-byte bank groups, and the
//   transposed ds_read_b64_tr_b16 reads (4 rows x 32 bytes per 16 lanes) stay
//   conflict free too.  For tiles read both ways.  Offsets are non-linear in
//   the column, so kernels precompute them per lane (OperandOffsets).
//
// PadTile: rows padded by PAD bytes, addresses linear in row and column.  With
//   64 banks of 4 bytes, PAD = 16 puts 16 consecutive rows at 16 distinct bank
//   groups (row-major operand reads); PAD = 64 makes the 4 rows of a
//   transposed read cover 16 distinct bank groups.  For tiles read one way.
// ---------------------------------------------------------------------------
template <int D>
struct XorTile {
  static constexpr int CH = D / 8;  // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr bool LINEAR = false;
  template <int ROWS>
  static constexpr int bytes() { return ROWS * ROW_BYTES; }
  static __device__ __forceinline__ int swz(int row) {
    if constexpr (CH == 16) {
      return ((row & 3) << 2) | ((row >> 2) & 3);
    } else {
      return (row >> 1) & (CH - 1);
    }
  }
  static __device__ __forceinline__ int chunk_off(int row, int c) { return row * ROW_BYTES + ((c ^ swz(row)) << 4); }
  static __device__ __forceinline__ int col_off(int row, int col) {
    return row * ROW_BYTES + (((col >> 3) ^ swz(row)) << 4) + ((col & 7) << 1);
  }
};

template <int D, int PAD>
struct PadTile {
  static constexpr int CH = D / 8;
  static constexpr int ROW_BYTES = D * 2 + PAD;
  static constexpr bool LINEAR = true;
  template <int ROWS>
  static constexpr int bytes() { return ROWS * ROW_BYTES; }
  static __device__ __forceinline__ int chunk_off(int row, int c) { return row * ROW_BYTES + (c << 4); }
  static __device__ __forceinline__ int col_off(int row, int col) { return row * ROW_BYTES + (col << 1); }
};

__device__ __forceinline__ u32x4_t lds_read16(const char* base, int off) {
  return *reinterpret_cast<const u32x4_t*>(base + off);
}
__device__ __forceinline__ void lds_write16(char* base, int off, const u32x4_t& v) {
  *reinterpret_cast<u32x4_t*>(base + off) = v;
}
// Transposed read: see the layout note at the top of the file.
__device__ __forceinline__ u32x2_t lds_read_tr(const char* base, int off) {
  i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + off));
  return __builtin_bit_cast(u32x2_t, r);
}

__device__ __forceinline__ u32x4_t gload16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ u32x4_t zero_u4() {
  u32x4_t z = {0u, 0u, 0u, 0u};
  return z;
}

// Loads of read-only schedule data (index lists, lengths, page tables) with a
// wave-uniform address, through the constant address space so they become
// scalar loads: they are then counted apart from the vector loads, and waiting
// for one never waits for tile loads in flight.
template <typename T>
__device__ __forceinline__ T ldu(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)(p))[i];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Combines x of lane l and lane l ^ 32 with v_permlane32_swap (a VALU op, no
// LDS round trip).  permlane32_swap(x, x) returns r0 = {x[0..31], x[0..31]}
// and r1 = {x[32..63], x[32..63]} (checked on the hardware), so every lane
// holds its own and its partner's value in r0 / r1.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max3f(float x, float y, float z) { return fmaxf(fmaxf(x, y), z); }
// Maximum of the 32 values of two accumulator fragments: a tree of 15
// three-input maxima (v_max3_f32) and one two-input one.
__device__ __forceinline__ float max32(const f32x16_t& a, const f32x16_t& b) {
  float v[32], m[12], n[4];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = a[i];
    v[16 + i] = b[i];
  }
#pragma unroll
  for (int k = 0; k < 10; ++k) m[k] = max3f(v[3 * k], v[3 * k + 1], v[3 * k + 2]);
  m[10] = v[30];
  m[11] = v[31];
#pragma unroll
  for (int k = 0; k < 4; ++k) n[k] = max3f(m[3 * k], m[3 * k + 1], m[3 * k + 2]);
  return fmaxf(max3f(n[0], n[1], n[2]), n[3]);
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return x;
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (l >= o) x += y;
  }
  return x;
}

}  // namespace bsa
