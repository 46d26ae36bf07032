// Device-side building blocks for the gfx950 (CDNA4) attention kernels.
//
// Operand conventions of v_mfma_f32_32x32x16_{bf16,f16} used throughout
// (wave64, g = lane / 32, c = lane % 32):
//   A (32 x 16): lane holds row c, eight k-slots of group g
//   B (16 x 32): lane holds column c, the same eight k-slots of group g
//   C (32 x 32): lane holds column c, rows 8*(v/4) + 4*g + (v%4), v = 0..15
// Which physical k a slot stands for never matters as long as A and B agree,
// so every contraction below picks the slot->k map that keeps its operands
// contiguous in registers or in LDS.
//
// A C-layout tile X (rows in registers, columns across lanes) can feed the
// next product directly as a B operand that contracts over X's rows.  The
// kernels are arranged so that every softmax row lives in one lane column:
// the forward computes S^T = K Q^T, so row statistics (m, l) and the output
// rescale are lane-local, as in the online softmax of the FlashAttention-2
// notes (eqs. (5), (6), (10)).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaskBlock = 128;  // tokens per block-mask entry

struct bf16_tag {};
struct f16_tag {};

// 32x32x16 MFMA on packed 16-bit operands (8 per lane in a u32x4).
template <typename Tag>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (std::is_same<Tag, bf16_tag>::value)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Round two floats to the 16-bit input type (nearest-even) and pack.
template <typename Tag>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (std::is_same<Tag, bf16_tag>::value) {
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
  } else {
    f16x2_t v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
  }
}

template <typename Tag>
__device__ __forceinline__ float to_f32(uint16_t bits) {
  if constexpr (std::is_same<Tag, bf16_tag>::value)
    return __uint_as_float(((uint32_t)bits) << 16);
  else
    return (float)__builtin_bit_cast(_Float16, bits);
}

// Eight consecutive C-layout values (v = base..base+7) as one B operand.
template <typename Tag>
__device__ __forceinline__ u32x4 pack8(const f32x16& x, int base) {
  u32x4 r;
  r[0] = pack2<Tag>(x[base + 0], x[base + 1]);
  r[1] = pack2<Tag>(x[base + 2], x[base + 3]);
  r[2] = pack2<Tag>(x[base + 4], x[base + 5]);
  r[3] = pack2<Tag>(x[base + 6], x[base + 7]);
  return r;
}

// Value held by lane (l % 32) combined with the value of lane (l % 32) + 32:
// v_permlane32_swap returns, in every lane, the lower-half and upper-half
// copies of the same column.
__device__ __forceinline__ float half_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// LDS tile layouts.  A tile is R rows x C columns of 16-bit elements stored
// row by row; 16-byte chunks inside a row are XOR-swizzled so that the
// 16 lanes served together by the LDS hit distinct banks both when a wave
// reads one chunk column down 32 consecutive rows (MFMA operand fetch) and
// when it writes a tile.
//   row-major ("RM"):   rows = tokens, columns = head dimension
//   transposed ("TT"):  rows = head dimension, columns = tokens, with token
//                       bits 2 and 3 swapped so the eight tokens of one
//                       lane's k-slots are contiguous (see tt_pos).
// ---------------------------------------------------------------------------
template <int COLS>
struct Layout {
  static constexpr int kRowBytes = COLS * 2;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kRowsPer256 = kRowBytes >= 256 ? 1 : 256 / kRowBytes;
  static constexpr int kBytes(int rows) { return rows * kRowBytes; }
  // byte offset of 16-byte chunk `c` of row `r`
  __device__ __forceinline__ static int off(int r, int c) {
    int f = ((r / kRowsPer256) ^ (r / (kRowsPer256 * kChunks))) % kChunks;
    return r * kRowBytes + ((c ^ f) << 4);
  }
};

// Position of token t inside a TT row: bits 2 and 3 of t exchanged.
__device__ __forceinline__ int tt_pos(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

// Transpose a 4 x 8 block of 16-bit values held as four rows of u32x4 into
// eight columns of four values (u32x2 each).
__device__ __forceinline__ void transpose4x8(const u32x4 (&in)[4], u32x2 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // column 2c takes the low halves of dword c, column 2c+1 the high halves
    out[2 * c][0] = (in[0][c] & 0xffffu) | (in[1][c] << 16);
    out[2 * c][1] = (in[2][c] & 0xffffu) | (in[3][c] << 16);
    out[2 * c + 1][0] = (in[0][c] >> 16) | (in[1][c] & 0xffff0000u);
    out[2 * c + 1][1] = (in[2][c] >> 16) | (in[3][c] & 0xffff0000u);
  }
}

// Global -> registers staging of a tile of ROWS tokens x D columns.  Thread
// `tid` of NT owns units of 4 consecutive tokens x 8 columns; ROWS*D/32 units
// per tile.  Token indices are clamped to [0, n-1] so every load is in
// bounds; callers mask tokens >= n.
template <int ROWS, int D, int NT>
struct Stage {
  static constexpr int kUnits = ROWS * D / 32;
  static constexpr int kPer = (kUnits + NT - 1) / NT;
  static_assert(kUnits % NT == 0, "tile units must divide evenly among threads");
  u32x4 r[kPer][4];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int row0, int n, int tid) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      int unit = tid + u * NT;
      int dc = unit % (D / 8);
      int tg = unit / (D / 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int row = min(row0 + tg * 4 + j, n - 1);
        r[u][j] = *reinterpret_cast<const u32x4*>(base + (size_t)row * D + dc * 8);
      }
    }
  }
  // row-major copy: [ROWS][D]
  __device__ __forceinline__ void store_rm(char* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      int unit = tid + u * NT;
      int dc = unit % (D / 8);
      int tg = unit / (D / 8);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x4*>(lds + Layout<D>::off(tg * 4 + j, dc)) = r[u][j];
    }
  }
  // transposed copy: [D][ROWS], token order permuted by tt_pos
  __device__ __forceinline__ void store_tt(char* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      int unit = tid + u * NT;
      int dc = unit % (D / 8);
      int tg = unit / (D / 8);
      u32x2 t[8];
      transpose4x8(r[u], t);
      int pos = tt_pos(tg * 4);  // 4-aligned; the 4 tokens stay contiguous
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int drow = dc * 8 + j;
        *reinterpret_cast<u32x2*>(lds + Layout<ROWS>::off(drow, pos >> 3) + ((pos & 4) << 1)) = t[j];
      }
    }
  }
};

// Map a linear workgroup id so that each XCD (ids are dealt round-robin to
// the 8 XCDs) receives a contiguous range of logical work items, keeping the
// K/V of one head in one XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int nblk) {
  constexpr int kX = 8;
  int q = nblk / kX, r = nblk % kX;
  int x = b % kX, local = b / kX;
  return (x < r) ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

}  // namespace fa
