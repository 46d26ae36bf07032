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

// D += A B with D pinned to accumulation registers (AGPRs) for its whole
// lifetime.  Left to itself the compiler copies long-lived accumulators
// between register files every iteration once a kernel needs more than 256
// registers.  Hazards the compiler cannot see through the asm are the
// caller's: a VALU write of A or B needs two wait states before a product
// reads it (valu_to_mfma()); dependent accumulation into the same registers
// is interlocked; VALU reads of D after the last product wait in
// agpr_drain() / vgpr_drain().  Operands loaded from memory are covered by
// the compiler's own s_waitcnt.
template <typename Tag>
__device__ __forceinline__ void mfma32_acc(f32x16& d, u32x4 a, u32x4 b) {
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (std::is_same<Tag, bf16_tag>::value)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
#endif
}

// D = A B (FIRST) or D += A B with D in VGPRs, for results the VALU reads
// next (vgpr_drain() covers the read latency); B_AGPR: B is held in AGPRs.
// These keep two wait states in front of the product: around branches the
// compiler may copy A or D with VALU moves right before it.
#define FA_MFMA_VD(PRE, OP, FIRST, BC)                                                    \
  do {                                                                                   \
    if (FIRST)                                                                           \
      asm volatile(PRE OP " %0, %1, %2, 0" : "=&v"(d) : "v"(a), BC(b));                   \
    else                                                                                 \
      asm volatile(PRE OP " %0, %1, %2, %0" : "+v"(d) : "v"(a), BC(b));                   \
  } while (0)
#define FA_CONSTRAINT_A(x) "a"(x)
#define FA_CONSTRAINT_V(x) "v"(x)
// NOP = false drops the two wait states, for call sites where no VALU
// instruction writes A, B or D (operands loaded from LDS or memory, D
// written by the products only).
template <typename Tag, bool FIRST, bool B_AGPR, bool NOP = true>
__device__ __forceinline__ void mfma32_vd(f32x16& d, u32x4 a, u32x4 b) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool BF = std::is_same<Tag, bf16_tag>::value;
  if constexpr (NOP) {
    if constexpr (BF && B_AGPR) FA_MFMA_VD("s_nop 1\n\t", "v_mfma_f32_32x32x16_bf16", FIRST, FA_CONSTRAINT_A);
    else if constexpr (BF) FA_MFMA_VD("s_nop 1\n\t", "v_mfma_f32_32x32x16_bf16", FIRST, FA_CONSTRAINT_V);
    else if constexpr (B_AGPR) FA_MFMA_VD("s_nop 1\n\t", "v_mfma_f32_32x32x16_f16", FIRST, FA_CONSTRAINT_A);
    else FA_MFMA_VD("s_nop 1\n\t", "v_mfma_f32_32x32x16_f16", FIRST, FA_CONSTRAINT_V);
  } else {
    if constexpr (BF && B_AGPR) FA_MFMA_VD("", "v_mfma_f32_32x32x16_bf16", FIRST, FA_CONSTRAINT_A);
    else if constexpr (BF) FA_MFMA_VD("", "v_mfma_f32_32x32x16_bf16", FIRST, FA_CONSTRAINT_V);
    else if constexpr (B_AGPR) FA_MFMA_VD("", "v_mfma_f32_32x32x16_f16", FIRST, FA_CONSTRAINT_A);
    else FA_MFMA_VD("", "v_mfma_f32_32x32x16_f16", FIRST, FA_CONSTRAINT_V);
  }
#endif
}
// D = A B + C with C a VGPR tuple (an accumulator starting value), B in AGPRs.
template <typename Tag>
__device__ __forceinline__ void mfma32_vc(f32x16& d, u32x4 a, u32x4 b, const f32x16& c) {
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (std::is_same<Tag, bf16_tag>::value)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
#endif
}
#undef FA_MFMA_VD
#undef FA_CONSTRAINT_A
#undef FA_CONSTRAINT_V

// Two wait states between VALU writes of the given operand registers and
// the asm products that read them (the asm ties the order to the values).
template <int N>
__device__ __forceinline__ void valu_to_mfma(u32x4 (&r)[N]) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 1" : "+v"(r[0]));
#pragma unroll
  for (int i = 1; i < N; ++i) asm volatile("" : "+v"(r[i]));
#endif
}

template <int N>
__device__ __forceinline__ void vgpr_drain(f32x16 (&d)[N]) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 3" : "+v"(d[0]));
#pragma unroll
  for (int i = 1; i < N; ++i) asm volatile("" : "+v"(d[i]));
#endif
}

// 16-byte global load straight into AGPRs, for operands that only ever feed
// products through the asm wrappers above.  The compiler does not track it:
// the caller waits with vm_wait<0>() before the first use.
__device__ __forceinline__ void gload_agpr(u32x4& r, const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_dwordx4 %0, %1, off" : "=a"(r) : "v"(p) : "memory");
#endif
}

// Wait out the product-to-VALU read latency (at most 20 wait states for a
// 32x32x16 product) before any accumulator in d is read.
template <int N>
__device__ __forceinline__ void agpr_drain(f32x16 (&d)[N]) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 3" : "+a"(d[0]));
#pragma unroll
  for (int i = 1; i < N; ++i) asm volatile("" : "+a"(d[i]));
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

// pack8 with dropout: elements whose keep bit is clear become 0.
template <typename Tag>
__device__ __forceinline__ u32x4 pack8_keep(const f32x16& x, int base, const u32x4& kb, uint32_t thr);

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

// max(a, b, c) as one instruction.  fmaxf() on values the compiler cannot
// prove canonical (results of asm products) costs an extra NaN-quieting
// max per operand; these kernels never hold signalling NaNs.
__device__ __forceinline__ float max3(float a, float b, float c) {
#if defined(__HIP_DEVICE_COMPILE__)
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
#else
  return fmaxf(a, fmaxf(b, c));
#endif
}

// ---------------------------------------------------------------------------
// LDS tiles.  A tile holds ROWS tokens x D columns of 16-bit elements, row
// major, with padded rows so that every operand fetch is a per-lane base
// address plus a compile-time offset (no per-read address arithmetic).
//   Pad<D, false>: stride 2D+16 bytes; serves 16-byte row reads.
//   Pad<D, true>:  stride 2D+64 bytes and a 16-byte rotation every 4 rows;
//                  serves 16-byte row reads AND ds_read_b64_tr_b16 column
//                  reads.
// Both were chosen by enumerating strides/rotations against the 64-bank LDS
// so that the MFMA operand fetches (16-lane groups for 16-byte reads, 32-lane
// groups for 8-byte transpose reads) and the tile stores hit distinct banks.
// ---------------------------------------------------------------------------
template <int D, bool TR>
struct Pad {
  static constexpr int S = 2 * D + (TR ? 64 : 16);  // row stride, bytes
  __host__ __device__ static constexpr int rot(int r) { return TR ? 16 * ((r >> 2) & 3) : 0; }
  __host__ __device__ static constexpr int bytes(int rows) { return rows * S; }

  // Row read: lane (c32, g) fetches 16 bytes = k-slots of group g, i.e. the
  // columns 16*ks + 8*g .. +7 of row 32*blk + c32:  base + row_off(blk, ks).
  __device__ static int row_base(int c32, int g) { return c32 * S + rot(c32) + 16 * g; }
  __host__ __device__ static constexpr int row_off(int blk, int ks) { return 32 * blk * S + 32 * ks; }

  // Transpose read (ds_read_b64_tr_b16, two per operand).  Within a 16-lane
  // group, output lane i slot j is element (i % 4) of the 8 bytes addressed by
  // source lane 4j + i/4.  To give lane (c32, g) the column 32*mb + c32 of
  // the tokens 32*kb + 16*h + 8*(t/4) + 4*g + t%4 (slots t = 0..7, the
  // C-layout order of a 32-token block), source lane l = 16*G + 4*j + u
  // addresses token 32*kb + 16*h + 8*second + 4*g + j, columns
  // 32*mb + 16*(G%2) + 4*u .. +3.
  __device__ static int tr_base(int lane) {
    const int g = lane >> 5, j = (lane >> 2) & 3, u = lane & 3, half = (lane >> 4) & 1;
    return (4 * g + j) * S + 16 * g + 32 * half + 8 * u;
  }
  __host__ __device__ static constexpr int tr_off(int kb, int h, int second, int mb) {
    return (32 * kb + 16 * h + 8 * second) * S + 32 * second + 64 * mb;
  }
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;


// Value of lane 4*(lane/4) + i in every lane of the quad (DPP quad_perm
// broadcast; i is a compile-time constant after unrolling).
__device__ __forceinline__ float quad_bcast(float x, int i) {
  const int bits = __builtin_bit_cast(int, x);
  int r;
  switch (i) {
    case 0: r = __builtin_amdgcn_mov_dpp(bits, 0x00, 0xf, 0xf, true); break;
    case 1: r = __builtin_amdgcn_mov_dpp(bits, 0x55, 0xf, 0xf, true); break;
    case 2: r = __builtin_amdgcn_mov_dpp(bits, 0xaa, 0xf, 0xf, true); break;
    default: r = __builtin_amdgcn_mov_dpp(bits, 0xff, 0xf, 0xf, true); break;
  }
  return __builtin_bit_cast(float, r);
}

// ------------------------------------------------------------ dropout bits
// Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
// Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten
// rounds of two 32x32->64-bit multiplies by fixed constants, the high
// halves xor-ed into the other counter words together with the key, which
// is bumped by two Weyl constants between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
  // the multipliers in vector registers too (no scalar registers taken)
  uint32_t m0 = 0xD2511F53u, m1 = 0xCD9E8D57u;
  asm volatile("" : "+v"(m0), "+v"(m1));
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // high and low halves by separate multiplies (the fused 64-bit
    // multiply-add also writes a scalar carry register pair)
    u32x4 n;
    n[0] = __umulhi(m1, c[2]) ^ c[1] ^ k0;
    n[1] = m1 * c[2];
    n[2] = __umulhi(m0, c[0]) ^ c[3] ^ k1;
    n[3] = m0 * c[0];
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
    // keep the key schedule in two vector registers (bumped each round)
    // instead of twenty hoisted scalar constants
    asm volatile("" : "+v"(k0), "+v"(k1));
  }
  return c;
}

// 4x4 transpose of dwords across the four lanes of a quad: word c of lane
// a moves to word a of lane c.  Two exchange stages: words whose index
// differs from the lane in bit 1 swap with lane ^ 2 (word ^ 2), then those
// differing in bit 0 with lane ^ 1 (word ^ 1).
__device__ __forceinline__ u32x4 quad_transpose4(u32x4 w, int lane) {
  const bool b1 = (lane & 2) != 0, b0 = (lane & 1) != 0;
  u32x4 t, r;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t x = (uint32_t)__builtin_amdgcn_mov_dpp((int)w[c ^ 2], 0x4e, 0xf, 0xf, true);  // lane ^ 2
    t[c] = (((c >> 1) & 1) != (int)b1) ? x : w[c];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t x = (uint32_t)__builtin_amdgcn_mov_dpp((int)t[c ^ 1], 0xb1, 0xf, 0xf, true);  // lane ^ 1
    r[c] = ((c & 1) != (int)b0) ? x : t[c];
  }
  return r;
}

// 4x4 transpose of bytes within a lane: byte c of word b moves to byte b
// of word c.
__device__ __forceinline__ u32x4 byte_transpose4(u32x4 w) {
  u32x4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    r[c] = ((w[0] >> (8 * c)) & 0xffu) | (((w[1] >> (8 * c)) & 0xffu) << 8) |
           (((w[2] >> (8 * c)) & 0xffu) << 16) | (((w[3] >> (8 * c)) & 0xffu) << 24);
  return r;
}

// Keep decision of element v (0..15) of a lane whose dropout bytes are kb:
// byte v % 4 of word v / 4 at or above the drop threshold.
__device__ __forceinline__ bool keep_bit(const u32x4& kb, int v, uint32_t thr) {
  return ((kb[v >> 2] >> (8 * (v & 3))) & 0xffu) >= thr;
}
// The same decision as a bit mask (all ones: keep), formed with vector
// integer operations only, so no scalar condition registers are taken.
__device__ __forceinline__ uint32_t keep_mask(const u32x4& kb, int v, uint32_t thr) {
  const int byte = (int)((kb[v >> 2] >> (8 * (v & 3))) & 0xffu);
  return ~(uint32_t)((byte - (int)thr) >> 31);
}
__device__ __forceinline__ float masked(float x, uint32_t m) {
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) & m);
}

template <typename Tag>
__device__ __forceinline__ u32x4 pack8_keep(const f32x16& x, int base, const u32x4& kb, uint32_t thr) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = keep_bit(kb, base + i, thr) ? x[base + i] : 0.0f;
  u32x4 r;
  r[0] = pack2<Tag>(y[0], y[1]);
  r[1] = pack2<Tag>(y[2], y[3]);
  r[2] = pack2<Tag>(y[4], y[5]);
  r[3] = pack2<Tag>(y[6], y[7]);
  return r;
}

// 32-bit LDS pointers.  lds_opaque() hides a per-iteration base from the
// optimiser so constant offsets stay in the instructions' offset fields
// instead of being hoisted into one register per offset.
typedef __attribute__((address_space(3))) char lchar;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
__device__ __forceinline__ lchar* lds_ptr(char* p) { return (lchar*)p; }
__device__ __forceinline__ const lchar* lds_opaque(const lchar* p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass never runs this; its asm constraints are x86's
  asm volatile("" : "+v"(p));
#endif
  return p;
}
__device__ __forceinline__ u32x4 ld_row(const lchar* p) { return *(const lds_u32x4*)p; }

// One MFMA operand (8 slots) by two transpose reads.
__device__ __forceinline__ u32x4 ld_tr(const lchar* p0, const lchar* p1) {
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  const s16x8_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(u32x4, ab);
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane.  Issued
// through asm so the compiler does not track the LDS write: left to itself
// it makes the next LDS read wait for every outstanding DMA (vmcnt(0)),
// which would serialise the prefetch.  The caller orders the data with
// explicit vm_wait<>() and barriers.  (An M0 write needs one wait state
// before the DMA reads it.)
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
#endif
}
// Same, from a wave-uniform base plus a per-lane 32-bit byte offset (no
// 64-bit address arithmetic per lane).
__device__ __forceinline__ void dma16_s(const void* base, uint32_t off, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
#endif
}

// Global -> LDS staging without registers (global_load_lds_dwordx4: lane i
// of a wave writes its 16 bytes at M0 + 16*i).  The padded LDS image of a
// tile is cut into 1 KB blocks; block b is moved by wave b % NW, whose lane i
// fetches the 16 bytes that belong at block offset 16*i.  Every wave issues
// exactly kPer instructions per tile with every lane active: a lane whose
// destination is row padding or lies past the tile (bytes no operand fetch
// reads) loads the tile's first 16 bytes there, so outstanding-load counts
// are exact and uniform across waves.  Rows at or beyond the last valid row
// re-read it, so every load stays in bounds.  Completion is awaited with
// vm_wait<>() before the workgroup barrier.
template <int ROWS, int D, bool TR, int NW>
struct Dma {
  using L = Pad<D, TR>;
  static constexpr int kBytes = ROWS * L::S;
  static constexpr int kBlocks = (kBytes + 1023) / 1024;
  static constexpr int kPer = (kBlocks + NW - 1) / NW;   // DMA instructions per wave per tile
  static constexpr int kSlot = kPer * NW * 1024;         // LDS bytes reserved per tile
  int row[kPer];   // source row of instruction k's 16 bytes (0 for padding / past the tile)
  int colb[kPer];  // and its column, in bytes

  __device__ void init(int w, int lane) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int off = (w + NW * k) * 1024 + 16 * lane;
      int src = 0;  // element offset inside the tile
      if (off < kBytes) {
        const int r = off / L::S;
        const int p = off - r * L::S - L::rot(r);
        if (p >= 0 && p < 2 * D) src = r * D + p / 2;
      }
      row[k] = src / D;
      colb[k] = 2 * (src % D);
    }
  }
  // Instruction k of wave w's share of a tile, with the tile's addressing
  // hoisted by the caller (once per tile): t0 its first row, last its last
  // valid row (rows past it re-read it), rsb the source row stride in bytes
  // (below 2^24), lds_w the LDS byte address of the tile plus 1024 * w.
  __device__ __forceinline__ void issue_at(int k, const uint16_t* __restrict__ t0, int last, uint32_t rsb,
                                           uint32_t lds_w) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t off = __umul24((uint32_t)min(row[k], last), rsb) + colb[k];
    dma16_s(t0, off, lds_w + NW * k * 1024);
#endif
  }
};

// The K and V tiles of one ring slot as one run of 1 KB DMA blocks: the K
// image (row-read layout) first, the V image (transpose-read layout) from
// byte kBytesK on, block b moved by wave b % NW as in Dma.  One run wastes
// less LDS on block rounding than two Dma images.
template <int ROWS, int D, int NW>
struct DmaKV {
  using LK = Pad<D, false>;
  using LV = Pad<D, true>;
  static constexpr int kBytesK = ROWS * LK::S;
  static constexpr int kBytesV = ROWS * LV::S;
  static_assert(kBytesK % 1024 == 0, "K image in whole blocks");
  static constexpr int kBlocksK = kBytesK / 1024;
  static constexpr int kBlocks = kBlocksK + (kBytesV + 1023) / 1024;
  static constexpr int kPer = (kBlocks + NW - 1) / NW;  // DMA instructions per wave per tile
  static constexpr int kSlot = kPer * NW * 1024;        // LDS bytes reserved per slot
  int row[kPer];   // source row of instruction k's 16 bytes (0 for padding / past the images)
  int colb[kPer];  // and its column, in bytes
  bool isv[kPer];  // instruction k moves V (else K)

  __device__ void init(int w, int lane) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = w + NW * k;
      int src = 0;
      isv[k] = b >= kBlocksK;
      if (b < kBlocksK) {
        const int off = b * 1024 + 16 * lane;
        const int r = off / LK::S;
        const int p = off - r * LK::S - LK::rot(r);
        if (p >= 0 && p < 2 * D) src = r * D + p / 2;
      } else {
        const int off = (b - kBlocksK) * 1024 + 16 * lane;
        if (off < kBytesV) {
          const int r = off / LV::S;
          const int p = off - r * LV::S - LV::rot(r);
          if (p >= 0 && p < 2 * D) src = r * D + p / 2;
        }
      }
      row[k] = src / D;
      colb[k] = 2 * (src % D);
    }
  }
  // As Dma::issue_at, with the K and V tiles' first rows kt and vt (same
  // row stride and last valid row).
  __device__ __forceinline__ void issue_at(int k, const uint16_t* __restrict__ kt, const uint16_t* __restrict__ vt,
                                           int last, uint32_t rsb, uint32_t lds_w) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t off = __umul24((uint32_t)min(row[k], last), rsb) + colb[k];
    dma16_s(isv[k] ? vt : kt, off, lds_w + NW * k * 1024);
#endif
  }
};

// As Dma, for tile images packed back to back in LDS: the image takes
// exactly kBytes (a whole number of 1 KB blocks), and the instructions of
// the last round that have no block of the image left (block >= kBlocks)
// write to a caller-given 1 KB scratch block instead of past the image, so
// several images can sit next to each other without padding between them.
template <int ROWS, int D, bool TR, int NW>
struct DmaPacked {
  using L = Pad<D, TR>;
  static constexpr int kBytes = ROWS * L::S;
  static_assert(kBytes % 1024 == 0, "image in whole blocks");
  static constexpr int kBlocks = kBytes / 1024;
  static constexpr int kPer = (kBlocks + NW - 1) / NW;  // DMA instructions per wave per tile
  int row[kPer];    // source row of instruction k's 16 bytes (0 for padding)
  int colb[kPer];   // and its column, in bytes
  bool pad_last;    // this wave's last instruction has no block of the image

  __device__ void init(int w, int lane) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = w + NW * k;
      int src = 0;
      if (b < kBlocks) {
        const int off = b * 1024 + 16 * lane;
        const int r = off / L::S;
        const int p = off - r * L::S - L::rot(r);
        if (p >= 0 && p < 2 * D) src = r * D + p / 2;
      }
      row[k] = src / D;
      colb[k] = 2 * (src % D);
    }
    pad_last = w + NW * (kPer - 1) >= kBlocks;
  }
  // Instruction k of wave w's share: t0 the tile's first row, last its last
  // valid row, rsb the row stride in bytes, lds_w the LDS byte address of
  // the image plus 1024 * w, lds_pad that of the scratch block.  Only the
  // last round can hold padding.
  __device__ __forceinline__ void issue_at(int k, const uint16_t* __restrict__ t0, int last, uint32_t rsb,
                                           uint32_t lds_w, uint32_t lds_pad) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t off = __umul24((uint32_t)min(row[k], last), rsb) + colb[k];
    const bool pad = kBlocks % NW != 0 && k == kPer - 1 && pad_last;
    dma16_s(t0, off, pad ? lds_pad : lds_w + NW * k * 1024);
#endif
  }
};

// Wait until at most N of this wave's global loads (LDS DMA included) are
// outstanding; a workgroup barrier must follow before other waves read the
// data.  gfx9 s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt and
// lgkmcnt left at their "no wait" maxima.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// makes every wave first wait for its own outstanding LDS reads, which
// serialises the operand prefetch issued right before the barrier.  DMA
// completion is ordered by the vm_wait<>() in front of it; the memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_barrier" ::: "memory");
#endif
}

// ------------------------------------------------------------ block-mask tables
// The kept entries of one or two rows (or one column) of the block mask,
// built in LDS once per sweep: bits per row (is this tile's block kept for
// my rows?) and, for the union of the rows, the next kept entry at or after
// each entry.  Finding the next kept tile then costs one LDS read (counted
// by lgkmcnt) instead of global byte loads inside the sweep: a global load
// makes the wave wait on vmcnt, which also counts every outstanding tile
// DMA, so each lookup would drain the prefetch ring.
constexpr int kMaskMaxT = 2048;             // mask entries per row the kernels accept (< 4096)
constexpr int kMaskWords = kMaskMaxT / 64;  // LDS words per row of bits

typedef __attribute__((address_space(3))) uint64_t lds_u64;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// Wave w of nw fills words w, w + nw, ... with bit b = (src[b * stride] != 0)
// for b < T (0 beyond).  A workgroup barrier must follow before any wave
// reads the words.
__device__ __forceinline__ void mask_bits_build(lds_u64* words, const uint8_t* src, long stride, int T, int w, int nw,
                                                int lane) {
  for (int wd = w; wd < (T + 63) / 64; wd += nw) {
    const int b = 64 * wd + lane;
    const bool kept = b < T && src[(size_t)b * stride] != 0;
    const uint64_t bits = __builtin_amdgcn_ballot_w64(kept);
    if (lane == 0) words[wd] = bits;
  }
}
// After the bits are visible: thread t of nt fills entry e (e = t, t + nt,
// ...) of `table` with the smallest entry >= e kept in the bits at words
// (or, with rb >= 0, in their union with the bits at words + rb; T if none)
// in bits 0-11, and whether e itself is kept in the first row (bit 12) and
// in the second (bit 13).  A workgroup barrier must follow.
__device__ __forceinline__ void mask_table_build(lds_u16* table, const lds_u64* words, int rb, int T, int t, int nt) {
  const int nwd = (T + 63) >> 6;
  for (int e = t; e < T; e += nt) {
    int wd = e >> 6;
    auto word = [&](int i) { return rb >= 0 ? (words[i] | words[rb + i]) : words[i]; };
    uint64_t x = word(wd) & (~0ull << (e & 63));
    while (!x && ++wd < nwd) x = word(wd);
    const int nxt = x ? 64 * wd + (int)__builtin_ctzll(x) : T;
    const int k0 = (words[e >> 6] >> (e & 63)) & 1;
    const int k1 = rb >= 0 ? (words[rb + (e >> 6)] >> (e & 63)) & 1 : k0;
    table[e] = (uint16_t)(nxt | (k0 << 12) | (k1 << 13));
  }
}
// Table entry e (wave-uniform e < T).
__device__ __forceinline__ int mask_entry(const lds_u16* table, int e) {
  return __builtin_amdgcn_readfirstlane((int)table[e]);
}
// The next kept entry at or after e, and whether e is kept in row r (0, 1).
__device__ __forceinline__ int mask_next(const lds_u16* table, int e) { return mask_entry(table, e) & 0xfff; }
__device__ __forceinline__ bool mask_kept(const lds_u16* table, int r, int e) {
  return (mask_entry(table, e) >> (12 + r)) & 1;
}

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
