// Exact-attention backward for gfx950, 16-bit inputs.
//
// Recomputes S and P tile by tile from Q, K, V and the stored log-sum-exp L
// (P = exp(S - L), FlashAttention-2 notes eq. (16)) instead of reading an
// N x N matrix, and uses D_i = rowsum(dO o O) for the softmax Jacobian
// dS = P o (dP - D) (notes, Algorithm 2 and eqs. (17), (27)-(30); paper
// summary, Technique 2).
//
// Three launches on the caller's stream:
//  1. pre-pass   D = rowsum(dO o O) in float32 (memory bound);
//  2. dK/dV pass one workgroup per 128 keys (4 waves x 32 keys); the wave
//                keeps its K and V rows in registers and sweeps query tiles:
//                  S = Q K^T,  P = exp2(S c - L log2 e),  dP = dO V^T,
//                  dS = P o (dP - D),  dV^T += dO^T P,  dK^T += Q^T dS;
//                every row of P and dS is a register row, so P and dS feed
//                the dV/dK products as B operands without leaving registers;
//                Q and dO are staged once, row-major, and read both by rows
//                (for S, dP) and by LDS transpose reads (for dV, dK);
//  3. dQ pass    one workgroup per 256 queries (4 waves x 64 queries), the
//                forward's orientation: S^T = K Q^T, dP^T = V dO^T,
//                dS^T = P^T o (dP^T - D), dQ^T += K^T dS^T.
// dQ is computed in a separate pass instead of by cross-workgroup atomic
// adds (the pages' choice): no float32 dQ buffer, no atomics, and the result
// is deterministic; the cost is recomputing S and dP once more.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

constexpr int kNT = 256;
constexpr int kDqRows = 256;  // queries per dQ workgroup

// ------------------------------------------------------------ D pre-pass
template <typename Tag, int D>
__global__ __launch_bounds__(kNT) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dout,
                                                      float* __restrict__ dvec, long rows) {
  constexpr int TPR = D / 8;  // threads per row, 16 bytes each
  const long row = (long)blockIdx.x * (kNT / TPR) + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.0f;
  if (row < rows) {
    u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + 8 * c);
    u32x4 b = *reinterpret_cast<const u32x4*>(dout + row * D + 8 * c);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc = fmaf(to_f32<Tag>(a[t] & 0xffff), to_f32<Tag>(b[t] & 0xffff), acc);
      acc = fmaf(to_f32<Tag>(a[t] >> 16), to_f32<Tag>(b[t] >> 16), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) dvec[row] = acc;
}

// ------------------------------------------------------------ dK / dV pass
template <typename Tag, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kNT, 2) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BKV = 128;            // keys per workgroup (4 waves x 32)
  constexpr int BQ = 32;              // queries per tile
  constexpr int NQB = BQ / 32;        // 32-query blocks per tile
  constexpr int KS = D / 16;
  constexpr int NB = D / 32;
  constexpr int PK = BQ / 16;
  using TL = Pad<D, true>;            // Q and dO: row reads and transpose reads
  using QD = Dma<BQ, D, true, kNT / 64>;
  constexpr int TILE = QD::kSlot;     // LDS bytes per tile (DMA writes whole slots)
  constexpr int BUF = 2 * TILE + 2 * BQ * 4;  // Q, dO, L*log2e, D
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c32 = lane & 31, g = lane >> 5;
  const int n = a.n;
  const int lb = xcd_remap(blockIdx.x, a.nblk_kv);
  const int bh = lb / a.nkb;
  const int kb = lb % a.nkb;  // low key blocks see the most queries under causal
  const size_t hoff = (size_t)bh * n * D;
  const uint16_t* __restrict__ Qg = reinterpret_cast<const uint16_t*>(a.q) + hoff;
  const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + hoff;
  const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + hoff;
  const uint16_t* __restrict__ dOg = reinterpret_cast<const uint16_t*>(a.dout) + hoff;
  const float* __restrict__ Lg = a.lse + (size_t)bh * n;
  const float* __restrict__ Dg = a.dvec + (size_t)bh * n;

  const int k0 = kb * BKV;
  const int kw0 = k0 + w * 32;
  const int my_k = kw0 + c32;

  u32x4 kreg[KS], vreg[KS];
  {
    const size_t r = (size_t)min(my_k, n - 1) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kreg[ks] = *reinterpret_cast<const u32x4*>(Kg + r + 16 * ks);
      vreg[ks] = *reinterpret_cast<const u32x4*>(Vg + r + 16 * ks);
    }
  }

  const int n_tiles = (n + BQ - 1) / BQ;
  auto live = [&](int i) {
    if constexpr (SPARSE) return a.mask[(size_t)((i * BQ) / kMaskBlock) * a.mask_t + kb] != 0;
    return true;
  };
  auto next_tile = [&](int i) {
    ++i;
    while (i < n_tiles && !live(i)) ++i;
    return i;
  };

  QD dma;  // Q and dO tiles share one geometry
  dma.init(w, lane);
  float lv = 0.0f, dv = 0.0f;
  // issue the DMA of tile i into buffer b; L*log2(e) and D go through registers
  auto stage_ld = [&](int i, char* b) {
    dma.issue2(Qg + (size_t)i * BQ * D, dOg + (size_t)i * BQ * D, n - i * BQ, b, b + TILE);
    if (tid < BQ) {
      const int row = i * BQ + tid;
      const float L = row < n ? Lg[row] : -INFINITY;
      lv = (L == -INFINITY) ? INFINITY : L * kLog2e;  // rows with no keys get P = 0
      dv = row < n ? Dg[row] : 0.0f;
    }
  };
  auto stage_st = [&](char* b) {
    if (tid < BQ) {
      reinterpret_cast<float*>(b + 2 * TILE)[tid] = lv;
      reinterpret_cast<float*>(b + 2 * TILE + BQ * 4)[tid] = dv;
    }
  };
  const int rread = TL::row_base(c32, g);
  const int tread = TL::tr_base(lane);

  int i = CAUSAL ? k0 / BQ : 0;
  if (!live(i)) i = next_tile(i);
  if (i < n_tiles) {
    stage_ld(i, smem);
    stage_st(smem);
  }
  settle(kreg);
  settle(vreg);
  dma_wait();
  __syncthreads();

  f32x16 dkacc[NB], dvacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    dkacc[nb] = 0.0f;
    dvacc[nb] = 0.0f;
  }
  const float cs = a.c;
  int buf = 0;

  while (i < n_tiles) {
    const int in = next_tile(i);
    if (in < n_tiles) stage_ld(in, smem + (buf ^ 1) * BUF);
    const char* B = smem + buf * BUF;
    const char* qr = B + rread;
    const char* orr = B + TILE + rread;
    const char* qt = B + tread;
    const char* ot = B + TILE + tread;
    const float* Ls = reinterpret_cast<const float*>(B + 2 * TILE) + 4 * g;
    const float* Ds = reinterpret_cast<const float*>(B + 2 * TILE + BQ * 4) + 4 * g;
    const int q0 = i * BQ;
    const bool wave_live = !CAUSAL || (q0 + BQ - 1 >= kw0);
    if (wave_live) {
      f32x16 s[NQB], dp[NQB];
      const f32x16 zero = {};
#pragma unroll
      for (int mq = 0; mq < NQB; ++mq) {
        s[mq] = mfma32<Tag>(ld_row(qr + TL::row_off(mq, 0)), kreg[0], zero);
        dp[mq] = mfma32<Tag>(ld_row(orr + TL::row_off(mq, 0)), vreg[0], zero);
      }
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) {
#pragma unroll
        for (int mq = 0; mq < NQB; ++mq) {
          s[mq] = mfma32<Tag>(ld_row(qr + TL::row_off(mq, ks)), kreg[ks], s[mq]);
          dp[mq] = mfma32<Tag>(ld_row(orr + TL::row_off(mq, ks)), vreg[ks], dp[mq]);
        }
      }
      const bool need_mask = CAUSAL && (q0 < kw0 + 31);
#pragma unroll
      for (int mq = 0; mq < NQB; ++mq) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + 32 * mq + 8 * r4);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ds + 32 * mq + 8 * r4);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int v = 4 * r4 + t;
            float p = fast_exp2(fmaf(s[mq][v], cs, -l4[t]));
            if (need_mask && (my_k > q0 + 32 * mq + 8 * r4 + 4 * g + t)) p = 0.0f;
            s[mq][v] = p;
            dp[mq][v] = p * (dp[mq][v] - d4[t]);
          }
        }
      }
#pragma unroll
      for (int kk = 0; kk < PK; ++kk) {
        const int mq = kk >> 1, h = kk & 1;
        const u32x4 pb = pack8<Tag>(s[mq], 8 * h);
        const u32x4 db = pack8<Tag>(dp[mq], 8 * h);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          dvacc[nb] = mfma32<Tag>(ld_tr(ot + TL::tr_off(mq, h, 0, nb), ot + TL::tr_off(mq, h, 1, nb)), pb, dvacc[nb]);
          dkacc[nb] = mfma32<Tag>(ld_tr(qt + TL::tr_off(mq, h, 0, nb), qt + TL::tr_off(mq, h, 1, nb)), db, dkacc[nb]);
        }
      }
    }
    if (in < n_tiles) stage_st(smem + (buf ^ 1) * BUF);
    dma_wait();
    __syncthreads();
    buf ^= 1;
    i = in;
  }

  if (my_k < n) {
    uint16_t* dkp = reinterpret_cast<uint16_t*>(a.dk) + hoff + (size_t)my_k * D;
    uint16_t* dvp = reinterpret_cast<uint16_t*>(a.dv) + hoff + (size_t)my_k * D;
    const float sc = a.scale;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 pk, pv;
        pk[0] = pack2<Tag>(dkacc[nb][4 * r] * sc, dkacc[nb][4 * r + 1] * sc);
        pk[1] = pack2<Tag>(dkacc[nb][4 * r + 2] * sc, dkacc[nb][4 * r + 3] * sc);
        pv[0] = pack2<Tag>(dvacc[nb][4 * r], dvacc[nb][4 * r + 1]);
        pv[1] = pack2<Tag>(dvacc[nb][4 * r + 2], dvacc[nb][4 * r + 3]);
        *reinterpret_cast<u32x2*>(dkp + 32 * nb + 8 * r + 4 * g) = pk;
        *reinterpret_cast<u32x2*>(dvp + 32 * nb + 8 * r + 4 * g) = pv;
      }
  }
}

// ------------------------------------------------------------ dQ pass
// K/V tiles stream through a ring of kRing LDS slots filled by DMA kRing-1
// tiles ahead; each iteration waits (vmcnt) for its own tile, joins one
// barrier, refills the slot all waves have just finished reading, computes.
template <int C>
__device__ __forceinline__ void wait_ahead(int ahead) {  // ahead: tiles issued after the one needed
  if (ahead <= 0) vm_wait<0>();
  else if (ahead == 1) vm_wait<C>();
  else vm_wait<2 * C>();
}

// Each wave owns 64 queries, two 32-query blocks h = 0, 1, and runs one wave
// per SIMD (the operands take ~400 registers).  Within a wave the matrix
// cores and the vector ALU overlap only when their instructions are
// interleaved, and every step of a block depends on the previous one
// (S, dP -> dS -> dQ), so the wave software-pipelines its two blocks with
// block 0 one step ahead.  Iteration t (tile j_t, next tile j_{t+1}):
//   segment 1: products S^T, dP^T of (j_t, block 1)      | dS of (j_t, block 0)
//   segment 2: products dQ^T of (j_t, block 0),
//              S^T, dP^T of (j_{t+1}, block 0)           | dS of (j_t, block 1), DMA
//   segment 3: products dQ^T of (j_t, block 1)
// K/V tiles stream through a ring of four LDS slots; DMA runs two tiles
// ahead, one barrier per iteration makes the next tile visible and frees
// the slot refilled in the same iteration.
template <typename Tag, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kNT, 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BR = kDqRows;         // queries per workgroup (4 waves x 64)
  constexpr int BC = 32;              // keys per tile
  constexpr int KS = D / 16;          // k-steps of the S/dP products
  constexpr int MB = D / 32;          // 32-row blocks of dQ^T
  constexpr int PK = BC / 16;         // k-steps of the dQ products
  constexpr int NF = PK * MB;         // K^T fragments per tile
  constexpr int kRing = 4;
  using KL = Pad<D, true>;            // K: row reads (S^T) and transpose reads (dQ^T)
  using VL = Pad<D, false>;           // V: row reads (dP^T)
  using KD = Dma<BC, D, true, kNT / 64>;
  using VD = Dma<BC, D, false, kNT / 64>;
  constexpr int SLOT = KD::kSlot + VD::kSlot;
  constexpr int C = KD::kPer + VD::kPer;  // DMA instructions per wave per tile
  static_assert(3 * C < 64, "vmcnt range");
  static_assert(C <= NF, "DMA issue slots");
  __shared__ __attribute__((aligned(16))) char smem[kRing * SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so loop control stays scalar
  const int c32 = lane & 31, g = lane >> 5;
  const int n = a.n;
  const int lb = xcd_remap(blockIdx.x, a.nblk_q);
  const int bh = lb / a.nqb;
  const int qb = a.nqb - 1 - (lb % a.nqb);
  const size_t hoff = (size_t)bh * n * D;
  const uint16_t* __restrict__ Qg = reinterpret_cast<const uint16_t*>(a.q) + hoff;
  const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + hoff;
  const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + hoff;
  const uint16_t* __restrict__ dOg = reinterpret_cast<const uint16_t*>(a.dout) + hoff;

  const int q0 = qb * BR;
  const int qw0 = q0 + w * 64;        // the wave's first query; block h starts at qw0 + 32h

  u32x4 qreg[2][KS], oreg[2][KS];     // Q^T and dO^T fragments, in AGPRs
  float Lq[2], Dq[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int my_q = qw0 + 32 * h + c32;
    const int qr = min(my_q, n - 1);
    const size_t r = (size_t)qr * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      gload_agpr(qreg[h][ks], Qg + r + 16 * ks);
      gload_agpr(oreg[h][ks], dOg + r + 16 * ks);
    }
    const float l = a.lse[(size_t)bh * n + qr];
    Lq[h] = (l == -INFINITY || my_q >= n) ? INFINITY : l * kLog2e;
    Dq[h] = a.dvec[(size_t)bh * n + qr];
  }

  const int n_tiles = (n + BC - 1) / BC;
  int j_end = n_tiles;
  if constexpr (CAUSAL) j_end = min(n_tiles, (min(q0 + BR, n) - 1) / BC + 1);
  // block-sparse: the workgroup spans two 128-query mask rows, each wave one
  const uint8_t* mrow0 = nullptr;
  const uint8_t* mrow1 = nullptr;
  const uint8_t* mwave = nullptr;
  if constexpr (SPARSE) {
    const int t0 = q0 / kMaskBlock;
    const int t1 = min(t0 + 1, (n - 1) / kMaskBlock);
    mrow0 = a.mask + (size_t)t0 * a.mask_t;
    mrow1 = a.mask + (size_t)t1 * a.mask_t;
    mwave = (qw0 / kMaskBlock == t0) ? mrow0 : mrow1;
  }
  auto next_tile = [&](int j) {
    ++j;
    if constexpr (SPARSE)
      while (j < j_end && !(mrow0[(j * BC) / kMaskBlock] | mrow1[(j * BC) / kMaskBlock])) ++j;
    return j;
  };
  // tiles of this wave's queries that have allowed keys
  auto live = [&](int jt) {
    bool l = jt < j_end;
    if constexpr (CAUSAL) l = l && (jt * BC <= qw0 + 63);
    if constexpr (SPARSE) l = l && mwave[(jt * BC) / kMaskBlock];
    return l;
  };

  KD kd;
  VD vd;
  kd.init(w, lane);
  vd.init(w, lane);
  // DMA instruction i (of C) of tile jt into the slot at byte offset so
  auto dma = [&](int i, int jt, int so) {
    char* b = smem + so;
    if (i < KD::kPer) kd.issue_one(i, Kg + (size_t)jt * BC * D, n - jt * BC, b);
    else vd.issue_one(i - KD::kPer, Vg + (size_t)jt * BC * D, n - jt * BC, b + KD::kSlot);
  };
  const int krow = KL::row_base(c32, g);
  const int ktr = KL::tr_base(lane);
  const int vrow = KD::kSlot + VL::row_base(c32, g);
  auto slot_next = [&](int so) { return so + SLOT == kRing * SLOT ? 0 : so + SLOT; };

  vm_wait<0>();  // operand loads done: from here vmcnt counts DMA only

  const int j_first = SPARSE ? next_tile(-1) : 0;
  if (j_first >= j_end) {  // no key tile at all: dQ = 0
    for (int h = 0; h < 2; ++h) {
      const int my_q = qw0 + 32 * h + c32;
      if (my_q < n) {
        uint16_t* dqp = reinterpret_cast<uint16_t*>(a.dq) + hoff + (size_t)my_q * D;
        for (int c = 0; c < D; c += 8) *reinterpret_cast<u32x4*>(dqp + c) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    return;
  }
  // Every iteration issues exactly C DMA instructions (past the last tile
  // they reload the first tile into a slot nobody reads), so "tile t+1 has
  // landed" is always vmcnt <= C at the top of iteration t.
  int jq = j_first;  // next tile to load
  int sq = 0;        // its slot
  auto dma_tile = [&](int i) { dma(i, jq < j_end ? jq : j_first, sq); };
  auto dma_advance = [&]() {
    if (jq < j_end) jq = next_tile(jq);
    sq = slot_next(sq);
  };
  for (int t = 0; t < kRing - 1; ++t) {
#pragma unroll
    for (int i = 0; i < C; ++i) dma_tile(i);
    dma_advance();
  }

  f32x16 acc[2][MB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[h][mb] = 0.0f;
  const float cs = a.c;
  f32x16 s[2], dp[2];  // S^T and dP^T - D of one block; block 0 runs a tile ahead

  // S^T, dP^T of block h from the K/V slot at byte offset so
  auto sdp_first = [&](int h, int so) {  // no interleaved vector work
    const lchar* base = lds_ptr(smem) + so;
    const lchar* kr = lds_opaque(base + krow);
    const lchar* vr = lds_opaque(base + vrow);
    u32x4 kf[2], vf[2];
    kf[0] = ld_row(kr + KL::row_off(0, 0));
    vf[0] = ld_row(vr + VL::row_off(0, 0));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
        kf[(ks + 1) & 1] = ld_row(kr + KL::row_off(0, ks + 1));
        vf[(ks + 1) & 1] = ld_row(vr + VL::row_off(0, ks + 1));
      }
      if (ks == 0) {
        mfma32_vd<Tag, true, true>(s[h], kf[0], qreg[h][0]);
        mfma32_vd<Tag, true, true>(dp[h], vf[0], oreg[h][0]);
      } else {
        mfma32_vd<Tag, false, true>(s[h], kf[ks & 1], qreg[h][ks]);
        mfma32_vd<Tag, false, true>(dp[h], vf[ks & 1], oreg[h][ks]);
      }
    }
  };

  // the first tile's block-0 products, then the pipelined sweep
  vm_wait<2 * C>();
  __syncthreads();
  int j = j_first;
  int so = 0;  // slot of tile j
  if (!SPARSE || live(j)) sdp_first(0, so);

  auto step = [&](auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int jn = next_tile(j);
    const int son = slot_next(so);
    vm_wait<C>();      // tile jn has landed (for this wave's share) ...
    __syncthreads();   // ... for every wave; the slot refilled below is free
    // Dense sweeps compute every tile (the causal mask zeroes what lies past
    // the diagonal, and past the last tile the slot holds a valid reload), so
    // their loop body has no branch; sparse sweeps skip what the mask drops.
    const bool live_j = SPARSE ? live(j) : true;
    const bool live_n = SPARSE ? live(jn) : true;
    const int k0 = j * BC;
    const lchar* base = lds_ptr(smem) + so;
    const lchar* kr = lds_opaque(base + krow);
    const lchar* vr = lds_opaque(base + vrow);
    const lchar* kt = lds_opaque(base + ktr);
    u32x4 db[2][PK];
    // dS^T of block h, elements v0..v1-1 (row v of this lane's column)
    auto valu = [&](int h, int v0, int v1) {
#pragma unroll
      for (int v = v0; v < v1; ++v) {
        const float p = fast_exp2(fmaf(s[h][v], cs, -Lq[h]));
        float x = p * (dp[h][v] - Dq[h]);
        if constexpr (MASK) {
          // element v holds key k0 + 4g + 8(v/4) + v%4
          int last = n - 1;
          if constexpr (CAUSAL) last = min(last, qw0 + 32 * h + c32);
          x = (8 * (v >> 2) + (v & 3) > last - k0 - 4 * g) ? 0.0f : x;
        }
        dp[h][v] = x;
      }
    };
    auto pack = [&](int h) {
#pragma unroll
      for (int kk = 0; kk < PK; ++kk) db[h][kk] = pack8<Tag>(dp[h], 8 * kk);
    };
    auto zero = [&](int h) {
#pragma unroll
      for (int kk = 0; kk < PK; ++kk) db[h][kk] = 0u;
    };

    // DMA of the tile two ahead, spread over the iteration (one at a time
    // keeps the address unit from stalling every wave at once)
    auto dma_at = [&](int seg, int step, int nsteps) {
      constexpr int kPerSeg = (C + 2) / 3;
#pragma unroll
      for (int q = 0; q < kPerSeg; ++q) {
        const int i = seg * kPerSeg + q;
        if (i < C && step == (2 * q + 1) * nsteps / (2 * kPerSeg)) dma_tile(i);
      }
    };
    // S^T, dP^T of block h from the K/V rows at kr/vr; the fragments run kPD
    // k-steps ahead of the products; vec(ks) is interleaved vector work
    constexpr int kPD = 3;
    auto sdp = [&](int h, const lchar* rk, const lchar* rv, auto&& vec) {
      u32x4 kf[kPD + 1], vf[kPD + 1];
#pragma unroll
      for (int ks = 0; ks < kPD && ks < KS; ++ks) {
        kf[ks] = ld_row(rk + KL::row_off(0, ks));
        vf[ks] = ld_row(rv + VL::row_off(0, ks));
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + kPD < KS) {
          kf[(ks + kPD) % (kPD + 1)] = ld_row(rk + KL::row_off(0, ks + kPD));
          vf[(ks + kPD) % (kPD + 1)] = ld_row(rv + VL::row_off(0, ks + kPD));
        }
        const int r = ks % (kPD + 1);
        if (ks == 0) {
          mfma32_vd<Tag, true, true>(s[h], kf[r], qreg[h][0]);
          mfma32_vd<Tag, true, true>(dp[h], vf[r], oreg[h][0]);
        } else {
          mfma32_vd<Tag, false, true>(s[h], kf[r], qreg[h][ks]);
          mfma32_vd<Tag, false, true>(dp[h], vf[r], oreg[h][ks]);
        }
        vec(ks);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // ---- segment 1: S^T, dP^T (j, block 1) | dS (j, block 0)
    if (live_j) {
      sdp(1, kr, vr, [&](int ks) {
        valu(0, ks * 16 / KS, (ks + 1) * 16 / KS);
        dma_at(0, ks, KS);
      });
      pack(0);
    } else {
      for (int ks = 0; ks < KS; ++ks) dma_at(0, ks, KS);
      zero(0);
    }

    // ---- segment 2: S^T, dP^T (jn, block 0) | dS (j, block 1)
    if (live_n) {
      const lchar* nbase = lds_ptr(smem) + son;
      sdp(0, lds_opaque(nbase + krow), lds_opaque(nbase + vrow), [&](int ks) {
        if (ks == 0 && live_j) {  // block 1's S^T, dP^T complete before its vector work
          vgpr_drain(s);
          vgpr_drain(dp);
        }
        if (live_j) valu(1, ks * 16 / KS, (ks + 1) * 16 / KS);
        dma_at(1, ks, KS);
      });
    } else {
      if (live_j) {
        vgpr_drain(s);
        vgpr_drain(dp);
        valu(1, 0, 16);
      }
      for (int ks = 0; ks < KS; ++ks) dma_at(1, ks, KS);
    }
    if (live_j) pack(1);
    else zero(1);

    // ---- segment 3: dQ^T (j, blocks 0 and 1)
    u32x4 kq[kPD + 1];
#pragma unroll
    for (int f = 0; f < kPD && f < NF; ++f)
      kq[f] = ld_tr(kt + KL::tr_off(0, f / MB, 0, f % MB), kt + KL::tr_off(0, f / MB, 1, f % MB));
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f + kPD < NF) {
        const int fn = f + kPD;
        kq[fn % (kPD + 1)] = ld_tr(kt + KL::tr_off(0, fn / MB, 0, fn % MB), kt + KL::tr_off(0, fn / MB, 1, fn % MB));
      }
      mfma32_acc<Tag>(acc[0][f % MB], kq[f % (kPD + 1)], db[0][f / MB]);
      mfma32_acc<Tag>(acc[1][f % MB], kq[f % (kPD + 1)], db[1][f / MB]);
      dma_at(2, f, NF);
      __builtin_amdgcn_sched_barrier(0);
    }
    dma_advance();

    j = jn;
    so = son;
  };
  auto masked = [&](int jt) {
    return (CAUSAL && jt * BC + BC - 1 > qw0) || (jt * BC + BC > n);
  };
  // masked tiles come last: two loops over one body keep the accumulators
  // out of any branch (the register allocator would copy them there)
  while (j < j_end && !masked(j)) step(std::false_type{});
  while (j < j_end) step(std::true_type{});

  agpr_drain(acc[0]);
  agpr_drain(acc[1]);
  const float sc = a.scale;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int my_q = qw0 + 32 * h + c32;
    if (my_q < n) {
      uint16_t* dqp = reinterpret_cast<uint16_t*>(a.dq) + hoff + (size_t)my_q * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u32x2 pk;
          pk[0] = pack2<Tag>(acc[h][mb][4 * r] * sc, acc[h][mb][4 * r + 1] * sc);
          pk[1] = pack2<Tag>(acc[h][mb][4 * r + 2] * sc, acc[h][mb][4 * r + 3] * sc);
          *reinterpret_cast<u32x2*>(dqp + 32 * mb + 8 * r + 4 * g) = pk;
        }
    }
  }
}

template <typename Tag, int D, bool CAUSAL, bool SPARSE>
hipError_t launch_all(int bh, const BwdArgs& a, hipStream_t st) {
  const long rows = (long)bh * a.n;
  constexpr int rows_per_blk = kNT / (D / 8);
  timing_begin(kBwdPre, st);
  hipLaunchKernelGGL((bwd_pre_kernel<Tag, D>), dim3((rows + rows_per_blk - 1) / rows_per_blk), dim3(kNT),
                     0, st, reinterpret_cast<const uint16_t*>(a.o),
                     reinterpret_cast<const uint16_t*>(a.dout), a.dvec, rows);
  hipError_t e = hipGetLastError();
  timing_end(kBwdPre, st);
  if (e != hipSuccess) return e;
  timing_begin(kBwdDkDv, st);
  hipLaunchKernelGGL((bwd_dkdv_kernel<Tag, D, CAUSAL, SPARSE>), dim3(a.nblk_kv), dim3(kNT), 0, st, a);
  e = hipGetLastError();
  timing_end(kBwdDkDv, st);
  if (e != hipSuccess) return e;
  timing_begin(kBwdDq, st);
  hipLaunchKernelGGL((bwd_dq_kernel<Tag, D, CAUSAL, SPARSE>), dim3(a.nblk_q), dim3(kNT), 0, st, a);
  e = hipGetLastError();
  timing_end(kBwdDq, st);
  return e;
}

template <typename Tag, int D>
hipError_t launch_d(bool causal, bool sparse, int bh, const BwdArgs& a, hipStream_t st) {
  if (causal && sparse) return launch_all<Tag, D, true, true>(bh, a, st);
  if (causal) return launch_all<Tag, D, true, false>(bh, a, st);
  if (sparse) return launch_all<Tag, D, false, true>(bh, a, st);
  return launch_all<Tag, D, false, false>(bh, a, st);
}

}  // namespace

hipError_t launch_bwd(Dt dt, int d, bool causal, bool sparse, int bh, BwdArgs a, hipStream_t st) {
  a.nqb = (a.n + kDqRows - 1) / kDqRows;
  a.nblk_q = a.nqb * bh;
  a.nkb = (a.n + 127) / 128;
  a.nblk_kv = a.nkb * bh;
  if (dt == Dt::BF16) return d == 64 ? launch_d<bf16_tag, 64>(causal, sparse, bh, a, st)
                                     : launch_d<bf16_tag, 128>(causal, sparse, bh, a, st);
  return d == 64 ? launch_d<f16_tag, 64>(causal, sparse, bh, a, st)
                 : launch_d<f16_tag, 128>(causal, sparse, bh, a, st);
}

}  // namespace fa
