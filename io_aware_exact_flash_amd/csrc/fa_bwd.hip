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
//  3. dQ pass    one workgroup per 128 queries (4 waves x 32 queries), the
//                forward's orientation: S^T = K Q^T, dP^T = V dO^T,
//                dS^T = P^T o (dP^T - D), dQ^T += K^T dS^T.
// dQ is computed in a separate pass instead of by cross-workgroup atomic
// adds (the pages' choice): no float32 dQ buffer, no atomics, and the result
// is deterministic; the cost is recomputing S and dP once more.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

constexpr int kNT = 256;

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

template <typename Tag, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kNT, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BR = 128;
  constexpr int BC = 32;
  constexpr int KS = D / 16;
  constexpr int MB = D / 32;
  constexpr int PK = BC / 16;
  constexpr int kRing = 3;
  using KL = Pad<D, true>;            // K: row reads (S^T) and transpose reads (dQ^T)
  using VL = Pad<D, false>;           // V: row reads (dP^T)
  using KD = Dma<BC, D, true, kNT / 64>;
  using VD = Dma<BC, D, false, kNT / 64>;
  constexpr int SLOT = KD::kSlot + VD::kSlot;
  constexpr int C = KD::kPer + VD::kPer;  // DMA instructions per wave per tile
  static_assert(2 * C < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem[kRing * SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
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
  const int qw0 = q0 + w * 32;
  const int my_q = qw0 + c32;
  const int qr = min(my_q, n - 1);

  u32x4 qreg[KS], oreg[KS];
  {
    const size_t r = (size_t)qr * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qreg[ks] = *reinterpret_cast<const u32x4*>(Qg + r + 16 * ks);
      oreg[ks] = *reinterpret_cast<const u32x4*>(dOg + r + 16 * ks);
    }
  }
  float Lq = a.lse[(size_t)bh * n + qr];
  Lq = (Lq == -INFINITY || my_q >= n) ? INFINITY : Lq * kLog2e;
  const float Dq = a.dvec[(size_t)bh * n + qr];

  const int n_tiles = (n + BC - 1) / BC;
  int j_end = n_tiles;
  if constexpr (CAUSAL) j_end = min(n_tiles, (min(q0 + BR, n) - 1) / BC + 1);
  const uint8_t* mrow = SPARSE ? a.mask + (size_t)(q0 / kMaskBlock) * a.mask_t : nullptr;
  auto next_tile = [&](int j) {
    ++j;
    if constexpr (SPARSE)
      while (j < j_end && !mrow[(j * BC) / kMaskBlock]) ++j;
    return j;
  };

  KD kd;
  VD vd;
  kd.init(w, lane);
  vd.init(w, lane);
  auto issue = [&](int jt, int slot) {
    char* b = smem + slot * SLOT;
    kd.issue(Kg + (size_t)jt * BC * D, n - jt * BC, b);
    vd.issue(Vg + (size_t)jt * BC * D, n - jt * BC, b + KD::kSlot);
  };
  const int krow = KL::row_base(c32, g);
  const int ktr = KL::tr_base(lane);
  const int vrow = KD::kSlot + VL::row_base(c32, g);

  // settle the register loads before the DMA so waits below count only DMA
  settle(qreg);
  settle(oreg);
  int j = SPARSE ? next_tile(-1) : 0;
  int jq = j;       // next tile to issue
  int ahead = 0;    // tiles issued and not yet consumed
  for (int s = 0; s < kRing - 1 && jq < j_end; ++s) {
    issue(jq, s);
    jq = next_tile(jq);
    ++ahead;
  }

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = 0.0f;
  const float cs = a.c;
  int it = 0;

  while (j < j_end) {
    wait_ahead<C>(ahead - 1);
    __syncthreads();
    if (jq < j_end) {  // refill the slot every wave finished reading last iteration
      issue(jq, (it + kRing - 1) % kRing);
      jq = next_tile(jq);
      ++ahead;
    }
    const char* base = smem + (it % kRing) * SLOT;
    const char* kr = base + krow;
    const char* kt = base + ktr;
    const char* vr = base + vrow;
    const int k0 = j * BC;
    const bool wave_live = !CAUSAL || (k0 <= qw0 + 31);
    if (wave_live) {
      f32x16 s, dp;
      const f32x16 zero = {};
      s = mfma32<Tag>(ld_row(kr + KL::row_off(0, 0)), qreg[0], zero);
      dp = mfma32<Tag>(ld_row(vr + VL::row_off(0, 0)), oreg[0], zero);
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) {
        s = mfma32<Tag>(ld_row(kr + KL::row_off(0, ks)), qreg[ks], s);
        dp = mfma32<Tag>(ld_row(vr + VL::row_off(0, ks)), oreg[ks], dp);
      }
      const bool need_mask = (CAUSAL && (k0 + BC - 1 > qw0)) || (k0 + BC > n);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float p = fast_exp2(fmaf(s[v], cs, -Lq));
        if (need_mask) {
          const int key = k0 + 8 * (v >> 2) + 4 * g + (v & 3);
          bool dead = key >= n;
          if constexpr (CAUSAL) dead = dead || key > my_q;
          if (dead) p = 0.0f;
        }
        dp[v] = p * (dp[v] - Dq);
      }
#pragma unroll
      for (int kk = 0; kk < PK; ++kk) {
        const u32x4 db = pack8<Tag>(dp, 8 * kk);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = mfma32<Tag>(ld_tr(kt + KL::tr_off(0, kk, 0, mb), kt + KL::tr_off(0, kk, 1, mb)), db, acc[mb]);
      }
    }
    --ahead;
    ++it;
    j = next_tile(j);
  }

  if (my_q < n) {
    uint16_t* dqp = reinterpret_cast<uint16_t*>(a.dq) + hoff + (size_t)my_q * D;
    const float sc = a.scale;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 pk;
        pk[0] = pack2<Tag>(acc[mb][4 * r] * sc, acc[mb][4 * r + 1] * sc);
        pk[1] = pack2<Tag>(acc[mb][4 * r + 2] * sc, acc[mb][4 * r + 3] * sc);
        *reinterpret_cast<u32x2*>(dqp + 32 * mb + 8 * r + 4 * g) = pk;
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
  a.nqb = (a.n + 127) / 128;       // 128 queries per dQ workgroup
  a.nblk_q = a.nqb * bh;
  a.nkb = (a.n + 127) / 128;
  a.nblk_kv = a.nkb * bh;
  if (dt == Dt::BF16) return d == 64 ? launch_d<bf16_tag, 64>(causal, sparse, bh, a, st)
                                     : launch_d<bf16_tag, 128>(causal, sparse, bh, a, st);
  return d == 64 ? launch_d<f16_tag, 64>(causal, sparse, bh, a, st)
                 : launch_d<f16_tag, 128>(causal, sparse, bh, a, st);
}

}  // namespace fa
