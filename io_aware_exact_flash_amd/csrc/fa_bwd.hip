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
//                (for S, dP) and by LDS transpose reads (for dV, dK); the
//                tiles stream through a ring of five LDS slots with the
//                workgroup barrier between the S, dP products of the next
//                tile and the dV, dK products of the current one, so each
//                phase's first operand reads are issued during the phase
//                before it (with one wave per SIMD nothing else hides their
//                latency);
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
// Also writes the base-2 log-sum-exp L log2(e) the dK/dV pass subtracts,
// +inf for rows without any allowed key (so that P = exp2(S c - Lt) = 0).
// Workgroup x covers rows of query head x / blocks_per_head.
template <typename Tag, int D>
__global__ __launch_bounds__(kNT) void bwd_pre_kernel(BwdArgs args, int blocks_per_head) {
  constexpr int TPR = D / 8;  // threads per row, 16 bytes each
  constexpr int RPB = kNT / TPR;
  const int bh = blockIdx.x / blocks_per_head;
  const int row = (blockIdx.x % blocks_per_head) * RPB + threadIdx.x / TPR;
  const HeadAt at = query_head(args.sq, bh, args.n);
  const int c = threadIdx.x % TPR;
  const uint16_t* __restrict__ o = reinterpret_cast<const uint16_t*>(args.o) + at.q;
  const uint16_t* __restrict__ dout = reinterpret_cast<const uint16_t*>(args.dout) + at.q;
  const size_t ro = (size_t)min(row, max(at.n - 1, 0)) * args.sq.qsr + 8 * c;
  float acc = 0.0f;
  if (row < at.n) {
    u32x4 a = *reinterpret_cast<const u32x4*>(o + ro);
    u32x4 b = *reinterpret_cast<const u32x4*>(dout + ro);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc = fmaf(to_f32<Tag>(a[t] & 0xffff), to_f32<Tag>(b[t] & 0xffff), acc);
      acc = fmaf(to_f32<Tag>(a[t] >> 16), to_f32<Tag>(b[t] >> 16), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < at.n && c == 0) {
    args.dvec[at.l + row] = acc;
    const float l = args.lse[at.l + row];
    args.lt[at.l + row] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
}

// ------------------------------------------------------------ dK / dV pass
// One workgroup per 128 keys, four waves of 32 keys, one wave per SIMD.  A
// wave keeps its K^T and V^T fragments and its dK^T, dV^T accumulators in
// AGPRs and sweeps the query tiles (32 queries), which stream through a ring
// of four LDS slots by DMA two tiles ahead (Q and dO row-major and padded,
// read by rows for S, dP and by transpose reads for dV, dK; plus the
// tile's base-2 LSE and D).  Per tile:
//   S = Q K^T, dP - D = dO V^T, P = exp2(S c - Lt), dS = P o (dP - D),
//   dV^T += dO^T P, dK^T += Q^T dS.
// Every row of P and dS is a register row (the lane holds one key), so they
// feed the dV/dK products as B operands without leaving registers.  The
// sweep is software-pipelined by one tile: S, dP of the next tile run
// interleaved with the vector work (P, dS) of the current one.
template <typename Tag, int D, bool CAUSAL, bool SPARSE, bool DROP = false>
__global__ __launch_bounds__(kNT, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BKV = 128;            // keys per workgroup (4 waves x 32)
  constexpr int BQ = 32;              // queries per tile
  constexpr int KS = D / 16;          // k-steps of the S/dP products
  constexpr int NB = D / 32;          // 32-row blocks of dK^T / dV^T
  constexpr int PK = BQ / 16;         // k-steps of the dK/dV products
  constexpr int NF = PK * NB;         // transpose fragments per operand per tile
  constexpr int kRing = 5;
  using TL = Pad<D, true>;            // Q and dO tiles: row reads and transpose reads
  // At d = 64 the Q and dO images sit back to back (the DMA's padding
  // instructions write a 1 KB scratch block), which keeps the five slots
  // small enough for two workgroups per compute unit where the registers
  // allow it (the block-sparse variant); at d = 128 (one workgroup per unit
  // in any case, and no scalar registers to spare) each image is padded to
  // whole rounds of the four waves' blocks.
  constexpr bool kPacked = D == 64;
  using QD = std::conditional_t<kPacked, DmaPacked<BQ, D, true, kNT / 64>, Dma<BQ, D, true, kNT / 64>>;
  constexpr int kImg = kPacked ? BQ * TL::S : QD::kPer * kNT / 64 * 1024;  // LDS bytes per image
  constexpr int LDO = kImg;                 // dO tile within a slot
  constexpr int LPAD = 2 * kImg;            // scratch block of the packed images
  constexpr int LLD = LPAD + (kPacked ? 1024 : 0);  // base-2 LSE (32 floats) then D (32 floats)
  constexpr int SLOT = LLD + 256;
  constexpr int C = 2 * QD::kPer + 1;       // DMA instructions per wave per tile
  static_assert((kRing - 1) * C < 64, "vmcnt range");
  static_assert(SLOT % 256 == 0, "slot alignment");
  __shared__ __attribute__((aligned(256))) char smem[kRing * SLOT];
  __shared__ uint64_t mbits[SPARSE ? kMaskWords : 1];  // kept mask blocks of this key block's column
  __shared__ uint16_t mnext[SPARSE ? kMaskMaxT : 1];   // next kept block, kept flag

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so loop control stays scalar
  const int c32 = lane & 31, g = lane >> 5;
  // Causal: workgroup p of a head runs the key blocks p and nkb-1-p one
  // after the other, so every workgroup sees the same number of query
  // tiles (low key blocks see the most queries).  The grid covers the
  // longest sequence; a shorter one leaves workgroups idle.
  const int per = CAUSAL ? (a.nkb + 1) / 2 : a.nkb;
  const int lb = xcd_remap(blockIdx.x, a.nblk_kv);
  const int unit = lb / per;
  const int pk_ = lb % per;
  const int bh = unit / a.hsplit;   // K/V head, an index over B x Hkv
  const int rng = unit % a.hsplit;  // range of the group's query heads
  // the group's first query head locates the K/V head and the sequence
  const HeadAt at = group_head(a.sq, bh, a.hkv, a.n);
  const int n = at.n;  // this sequence's length
  const int qsr = a.sq.qsr, ksr = a.sq.ksr;
  const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + at.kv;
  const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + at.kv;
  // Grouped heads: the grp consecutive query heads that read this K/V head
  // each contribute to dK and dV; the workgroup sweeps those of its range
  // one after the other into the same accumulators.  With several ranges
  // (a.hsplit > 1) it writes float32 partial sums that a reduction pass
  // adds up.
  const int grp = a.sq.grp;
  const int h_lo = rng * grp / a.hsplit;
  const int h_hi = (rng + 1) * grp / a.hsplit;
  const bool partial = a.hsplit > 1;
  const size_t poff = ((size_t)rng * a.nbhkv + bh) * a.n * D;  // this range's partial dK, dV
  const uint16_t* Qg = nullptr;
  const uint16_t* dOg = nullptr;
  const float* Ltg = nullptr;
  const float* Dg = nullptr;
  int hcan = 0;  // b*H + h of the current query head (dropout counter)
  int hcan0 = 0;
  // dropout parameters, held in vector registers (scalar registers are
  // the scarcer file in this kernel)
  uint32_t d_k0 = a.drop.k0, d_k1 = a.drop.k1, d_off = a.drop.offset, d_thr = a.drop.thr;
  float d_scale = a.drop.scale;
  if constexpr (DROP) {
    int b_, hk_;
    split_bh(a.sq, bh, a.hkv, b_, hk_);
    hcan0 = b_ * a.sq.hq + hk_ * grp;
    asm volatile("" : "+v"(d_k0), "+v"(d_k1), "+v"(d_off), "+v"(d_thr), "+v"(d_scale), "+v"(hcan0));
  }
  auto set_head = [&](int hg) {  // query head hg of the group
    hcan = hcan0 + hg;
    const long long qo = at.q + hg * a.sq.qsh;
    const long long lo = at.l + hg * a.sq.lh;
    Qg = reinterpret_cast<const uint16_t*>(a.q) + qo;
    dOg = reinterpret_cast<const uint16_t*>(a.dout) + qo;
    Ltg = a.lt + lo;
    Dg = a.dvec + lo;
  };

  auto run = [&](const int kb) {
    const int k0 = kb * BKV;
    const int kw0 = k0 + w * 32;
    const int my_k = kw0 + c32;

    u32x4 kreg[KS], vreg[KS];  // K^T, V^T fragments (B operands), in AGPRs
    {
      const size_t r = (size_t)min(my_k, n - 1) * ksr + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        gload_agpr(kreg[ks], Kg + r + 16 * ks);
        gload_agpr(vreg[ks], Vg + r + 16 * ks);
      }
    }
    vm_wait<0>();  // operand loads done: from here vmcnt counts DMA only

    const int n_tiles = (n + BQ - 1) / BQ;
    // block-sparse: the kept entries of this key block's mask column, as
    // bits in LDS (built once)
    constexpr int TPB = kMaskBlock / BQ;  // query tiles per mask block
    lds_u64* mb = (lds_u64*)mbits;
    lds_u16* mn = (lds_u16*)mnext;
    if constexpr (SPARSE) {
      mask_bits_build(mb, a.mask + kb, a.mask_t, a.mask_t, w, kNT / 64, lane);
      __syncthreads();
      mask_table_build(mn, mb, -1, a.mask_t, 64 * w + lane, kNT);
      __syncthreads();
    }
    auto tile_live = [&](int i) {
      if constexpr (SPARSE) return mask_kept(mn, 0, i / TPB);
      return true;
    };
    auto next_tile = [&](int i) {
      ++i;
      if constexpr (SPARSE)
        if (i < n_tiles) i = min(max(i, TPB * mask_next(mn, i / TPB)), n_tiles);
      return i;
    };
    int i_first = CAUSAL ? k0 / BQ : 0;
    if (!tile_live(i_first)) i_first = next_tile(i_first);
    if (i_first >= n_tiles) {  // no query sees these keys: dK = dV = 0
      if (my_k < n && partial) {
        float* dkp = a.pdk + poff + (size_t)my_k * D;
        float* dvp = a.pdv + poff + (size_t)my_k * D;
        for (int c = 4 * g; c < D; c += 8) {
          *reinterpret_cast<f32x4*>(dkp + c) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          *reinterpret_cast<f32x4*>(dvp + c) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
      } else if (my_k < n) {
        uint16_t* dkp = reinterpret_cast<uint16_t*>(a.dk) + at.kv + (size_t)my_k * ksr;
        uint16_t* dvp = reinterpret_cast<uint16_t*>(a.dv) + at.kv + (size_t)my_k * ksr;
        for (int c = 8 * g; c < D; c += 16) {
          *reinterpret_cast<u32x4*>(dkp + c) = u32x4{0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(dvp + c) = u32x4{0u, 0u, 0u, 0u};
        }
      }
      return;
    }

    QD qd;  // Q and dO tiles share one geometry
    qd.init(w, lane);
    // DMA instruction t (of C) of tile it into the slot at byte offset so:
    // Q and dO share the tile geometry; the last one moves the tile's base-2
    // LSE (lanes 0-7) and D (lanes 8-15), four rows per lane.  A lane whose
    // rows start past the end reads the last row instead (those rows are
    // dead); one that straddles the end reads up to 3 floats past it, which
    // the workspace's spare bytes cover.
    // (The addressing of the tile being loaded is set once per tile, in
    // dma_set() below.)
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds_ptr(smem);
    const uint16_t* d_q = nullptr;
    const uint16_t* d_o = nullptr;
    const float* d_ld = nullptr;  // this lane's L or D source (lanes 0-15)
    int d_last = 0;
    uint32_t d_lds = 0, d_slot = 0;
    const int rrow = TL::row_base(c32, g);
    const int rtr = TL::tr_base(lane);
    auto slot_next = [&](int so) { return so + SLOT == kRing * SLOT ? 0 : so + SLOT; };

    // Every iteration issues exactly C DMA instructions (past the last tile
    // they reload the first tile into a slot nobody reads), so "tile t+1 has
    // landed" is always vmcnt <= C at the top of iteration t.
    int iq = i_first;  // next tile to load
    int sq = 0;        // its slot
    auto dma_set = [&]() {
      const int it = iq < n_tiles ? iq : i_first;
      d_q = Qg + (size_t)it * BQ * qsr;
      d_o = dOg + (size_t)it * BQ * qsr;
      d_last = n - 1 - it * BQ;
      d_slot = lds_base + sq;
      d_lds = d_slot + 1024 * w;
      d_ld = (lane < 8 ? Ltg : Dg) + min(it * BQ + 4 * (lane & 7), n - 1);
    };
    auto dma_tile = [&](int t) {
      if (t < 2 * QD::kPer) {
        const bool o = t >= QD::kPer;
        const int k = o ? t - QD::kPer : t;
        if constexpr (kPacked) qd.issue_at(k, o ? d_o : d_q, d_last, 2 * qsr, d_lds + (o ? LDO : 0), d_slot + LPAD);
        else qd.issue_at(k, o ? d_o : d_q, d_last, 2 * qsr, d_lds + (o ? LDO : 0));
      } else if (lane < 16) {
        dma16(d_ld, d_slot + LLD);
      }
    };
    auto dma_advance = [&]() {
      if (iq < n_tiles) iq = next_tile(iq);
      sq = slot_next(sq);
      dma_set();
    };

    f32x16 dkacc[NB], dvacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      dkacc[nb] = 0.0f;
      dvacc[nb] = 0.0f;
    }
    const float cs = a.c;
    // S and dP - D for two tiles: set X = the tile whose P, dS are being
    // formed, set Y = the next tile, whose products run meanwhile
    f32x16 s[2], dp[2];
    constexpr int kPD = 3;  // LDS fragments run kPD k-steps ahead of the products

    // S = Q K^T and dP = dO V^T for the tile in slot `so` into set Y, the two
    // accumulation chains interleaved (a single chain would wait out each
    // product's latency); vec(u) is vector work after product u (0 .. 2KS-1)
    // the first kPD row fragments of the next S, dP products, requested
    // ahead of them (at the end of the previous part B)
    u32x4 pq[kPD], po[kPD];
    auto prefetch_a = [&](int so) {
      const lchar* rq = lds_opaque(lds_ptr(smem) + so + rrow);
      const lchar* ro = lds_opaque(lds_ptr(smem) + so + LDO + rrow);
#pragma unroll
      for (int ks = 0; ks < kPD; ++ks) {
        pq[ks] = ld_row(rq + TL::row_off(0, ks));
        po[ks] = ld_row(ro + TL::row_off(0, ks));
      }
    };
    auto prod = [&](auto y_c, int so, auto&& vec) {
      constexpr int Y = decltype(y_c)::value;
      const lchar* rq = lds_opaque(lds_ptr(smem) + so + rrow);
      const lchar* ro = lds_opaque(lds_ptr(smem) + so + LDO + rrow);
      u32x4 fq[kPD + 1], fo[kPD + 1];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + kPD < KS) {
          fq[(ks + kPD) % (kPD + 1)] = ld_row(rq + TL::row_off(0, ks + kPD));
          fo[(ks + kPD) % (kPD + 1)] = ld_row(ro + TL::row_off(0, ks + kPD));
        }
        const int r = ks % (kPD + 1);
        const u32x4 aq = ks < kPD ? pq[ks] : fq[r];
        const u32x4 ao = ks < kPD ? po[ks] : fo[r];
        if (ks == 0) mfma32_vd<Tag, true, true>(s[Y], aq, kreg[0]);
        else mfma32_vd<Tag, false, true>(s[Y], aq, kreg[ks]);
        vec(2 * ks);
        __builtin_amdgcn_sched_barrier(0);
        if (ks == 0) mfma32_vd<Tag, true, true>(dp[Y], ao, vreg[0]);
        else mfma32_vd<Tag, false, true>(dp[Y], ao, vreg[ks]);
        vec(2 * ks + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    int i = i_first;  // the tile in set X
    int so = 0;       // its slot

    // Iteration over tile i (set X) with the next tile in (set Y = 1 - X):
    //   part A: S, dP of in                   | P, dS of i
    //   (barrier: the tile after in has landed; every wave is done with the
    //    previous iteration's part B, so its slot may be refilled)
    //   part B: dV^T, dK^T += ... of i        | DMA, the next part A's first fragments
    // A tile is visible from the barrier two iterations before it is X.
    auto step = [&](auto x_c, auto mask_c) {
      constexpr int X = decltype(x_c)::value;
      constexpr int Y = 1 - X;
      constexpr bool MASK = decltype(mask_c)::value;
      const int in = next_tile(i);
      const int son = slot_next(so);
      const int q0 = i * BQ;
      // dropout bytes of tile i: the quad's four lanes (keys 4m .. 4m+3)
      // draw the 4x4 blocks of queries 8a + 4g .. 8a + 4g + 3 (a = lane % 4);
      // a byte transpose and a word exchange leave each lane its own key's
      // 16 bytes in element order
      u32x4 kb;
      if constexpr (DROP) {
        const u32x4 ctr = {(uint32_t)(q0 / 4 + g + 2 * (c32 & 3)), (uint32_t)my_k >> 2, (uint32_t)hcan, d_off};
        kb = quad_transpose4(byte_transpose4(philox4x32_10(ctr, d_k0, d_k1)), lane);
      }
      const lchar* base = lds_ptr(smem) + so;
      // element v holds query q0 + 4g + 8(v/4) + v%4 (and this lane's key);
      // it is allowed while that offset lies in [lo, hi)
      const int lo = CAUSAL ? my_k - q0 - 4 * g : -BQ;
      const int hi = n - q0 - 4 * g;
      // element v needs the base-2 LSE and D of query 8(v/4) + 4g + v%4: the
      // LSE by four LDS reads; D by one read of group c32 % 4, the other groups
      // coming from the lanes of the quad by DPP broadcast folded into the
      // subtraction that uses them
      const lchar* ls = lds_opaque(base + LLD + 16 * g);
      f32x4 lt4[4];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) lt4[r4] = *(const __attribute__((address_space(3))) f32x4*)(ls + 32 * r4);
      const f32x4 dq4 = *(const __attribute__((address_space(3))) f32x4*)(ls + 128 + 32 * (c32 & 3));
      auto ltv = [&](int v) { return lt4[v >> 2][v & 3]; };
      auto dv = [&](int v) { return quad_bcast(dq4[v & 3], v >> 2); };
      // P and dS of element v in three stages, software-pipelined so that the
      // work after each product is three independent operations (a single
      // element's chain would stall on its own latencies while the matrix
      // core idles): t = S c - Lt, P = exp2(t), dS = P (dP - D) (+ mask).
      // The asm pins each finished element here, between the products.
      auto st1 = [&](int v) { s[X][v] = fmaf(s[X][v], cs, -ltv(v)); };
      auto st2 = [&](int v) { s[X][v] = fast_exp2(s[X][v]); };
      auto st3 = [&](int v) {
        float pp = s[X][v];
        float x;
        if constexpr (DROP) {  // dP = dP' Z / (1 - p) with dP' = dO V^T; dV takes P Z
          const uint32_t km = keep_mask(kb, v, d_thr);
          x = pp * fmaf(dp[X][v], masked(d_scale, km), -dv(v));
          pp = masked(pp, km);
        } else {
          x = pp * (dp[X][v] - dv(v));
        }
        if constexpr (MASK) {
          const int o = 8 * (v >> 2) + (v & 3);
          const bool dead = o < lo || o >= hi;
          pp = dead ? 0.0f : pp;
          x = dead ? 0.0f : x;
        }
        s[X][v] = pp;
        dp[X][v] = x;
        asm volatile("" : "+v"(s[X][v]), "+v"(dp[X][v]));
      };
      auto staged = [&](int u) {  // after product u: element u enters, u-2 leaves
        if (u < 16) st1(u);
        if (u >= 1 && u - 1 < 16) st2(u - 1);
        if (u >= 2 && u - 2 < 16) st3(u - 2);
      };
      // part B's first transpose fragments are requested during part A's
      // last products (tile i has been resident since the previous barrier)
      const lchar* ot = lds_opaque(base + LDO + rtr);
      const lchar* qt = lds_opaque(base + rtr);
      auto trf = [&](const lchar* t, int f) {
        return ld_tr(t + TL::tr_off(0, f / NB, 0, f % NB), t + TL::tr_off(0, f / NB, 1, f % NB));
      };
      u32x4 fo[kPD + 1], fq[kPD + 1];
      // ---- part A (16 elements over 2KS products: 1 or 2 per product)
      prod(std::integral_constant<int, Y>{}, son, [&](int u) {
        constexpr int R = 16 / (2 * KS);  // elements entering per product
#pragma unroll
        for (int e = 0; e < R; ++e) staged(u * R + e);
        if (u == 2 * KS - 2) {
#pragma unroll
          for (int f = 0; f < kPD && f < NF; ++f) {
            fo[f] = trf(ot, f);
            fq[f] = trf(qt, f);
          }
        }
      });
      staged(16);
      staged(17);
      u32x4 pb[PK], db[PK];
#pragma unroll
      for (int kk = 0; kk < PK; ++kk) {
        pb[kk] = pack8<Tag>(s[X], 8 * kk);
        db[kk] = pack8<Tag>(dp[X], 8 * kk);
      }
      valu_to_mfma(pb);
      valu_to_mfma(db);
      vm_wait<C>();   // the tile after `in` has landed (for this wave's share) ...
      wg_barrier();   // ... for every wave; the slot refilled below is free
      // ---- part B: dV^T += dO^T P, dK^T += Q^T dS (transpose fragments of tile i)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f + kPD < NF) {
          fo[(f + kPD) % (kPD + 1)] = trf(ot, f + kPD);
          fq[(f + kPD) % (kPD + 1)] = trf(qt, f + kPD);
        }
        mfma32_acc<Tag>(dvacc[f % NB], fo[f % (kPD + 1)], pb[f / NB]);
        mfma32_acc<Tag>(dkacc[f % NB], fq[f % (kPD + 1)], db[f / NB]);
#pragma unroll
        for (int t = 0; t < C; ++t)
          if (f == (2 * t + 1) * NF / (2 * C)) dma_tile(t);
        if (f == NF - 2) prefetch_a(slot_next(son));
        __builtin_amdgcn_sched_barrier(0);
      }
      dma_advance();
      i = in;
      so = son;
    };

    // Dense sweeps: the tiles crossing this wave's diagonal come first (an
    // even number, masked), then an even number without any per-element test,
    // then the rest (the sequence end), masked and padded to an even count
    // with a tile past the end (every row dead).  The total is the same for
    // every wave; two iterations per trip keep the sets X/Y in fixed roles
    // and the accumulators out of any branch.
#pragma clang loop unroll(disable)
    for (int hg = h_lo; hg < h_hi; ++hg) {
      // (formed per head from an opaque copy of n: hoisted out of the head
      // loop, these counts would hold scalar registers across the sweep)
      int n_pre = 0, n_plain = 0;
      if constexpr (!SPARSE) {
        int n_ = n;
        asm volatile("" : "+s"(n_));
        const int T = (n_ + BQ - 1) / BQ - i_first;
        if constexpr (CAUSAL) n_pre = min((w + 2) & ~1, (T + 1) & ~1);
        n_plain = max(n_ / BQ - (i_first + n_pre), 0) & ~1;
      }
      if (hg != h_lo) {
        vm_wait<0>();     // the previous head's DMA has landed ...
        __syncthreads();  // ... and every wave is out of its LDS tiles
      }
      set_head(hg);
      iq = i_first;
      sq = 0;
      dma_set();
      for (int t = 0; t < kRing - 1; ++t) {
#pragma unroll
        for (int u = 0; u < C; ++u) dma_tile(u);
        dma_advance();
      }
      // the first tile's products, then the pipelined sweep (the first two
      // tiles visible)
      vm_wait<(kRing - 3) * C>();
      __syncthreads();
      i = i_first;
      so = 0;
      prefetch_a(so);
      prod(std::integral_constant<int, 0>{}, so, [](int) {});
      prefetch_a(slot_next(so));
      vgpr_drain(s);
      vgpr_drain(dp);
      for (int t = 0; t < n_pre; t += 2) {
        step(std::integral_constant<int, 0>{}, std::true_type{});
        step(std::integral_constant<int, 1>{}, std::true_type{});
      }
      for (int t = 0; t < n_plain; t += 2) {
        step(std::integral_constant<int, 0>{}, std::false_type{});
        step(std::integral_constant<int, 1>{}, std::false_type{});
      }
      while (i < n_tiles) {
        step(std::integral_constant<int, 0>{}, std::true_type{});
        step(std::integral_constant<int, 1>{}, std::true_type{});
      }
    }

    agpr_drain(dkacc);
    agpr_drain(dvacc);
    if (my_k < n && partial) {
      float* dkp = a.pdk + poff + (size_t)my_k * D;
      float* dvp = a.pdv + poff + (size_t)my_k * D;
      const float sc = a.scale;
      const float sv = DROP ? d_scale : 1.0f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4 pk, pv;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            pk[t] = dkacc[nb][4 * r + t] * sc;
            pv[t] = dvacc[nb][4 * r + t] * sv;
          }
          *reinterpret_cast<f32x4*>(dkp + 32 * nb + 8 * r + 4 * g) = pk;
          *reinterpret_cast<f32x4*>(dvp + 32 * nb + 8 * r + 4 * g) = pv;
        }
    } else if (my_k < n) {
      uint16_t* dkp = reinterpret_cast<uint16_t*>(a.dk) + at.kv + (size_t)my_k * ksr;
      uint16_t* dvp = reinterpret_cast<uint16_t*>(a.dv) + at.kv + (size_t)my_k * ksr;
      const float sc = a.scale;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u32x2 pk, pv;
          pk[0] = pack2<Tag>(dkacc[nb][4 * r] * sc, dkacc[nb][4 * r + 1] * sc);
          pk[1] = pack2<Tag>(dkacc[nb][4 * r + 2] * sc, dkacc[nb][4 * r + 3] * sc);
          if constexpr (DROP) {
            const float sv = d_scale;
            pv[0] = pack2<Tag>(dvacc[nb][4 * r] * sv, dvacc[nb][4 * r + 1] * sv);
            pv[1] = pack2<Tag>(dvacc[nb][4 * r + 2] * sv, dvacc[nb][4 * r + 3] * sv);
          } else {
            pv[0] = pack2<Tag>(dvacc[nb][4 * r], dvacc[nb][4 * r + 1]);
            pv[1] = pack2<Tag>(dvacc[nb][4 * r + 2], dvacc[nb][4 * r + 3]);
          }
          *reinterpret_cast<u32x2*>(dkp + 32 * nb + 8 * r + 4 * g) = pk;
          *reinterpret_cast<u32x2*>(dvp + 32 * nb + 8 * r + 4 * g) = pv;
        }
    }
  };
  const int nkb = (n + BKV - 1) / BKV;  // this sequence's key blocks
  const int kb2 = nkb - 1 - pk_;
  // blocks pk_ and kb2 (paired causal), or pk_ alone; none past the end of
  // a shorter sequence
  const int nrun = CAUSAL ? (pk_ < kb2 ? 2 : pk_ == kb2 ? 1 : 0) : (pk_ < nkb ? 1 : 0);
#pragma clang loop unroll(disable)
  for (int r = 0; r < nrun; ++r) {
    if (r) {
      vm_wait<0>();      // the first block's DMA and stores are done ...
      __syncthreads();   // ... and every wave is out of its LDS tiles
    }
    run(r ? kb2 : pk_);
  }
}

// ------------------------------------------------------------ dK/dV range sum
// dK = sum over ranges of the float32 partials (already scaled), rounded to
// the input type once; dV likewise.  Thread i handles four consecutive
// elements of dK (i < n4) or dV; the partials are [range][B*Hkv][N][d]
// with N the longest sequence.  Memory bound: reads hsplit partials,
// writes one 16-bit result.
template <typename Tag, int D>
__global__ __launch_bounds__(kNT) void bwd_dkdv_reduce_kernel(BwdArgs a, long n4) {
  const long i = (long)blockIdx.x * kNT + threadIdx.x;
  if (i >= 2 * n4) return;
  const bool is_v = i >= n4;
  const long j = is_v ? i - n4 : i;
  const long row = j / (D / 4);
  const int c = 4 * (int)(j % (D / 4));
  const int bhkv = (int)(row / a.n);
  const int t = (int)(row % a.n);
  const HeadAt at = group_head(a.sq, bhkv, a.hkv, a.n);
  if (t >= at.n) return;  // past a shorter sequence
  const float* p = (is_v ? a.pdv : a.pdk) + row * D + c;
  f32x4 acc = *reinterpret_cast<const f32x4*>(p);
  for (int s = 1; s < a.hsplit; ++s) acc += *reinterpret_cast<const f32x4*>(p + (size_t)s * 4 * n4);
  u32x2 out;
  out[0] = pack2<Tag>(acc[0], acc[1]);
  out[1] = pack2<Tag>(acc[2], acc[3]);
  uint16_t* dst = reinterpret_cast<uint16_t*>(is_v ? a.dv : a.dk) + at.kv + (size_t)t * a.sq.ksr + c;
  *reinterpret_cast<u32x2*>(dst) = out;
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
// per SIMD (Q and dO fragments and the dQ accumulators fill the 256 AGPRs).
// Every K or V fragment read from LDS feeds both blocks' products, half the
// LDS traffic per product of a 32-query wave.  Within a wave the matrix
// cores and the vector ALU overlap only when their instructions are
// interleaved, and each tile's steps depend on each other (S, dP -> dS ->
// dQ), so the sweep is software-pipelined by one tile: the products S^T,
// dP^T of the next tile run interleaved with the softmax-gradient vector
// work of the current one.  K/V tiles stream through a ring of six LDS
// slots; DMA runs two tiles ahead, one barrier per iteration makes the next
// tile visible and frees the slot refilled in the same iteration.
// NW: waves per workgroup.  Block-sparse runs at d = 64 use two, so that a
// workgroup covers exactly one 128-row mask row (see fwd_kernel).
template <typename Tag, int D, bool CAUSAL, bool SPARSE, int NW = 4>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BR = NW * 64;         // queries per workgroup (NW waves x 64)
  constexpr int BC = 32;              // keys per tile
  constexpr int KS = D / 16;          // k-steps of the S/dP products
  constexpr int MB = D / 32;          // 32-row blocks of dQ^T
  constexpr int PK = BC / 16;         // k-steps of the dQ products
  constexpr int NF = PK * MB;         // K^T fragments per tile
  constexpr int kRing = 6;            // LDS tile slots
  using KL = Pad<D, true>;            // K: row reads (S^T) and transpose reads (dQ^T)
  using VL = Pad<D, false>;           // V: row reads (dP^T)
  using KD = Dma<BC, D, true, NW>;
  using VD = Dma<BC, D, false, NW>;
  constexpr int SLOT = KD::kSlot + VD::kSlot;
  constexpr int C = KD::kPer + VD::kPer;  // DMA instructions per wave per tile
  static_assert(4 * C < 64, "vmcnt range");
  static_assert(C / 2 <= NF - 1 && C - C / 2 <= 4 * KS - 2, "DMA issue slots");
  __shared__ __attribute__((aligned(16))) char smem[kRing * SLOT];
  __shared__ uint64_t mbits[SPARSE ? 2 * kMaskWords : 1];  // kept mask blocks of the two mask rows
  __shared__ uint16_t mnext[SPARSE ? kMaskMaxT : 1];       // next kept block, kept flags per row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so loop control stays scalar
  const int c32 = lane & 31, g = lane >> 5;
  // Causal: workgroup p of a head runs the query blocks nqb-1-p and p one
  // after the other (equal work for every workgroup).
  const int per = CAUSAL ? (a.nqb + 1) / 2 : a.nqb;
  const int lb = xcd_remap(blockIdx.x, a.nblk_q);
  const int bh = lb / per;
  const int pq_ = lb % per;
  const HeadAt at = query_head(a.sq, bh, a.n);
  const int n = at.n;  // this head's length
  const int qsr = a.sq.qsr, ksr = a.sq.ksr;
  const uint16_t* __restrict__ Qg = reinterpret_cast<const uint16_t*>(a.q) + at.q;
  const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + at.kv;
  const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + at.kv;
  const uint16_t* __restrict__ dOg = reinterpret_cast<const uint16_t*>(a.dout) + at.q;

  auto run = [&](const int qb) {
    const int q0 = qb * BR;
    const int qw0 = q0 + w * 64;        // the wave's first query; block h starts at qw0 + 32h

    u32x4 qreg[2][KS], oreg[2][KS];     // Q^T and dO^T fragments, in AGPRs
    float Lq[2], Dq[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int my_q = qw0 + 32 * h + c32;
      const int qr = min(my_q, n - 1);
      const size_t r = (size_t)qr * qsr + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        gload_agpr(qreg[h][ks], Qg + r + 16 * ks);
        gload_agpr(oreg[h][ks], dOg + r + 16 * ks);
      }
      const float l = a.lse[at.l + qr];
      Lq[h] = (l == -INFINITY || my_q >= n) ? INFINITY : l * kLog2e;
      Dq[h] = a.dvec[at.l + qr];
    }

    f32x16 negD[2];  // -D of each block's query, the dP^T accumulators' starting value
#pragma unroll
    for (int h = 0; h < 2; ++h) negD[h] = -Dq[h];
    const int n_tiles = (n + BC - 1) / BC;
    int j_end = n_tiles;
    if constexpr (CAUSAL) j_end = min(n_tiles, (min(q0 + BR, n) - 1) / BC + 1);
    // block-sparse: the workgroup spans one or two 128-query mask rows, each
    // wave lies in one of them; their kept entries go to LDS tables once
    // (kTable).  The causal block-sparse variant at d = 128 (no benchmark
    // shape) has no registers to spare for them and reads the mask bytes
    // from memory in the sweep instead.
    constexpr bool kTable = !(CAUSAL && D == 128);
    constexpr int TPB = kMaskBlock / BC;  // key tiles per mask block
    lds_u64* mb = (lds_u64*)mbits;
    lds_u16* mn = (lds_u16*)mnext;
    int mwave = 0;   // this wave's mask row: 0 or 1
    const uint8_t* mrow0 = nullptr;
    const uint8_t* mrow1 = nullptr;
    const uint8_t* mrw = nullptr;
    if constexpr (SPARSE) {
      const int t0 = q0 / kMaskBlock;
      const int t1 = min((q0 + BR - 1) / kMaskBlock, (n - 1) / kMaskBlock);
      if constexpr (kTable) {
        mask_bits_build(mb, a.mask + (size_t)t0 * a.mask_t, 1, a.mask_t, w, NW, lane);
        if (t1 != t0) mask_bits_build(mb + kMaskWords, a.mask + (size_t)t1 * a.mask_t, 1, a.mask_t, w, NW, lane);
        __syncthreads();
        mask_table_build(mn, mb, t1 != t0 ? kMaskWords : -1, a.mask_t, 64 * w + lane, NW * 64);
        __syncthreads();
        mwave = (qw0 / kMaskBlock == t0) ? 0 : 1;
      } else {
        mrow0 = a.mask + (size_t)t0 * a.mask_t;
        mrow1 = a.mask + (size_t)t1 * a.mask_t;
        mrw = (qw0 / kMaskBlock == t0) ? mrow0 : mrow1;
      }
    }
    // the next tile after j whose mask block either row keeps (j_end if none)
    auto next_tile = [&](int j) {
      ++j;
      if constexpr (SPARSE && kTable)
        if (j < j_end) j = min(max(j, TPB * mask_next(mn, j / TPB)), j_end);
      if constexpr (SPARSE && !kTable)
        while (j < j_end && !(mrow0[j / TPB] | mrow1[j / TPB])) ++j;
      return j;
    };
    // tiles of this wave's queries that have allowed keys
    auto live = [&](int jt) {
      bool l = jt < j_end;
      if constexpr (CAUSAL) l = l && (jt * BC <= qw0 + 63);
      if constexpr (SPARSE && kTable) l = l && mask_kept(mn, mwave, jt / TPB);
      if constexpr (SPARSE && !kTable) l = l && mrw[jt / TPB];
      return l;
    };

    KD kd;
    VD vd;
    kd.init(w, lane);
    vd.init(w, lane);
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
          uint16_t* dqp = reinterpret_cast<uint16_t*>(a.dq) + at.q + (size_t)my_q * qsr;
          for (int c = 0; c < D; c += 8) *reinterpret_cast<u32x4*>(dqp + c) = u32x4{0u, 0u, 0u, 0u};
        }
      }
      return;
    }
    // Every iteration issues exactly C DMA instructions (past the last tile
    // they reload the first tile into a slot nobody reads), so the tile
    // after the next one has landed once vmcnt <= C at the barrier.
    int jq = j_first;  // next tile to load
    int sq = 0;        // its slot
    // its addressing, set once per tile: K and V rows, last valid row, LDS
    // address of this wave's share
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds_ptr(smem);
    const uint16_t* dk = Kg;
    const uint16_t* dv = Vg;
    int d_last = 0;
    uint32_t d_lds = 0;
    auto dma_set = [&]() {
      const int jt = jq < j_end ? jq : j_first;
      dk = Kg + (size_t)jt * BC * ksr;
      dv = Vg + (size_t)jt * BC * ksr;
      d_last = n - 1 - jt * BC;
      d_lds = lds_base + sq + 1024 * w;
    };
    // DMA instruction i (of C) of the tile
    auto dma_tile = [&](int i) {
      if (i < KD::kPer) kd.issue_at(i, dk, d_last, 2 * ksr, d_lds);
      else vd.issue_at(i - KD::kPer, dv, d_last, 2 * ksr, d_lds + KD::kSlot);
    };
    auto dma_advance = [&]() {
      if (jq < j_end) jq = next_tile(jq);
      sq = slot_next(sq);
      dma_set();
    };
    // A tile's DMA is split: instructions 0..kDB-1 are issued in the B phase
    // of one iteration, the rest in the A phase of the next.
    constexpr int kDB = C / 2;
    dma_set();
    for (int t = 0; t < 3; ++t) {
#pragma unroll
      for (int i = 0; i < C; ++i) dma_tile(i);
      dma_advance();
    }
#pragma unroll
    for (int i = 0; i < kDB; ++i) dma_tile(i);

    f32x16 acc[2][MB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[h][mb] = 0.0f;
    const float cs = a.c;
    // S^T and dP^T - D of both blocks (turned into P and dS in place) for
    // two tiles, register sets by tile parity; packed dS^T likewise
    f32x16 s[2][2], dp[2][2];
    u32x4 db[2][2][PK];
    constexpr int kPD = SPARSE ? 4 : 5;  // LDS fragments run kPD products ahead (registers permitting)
    constexpr int kP = kPD < KS ? kPD : KS;   // row fragments in flight before a sweep
    constexpr int kPT = kPD < NF ? kPD : NF;  // K^T fragments in flight before phase B
    u32x4 fr[kPD + 1];  // K or V row fragments (ring)
    u32x4 kq[kPD + 1];  // K^T fragments (ring)
    auto rows_k = [&](int so) { return lds_opaque(lds_ptr(smem) + so + krow); };
    auto rows_v = [&](int so) { return lds_opaque(lds_ptr(smem) + so + vrow); };
    auto cols_k = [&](int so) { return lds_opaque(lds_ptr(smem) + so + ktr); };
    auto rd_k = [&](const lchar* r, int ks) { return ld_row(r + KL::row_off(0, ks)); };
    auto rd_v = [&](const lchar* r, int ks) { return ld_row(r + VL::row_off(0, ks)); };
    auto rd_kt = [&](const lchar* kt, int f) {
      return ld_tr(kt + KL::tr_off(0, f / MB, 0, f % MB), kt + KL::tr_off(0, f / MB, 1, f % MB));
    };
    auto prefetch_k = [&](int so) {
      const lchar* r = rows_k(so);
#pragma unroll
      for (int ks = 0; ks < kP; ++ks) fr[ks] = rd_k(r, ks);
    };
    // The dP sweep's first V fragments are read into the K ring during the
    // S sweep: fragment i goes to entry i once the last K fragment held
    // there (index kf(i)) has fed its products, i.e. after slot 2 kf(i) + 1.
    auto kf = [](int i) {
      int k = i;
      while (k + kPD + 1 < KS) k += kPD + 1;
      return k;
    };
    // V fragment reads after the product of slot u (u = 2 KS: after the sweep)
    auto prefetch_v_at = [&](const lchar* vr, int u) {
#pragma unroll
      for (int i = 0; i < kP; ++i)
        if (2 * kf(i) + 2 == u) fr[i] = rd_v(vr, i);
    };

    // One sweep of both blocks' products for the tile in slot `so` into set
    // Y, its first kP fragments already in flight: S^T = K Q^T (P = false)
    // or dP^T - D = V dO^T (P = true).  Every fragment feeds both blocks;
    // vec(u) is the vector work after product u = 2 ks + h.  (No VALU
    // instruction writes the operands: fragments come from LDS, Q^T and dO^T
    // from memory, -D is set once per block.)
    auto sweep = [&](auto y_c, auto p_c, int so, bool on, auto&& vec) {
      constexpr int Y = decltype(y_c)::value;
      constexpr bool P = decltype(p_c)::value;
      const lchar* rows = P ? rows_v(so) : rows_k(so);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + kPD < KS) fr[(ks + kPD) % (kPD + 1)] = P ? rd_v(rows, ks + kPD) : rd_k(rows, ks + kPD);
        const u32x4 f = fr[ks % (kPD + 1)];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (on) {
            f32x16& d = P ? dp[Y][h] : s[Y][h];
            const u32x4 b = P ? oreg[h][ks] : qreg[h][ks];
            if (ks == 0) {
              if (P) mfma32_vc<Tag>(d, f, b, negD[h]);  // dP^T - D accumulates from -D
              else mfma32_vd<Tag, true, true>(d, f, b);
            } else {
              mfma32_vd<Tag, false, true>(d, f, b);
            }
          }
          vec(2 * ks + h);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    // the first tile's products; its dS predecessor is zero
    vm_wait<C + kDB>();  // tiles 0 and 1 have landed (for this wave's share) ...
    __syncthreads();     // ... for every wave
    int j = j_first;
    int so = 0;  // slot of tile j
    int sp = 0;  // slot of the tile whose dQ products run next (none yet: any landed slot)
    {
      const bool on = !SPARSE || live(j);
      const lchar* vr = rows_v(so);
#pragma unroll
      for (int h = 0; h < 2; ++h) dp[0][h] = 0.0f;  // finite even where no product runs (dS = 0 * dP)
      prefetch_k(so);
      sweep(std::integral_constant<int, 0>{}, std::false_type{}, so, on, [&](int u) { prefetch_v_at(vr, u + 1); });
      prefetch_v_at(vr, 2 * KS);
      sweep(std::integral_constant<int, 0>{}, std::true_type{}, so, on, [](int) {});
    }
    vgpr_drain(s[0]);
    vgpr_drain(dp[0]);
#pragma unroll
    for (int h = 0; h < 2; ++h) dp[1][h] = 0.0f;
    int jn = next_tile(j);
    int sn = slot_next(so);
    prefetch_k(sn);

    // Iteration i (tile j = set X, its successor jn = set Y, its
    // predecessor jp in slot sp):
    //   A: S^T, dP^T of jn (VGPR products)
    //      | pack dS of jp; t = S^T c - L (+ mask) of j; DMA
    //   barrier (the tile after jn has landed; every wave is past A)
    //   B: dQ^T += K^T dS^T of jp (AGPR products)
    //      | P = exp2(t), dS = P (dP^T - D) of j; DMA
    // The exponentials share issue slots with AGPR-destination products
    // only: next to products that write VGPRs they issue markedly slower.
    // The body is unrolled for X = 0 and X = 1.  The tile count is the
    // workgroup's, so every wave runs every iteration: keys past a query's
    // diagonal or the sequence end get t = -inf, hence P = dS = 0.
    auto step = [&](auto x_c, auto mask_c) {
      constexpr int X = decltype(x_c)::value;
      constexpr int Y = 1 - X;
      constexpr bool MASK = decltype(mask_c)::value;
      // element v of block h of tile j holds key j*BC + 4g + 8(v/4) + v%4;
      // it is allowed while 8(v/4) + v%4 is at most lim[h]
      int lim[2];
      if constexpr (MASK) {
        const bool lv = SPARSE ? live(j) : true;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int last = n - 1;
          if constexpr (CAUSAL) last = min(last, qw0 + 32 * h + c32);
          lim[h] = lv ? last - j * BC - 4 * g : -1;
        }
      }
      const bool live_n = SPARSE ? live(jn) : true;
      // ---- A
      constexpr int NA = 4 * KS;        // product slots of phase A
      constexpr int RA = 32 / NA;       // elements of tile j per slot
      constexpr int RP = 8 * PK / (2 * KS);  // dS pairs of tile jp packed per slot of the S sweep
      auto va = [&](int u) {
#pragma unroll
        for (int r = 0; r < RA; ++r) {
          const int e = u * RA + r, h = e >> 4, v = e & 15;
          float t = fmaf(s[X][h][v], cs, -Lq[h]);
          if constexpr (MASK) t = (8 * (v >> 2) + (v & 3) > lim[h]) ? -INFINITY : t;
          s[X][h][v] = t;
        }
        if (u < 2 * KS) {
#pragma unroll
          for (int r = 0; r < RP; ++r) {
            const int q = u * RP + r, h = q / (4 * PK), kk = (q / 4) % PK, i = q & 3;
            db[Y][h][kk][i] = pack2<Tag>(dp[Y][h][8 * kk + 2 * i], dp[Y][h][8 * kk + 2 * i + 1]);
          }
        }
#pragma unroll
        for (int q = kDB; q < C; ++q)
          if (u == 1 + (q - kDB) * (NA - 2) / (C - kDB)) dma_tile(q);
      };
      const lchar* vrn = rows_v(sn);
      const lchar* ktp = cols_k(sp);
      sweep(std::integral_constant<int, Y>{}, std::false_type{}, sn, live_n, [&](int u) {
        va(u);
        prefetch_v_at(vrn, u + 1);
      });
      prefetch_v_at(vrn, 2 * KS);
      sweep(std::integral_constant<int, Y>{}, std::true_type{}, sn, live_n, [&](int u) {
        va(2 * KS + u);
        if (u >= 2 * KS - kPT) kq[u - (2 * KS - kPT)] = rd_kt(ktp, u - (2 * KS - kPT));
      });
      dma_advance();
      // ---- B, first products (independent of the barrier)
      auto dqp = [&](int f, int h) { mfma32_acc<Tag>(acc[h][f % MB], kq[f % (kPD + 1)], db[Y][h][f / MB]); };
      if (kPT < NF) kq[kPT % (kPD + 1)] = rd_kt(ktp, kPT);
      dqp(0, 0);
      dqp(0, 1);
      __builtin_amdgcn_sched_barrier(0);
      const int jnn = next_tile(jn);
      const int snn = slot_next(sn);
      vm_wait<C>();      // tile jnn has landed (for this wave's share) ...
      wg_barrier();      // ... for every wave; the slot refilled below is free
      // ---- B, the rest: element e (block e/16, row e%16) of tile j in two
      // stages one slot apart, P = exp2(t) then dS = P (dP^T - D).  Slot u
      // (2 .. 2NF-1) takes elements E(u-2) .. E(u-1)-1.
      auto stx = [&](int e) {
        const int h = e >> 4, v = e & 15;
        s[X][h][v] = fast_exp2(s[X][h][v]);
        asm volatile("" : "+v"(s[X][h][v]));
      };
      auto sty = [&](int e) {
        const int h = e >> 4, v = e & 15;
        dp[X][h][v] = s[X][h][v] * dp[X][h][v];
        asm volatile("" : "+v"(dp[X][h][v]));
      };
      constexpr int NS = 2 * NF - 2;
      auto E = [](int k) { return 32 * k / NS; };
      auto slot_work = [&](int u) {
        const int k = u - 2;
        if (k < NS)
          for (int e = E(k); e < E(k + 1); ++e) stx(e);
        if (k >= 1)
          for (int e = E(k - 1); e < E(k); ++e) sty(e);
      };
#pragma unroll
      for (int f = 1; f < NF; ++f) {
        if (f + kPT < NF) kq[(f + kPT) % (kPD + 1)] = rd_kt(ktp, f + kPT);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          dqp(f, h);
          slot_work(2 * f + h);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = 0; q < kDB; ++q)
          if (f == 1 + (2 * q + 1) * (NF - 1) / (2 * kDB)) dma_tile(q);
      }
      slot_work(2 * NF);
      prefetch_k(snn);
      sp = so;
      so = sn;
      sn = snn;
      j = jn;
      jn = jnn;
    };
    // Two iterations per trip keep the register sets in fixed roles.  The
    // sweep runs until the dQ products of the last tile are done; iterations
    // past it see no tile (all keys masked, slots holding valid reloads).
    // Dense sweeps start with the iterations whose tile j has no masked key
    // for this wave (keys below its diagonal and inside the sequence), an
    // even number of them, without any per-element test; the rest run with
    // the mask.  The total is the same for every wave.
    int n_plain = 0;
    if constexpr (!SPARSE) {
      int jm = n / BC;                                  // first tile reaching past the sequence end
      if constexpr (CAUSAL) jm = min(jm, qw0 / BC);    // first tile crossing the diagonal
      n_plain = max(jm - j_first, 0) & ~1;
    }
    for (int t = 0; t < n_plain; t += 2) {
      step(std::integral_constant<int, 0>{}, std::false_type{});
      step(std::integral_constant<int, 1>{}, std::false_type{});
    }
    // The iteration of tile j_end (the first past the last) runs the dQ
    // products of the last tile; the trip containing it is the last.
    do {
      step(std::integral_constant<int, 0>{}, std::true_type{});
      step(std::integral_constant<int, 1>{}, std::true_type{});
    } while (j <= j_end);

    agpr_drain(acc[0]);
    agpr_drain(acc[1]);
    const float sc = a.scale;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int my_q = qw0 + 32 * h + c32;
      if (my_q < n) {
        uint16_t* dqp = reinterpret_cast<uint16_t*>(a.dq) + at.q + (size_t)my_q * qsr;
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
  };
  const int nqb = (n + BR - 1) / BR;  // this head's query blocks
  const int qa = nqb - 1 - pq_;      // the longer block first
  const int nrun = CAUSAL ? (pq_ < qa ? 2 : pq_ == qa ? 1 : 0) : (qa >= 0 ? 1 : 0);
#pragma clang loop unroll(disable)
  for (int r = 0; r < nrun; ++r) {
    if (r) {
      vm_wait<0>();      // the first block's DMA and stores are done ...
      __syncthreads();   // ... and every wave is out of its LDS tiles
    }
    run(r ? pq_ : qa);
  }
}

// ------------------------------------------------------------ dQ pass with dropout
// dS^T = P^T o (dP'^T Z / (1 - p) - D) with dP'^T = V dO^T and Z the
// dropout decisions (drawn as in the forward: lane = query).  One wave per
// 32 queries (four per workgroup), K/V tiles of 32 keys in a ring of three
// LDS slots filled two tiles ahead, one barrier per tile; the small
// register and LDS footprint lets two workgroups (d = 128) or three
// (d = 64) share a compute unit, whose waves hide each other's latencies.
// Simpler than the pipelined pass above, whose registers leave no room for
// the dropout decisions.
constexpr int kDqDropRows = 128;

template <typename Tag, int D, bool CAUSAL>
__global__ __launch_bounds__(kNT, 1) void bwd_dq_drop_kernel(BwdArgs a) {
  constexpr int BC = 32;
  constexpr int KS = D / 16, MB = D / 32, PK = BC / 16, NF = PK * MB;
  using KL = Pad<D, true>;
  using VL = Pad<D, false>;
  using KD = Dma<BC, D, true, kNT / 64>;
  using VD = Dma<BC, D, false, kNT / 64>;
  constexpr int SLOT = KD::kSlot + VD::kSlot;
  constexpr int C = KD::kPer + VD::kPer;  // DMA instructions per wave per tile
  constexpr int kRing = 3;
  static_assert(2 * C < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem[kRing * SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, g = lane >> 5;
  const int nqb = (a.n + kDqDropRows - 1) / kDqDropRows;
  const int lb = xcd_remap(blockIdx.x, a.nblk_q);
  const int bh = lb / nqb;
  const HeadAt at = query_head(a.sq, bh, a.n);
  const int n = at.n;
  const int qb = (n + kDqDropRows - 1) / kDqDropRows - 1 - lb % nqb;  // the longest blocks first
  if (qb < 0) return;
  const int hcan = canon_head(a.sq, bh);
  const int qsr = a.sq.qsr, ksr = a.sq.ksr;
  const uint16_t* __restrict__ Qg = reinterpret_cast<const uint16_t*>(a.q) + at.q;
  const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + at.kv;
  const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + at.kv;
  const uint16_t* __restrict__ dOg = reinterpret_cast<const uint16_t*>(a.dout) + at.q;
  const int q0 = qb * kDqDropRows;
  const int qw0 = q0 + 32 * w;
  const int my_q = qw0 + c32;
  const int qr = min(my_q, n - 1);

  u32x4 qreg[KS], oreg[KS];  // Q^T, dO^T fragments (B operands), in AGPRs
  {
    const size_t r = (size_t)qr * qsr + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      gload_agpr(qreg[ks], Qg + r + 16 * ks);
      gload_agpr(oreg[ks], dOg + r + 16 * ks);
    }
  }
  const float l = a.lse[at.l + qr];
  const float Lq = (l == -INFINITY || my_q >= n) ? INFINITY : l * kLog2e;
  const float Dq = a.dvec[at.l + qr];
  vm_wait<0>();

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = 0.0f;
  const float cs = a.c;
  KD kd;
  VD vd;
  kd.init(w, lane);
  vd.init(w, lane);
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds_ptr(smem);
  const int n_tiles = (n + BC - 1) / BC;
  const int j_end = CAUSAL ? min(n_tiles, (min(q0 + kDqDropRows, n) - 1) / BC + 1) : n_tiles;
  // tile jt into slot jt % kRing (past the end: a reload of tile 0 into a
  // slot nobody reads, so every iteration issues C instructions)
  auto dma = [&](int jt) {
    const int tt = jt < j_end ? jt : 0;
    const uint16_t* kt = Kg + (size_t)tt * BC * ksr;
    const uint16_t* vt = Vg + (size_t)tt * BC * ksr;
    const int last = n - 1 - tt * BC;
    const uint32_t slot = lds_base + (jt % kRing) * SLOT + 1024 * w;
#pragma unroll
    for (int k = 0; k < KD::kPer; ++k) kd.issue_at(k, kt, last, 2 * ksr, slot);
#pragma unroll
    for (int k = 0; k < VD::kPer; ++k) vd.issue_at(k, vt, last, 2 * ksr, slot + KD::kSlot);
  };
  dma(0);
  dma(1);

  for (int j = 0; j < j_end; ++j) {
    vm_wait<C>();   // tile j has landed (for this wave's share; j + 1 may be in flight) ...
    wg_barrier();   // ... for every wave, and every wave is done with tile j - 1
    dma(j + 2);     // into tile j - 1's slot
    const int so = (j % kRing) * SLOT;
    const lchar* krows = lds_opaque(lds_ptr(smem) + so + KL::row_base(c32, g));
    const lchar* vrows = lds_opaque(lds_ptr(smem) + so + KD::kSlot + VL::row_base(c32, g));
    const lchar* kcols = lds_opaque(lds_ptr(smem) + so + KL::tr_base(lane));
    if (!(CAUSAL && j * BC > qw0 + 31)) {  // (else every key of the tile is after this wave's queries)

      f32x16 sv[1], dv[1];  // S^T, dP'^T
  #pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 fk = ld_row(krows + KL::row_off(0, ks));
        const u32x4 fv = ld_row(vrows + VL::row_off(0, ks));
        if (ks == 0) {
          mfma32_vd<Tag, true, true>(sv[0], fk, qreg[ks]);
          mfma32_vd<Tag, true, true>(dv[0], fv, oreg[ks]);
        } else {
          mfma32_vd<Tag, false, true>(sv[0], fk, qreg[ks]);
          mfma32_vd<Tag, false, true>(dv[0], fv, oreg[ks]);
        }
      }
      // dropout bytes of this lane's query row (drawn and exchanged as in
      // the forward)
      const u32x4 ctr = {(uint32_t)my_q >> 2, (uint32_t)(8 * j + g + 2 * (c32 & 3)), (uint32_t)hcan, a.drop.offset};
      const u32x4 kb = quad_transpose4(philox4x32_10(ctr, a.drop.k0, a.drop.k1), lane);
      vgpr_drain(sv);
      vgpr_drain(dv);
      // element v holds key j*BC + 4g + 8(v/4) + v%4
      const int lim = (CAUSAL ? min(n - 1, my_q) : n - 1) - j * BC - 4 * g;
      f32x16 ds;
  #pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool dead = 8 * (v >> 2) + (v & 3) > lim;
        const float p = dead ? 0.0f : fast_exp2(fmaf(sv[0][v], cs, -Lq));
        const float zs = masked(a.drop.scale, keep_mask(kb, v, a.drop.thr));
        ds[v] = p * fmaf(dv[0][v], zs, -Dq);
      }
      u32x4 db[PK];
  #pragma unroll
      for (int kk = 0; kk < PK; ++kk) db[kk] = pack8<Tag>(ds, 8 * kk);
      valu_to_mfma(db);
  #pragma unroll
      for (int f = 0; f < NF; ++f) {
        const u32x4 kt = ld_tr(kcols + KL::tr_off(0, f / MB, 0, f % MB), kcols + KL::tr_off(0, f / MB, 1, f % MB));
        mfma32_acc<Tag>(acc[f % MB], kt, db[f / MB]);
      }
    }
  }
  vm_wait<0>();  // the reloads issued past the last tile have landed

  agpr_drain(acc);
  if (my_q < n) {
    uint16_t* dqp = reinterpret_cast<uint16_t*>(a.dq) + at.q + (size_t)my_q * qsr;
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

// Waves per dQ workgroup (two for block-sparse runs at d = 64).
template <int D, bool SPARSE>
constexpr int dq_waves() { return (SPARSE && D == 64) ? 2 : 4; }

template <typename Tag, int D, bool CAUSAL, bool SPARSE, bool DROP = false>
hipError_t launch_all(int bh, const BwdArgs& a, hipStream_t st) {
  constexpr int rows_per_blk = kNT / (D / 8);
  const int blocks_per_head = (a.n + rows_per_blk - 1) / rows_per_blk;
  timing_begin(kBwdPre, st);
  hipLaunchKernelGGL((bwd_pre_kernel<Tag, D>), dim3((long)bh * blocks_per_head), dim3(kNT), 0, st, a,
                     blocks_per_head);
  hipError_t e = hipGetLastError();
  timing_end(kBwdPre, st);
  if (e != hipSuccess) return e;
  timing_begin(DROP ? kBwdDkDvDrop : kBwdDkDv, st);
  hipLaunchKernelGGL((bwd_dkdv_kernel<Tag, D, CAUSAL, SPARSE, DROP>), dim3(a.nblk_kv), dim3(kNT), 0, st, a);
  e = hipGetLastError();
  timing_end(DROP ? kBwdDkDvDrop : kBwdDkDv, st);
  if (e != hipSuccess) return e;
  if (a.hsplit > 1) {
    const long n4 = (long)a.nbhkv * a.n * (D / 4);
    timing_begin(kBwdDkDvReduce, st);
    hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<Tag, D>), dim3((2 * n4 + kNT - 1) / kNT), dim3(kNT), 0, st, a,
                       n4);
    e = hipGetLastError();
    timing_end(kBwdDkDvReduce, st);
    if (e != hipSuccess) return e;
  }
  if constexpr (DROP) {
    BwdArgs b = a;
    b.nblk_q = (a.n + kDqDropRows - 1) / kDqDropRows * bh;
    timing_begin(kBwdDqDrop, st);
    hipLaunchKernelGGL((bwd_dq_drop_kernel<Tag, D, CAUSAL>), dim3(b.nblk_q), dim3(kNT), 0, st, b);
    e = hipGetLastError();
    timing_end(kBwdDqDrop, st);
  } else {
    constexpr int NWQ = dq_waves<D, SPARSE>();
    timing_begin(kBwdDq, st);
    hipLaunchKernelGGL((bwd_dq_kernel<Tag, D, CAUSAL, SPARSE, NWQ>), dim3(a.nblk_q), dim3(64 * NWQ), 0, st, a);
    e = hipGetLastError();
    timing_end(kBwdDq, st);
  }
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

template <typename Tag, int D>
hipError_t launch_drop_d(bool causal, int bh, const BwdArgs& a, hipStream_t st) {
  return causal ? launch_all<Tag, D, true, false, true>(bh, a, st) : launch_all<Tag, D, false, false, true>(bh, a, st);
}

static void grid_sizes(bool causal, bool sparse, int d, int bh, BwdArgs& a) {
  const int rows = (sparse && d == 64) ? 64 * dq_waves<64, true>() : kDqRows;
  a.nqb = (a.n + rows - 1) / rows;
  a.nblk_q = (causal ? (a.nqb + 1) / 2 : a.nqb) * bh;
  a.nkb = (a.n + 127) / 128;
  a.nblk_kv = (causal ? (a.nkb + 1) / 2 : a.nkb) * (bh / a.sq.grp) * a.hsplit;  // per K/V head and range
}

hipError_t launch_bwd_dropout(Dt dt, int d, bool causal, int bh, BwdArgs a, hipStream_t st) {
  grid_sizes(causal, false, d, bh, a);
  if (dt == Dt::BF16) return d == 64 ? launch_drop_d<bf16_tag, 64>(causal, bh, a, st)
                                     : launch_drop_d<bf16_tag, 128>(causal, bh, a, st);
  return d == 64 ? launch_drop_d<f16_tag, 64>(causal, bh, a, st) : launch_drop_d<f16_tag, 128>(causal, bh, a, st);
}

hipError_t launch_bwd(Dt dt, int d, bool causal, bool sparse, int bh, BwdArgs a, hipStream_t st) {
  grid_sizes(causal, sparse, d, bh, a);
  if (dt == Dt::BF16) return d == 64 ? launch_d<bf16_tag, 64>(causal, sparse, bh, a, st)
                                     : launch_d<bf16_tag, 128>(causal, sparse, bh, a, st);
  return d == 64 ? launch_d<f16_tag, 64>(causal, sparse, bh, a, st)
                 : launch_d<f16_tag, 128>(causal, sparse, bh, a, st);
}

}  // namespace fa
