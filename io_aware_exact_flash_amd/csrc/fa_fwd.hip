// Fused exact-attention forward for gfx950, 16-bit inputs: the block-sparse,
// split-KV and dropout forwards (the dense forward is fwd2_kernel).
//
// Computes, per head, O = softmax(scale * Q K^T) V and the row log-sum-exp
// L = m + ln(l) in one pass over K and V (FlashAttention-2 notes,
// Algorithm 1 and eqs. (10)-(15)): each workgroup owns 256 query rows, keeps
// Q in registers, streams K/V tiles through LDS, and never writes the score
// or probability matrix anywhere.
//
// Work split (chosen for CDNA4, not taken from the pages' A100 design):
//  * 4 waves x 64 query rows, one wave per SIMD.  A wave holds two 32-query
//    blocks h = 0, 1 and computes S^T = K_j Q_h^T with v_mfma_f32_32x32x16,
//    so every query row is one lane column and the running statistics
//    (m, l), the exp(m_old - m_new) rescale of the accumulator, and the
//    final division are lane-local.  Every K or V fragment read from LDS
//    feeds the products of both blocks, half the LDS traffic per product of
//    a 32-query wave.
//  * The accumulator is O^T = V_j^T P^T: P^T comes straight out of the S^T
//    accumulator as the B operand; V_j^T is fetched from the row-major V
//    tile with LDS transpose reads (ds_read_b64_tr_b16).  Q^T and O^T live
//    in the accumulation registers (AGPRs) for the whole sweep.
//  * 32-key tiles stream through a ring of six LDS slots by global->LDS
//    DMA two tiles ahead; one barrier per tile.
//  * A lone wave per SIMD overlaps its matrix products with its own vector
//    work only when the two are interleaved, and a tile's steps depend on
//    each other (S -> max -> P -> PV), so the sweep is software-pipelined by
//    one tile: the S^T products of the next tile run interleaved with the
//    exponentials of the current one, and the PV products of the current
//    tile with the row sums of the current and the masks and row maxima of
//    the next.
//  * Causal: tiles above the diagonal are never loaded; only tiles crossing
//    it are masked element-wise (FlashAttention-2 notes, "Causal mask
//    optimisation").  Block-sparse: tiles whose 128 x 128 mask entry is zero
//    are never loaded (walkthrough on bluuewhale.github.io,
//    "Block-Sparse FlashAttention").
//  * The running maximum is refreshed only when a row's new maximum exceeds
//    it by more than 2^8 in exp2 units; the result is the same (every
//    contribution is scaled by the same stale m, and L = m + ln l holds for
//    any m), and the accumulator rescale is skipped whole-wave when no row
//    needs it.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

constexpr int kNT = 256;       // threads per workgroup
constexpr int kWQ = 64;        // query rows per wave
constexpr int kBR = 4 * kWQ;   // query rows per workgroup
constexpr float kLazy = 8.0f;

// SPLIT: split-KV mode.  Workgroup (row block, range rng) covers only the
// rng-th of a.nsplit contiguous chunks of the row block's key tiles and
// writes its partial output (normalised by its own row sums) and partial
// log-sum-exp to a.po / a.plse; fwd_merge_kernel combines the ranges.
// NW: waves per workgroup (rows per workgroup 64 NW).  Block-sparse runs at
// d = 64 use two: a workgroup then covers exactly one 128-row mask row, so
// it loads only that row's kept key tiles (with four waves it spans two mask
// rows and must sweep the union of their kept tiles), and two workgroups
// share a compute unit.
template <typename Tag, int D, bool CAUSAL, bool SPARSE, bool SPLIT = false, bool DROP = false, int NW = 4>
__global__ __launch_bounds__(NW * 64, 1) void fwd_kernel(FwdArgs a) {
  constexpr int BC = 32;              // keys per tile
  constexpr int KS = D / 16;          // k-steps of the S^T products
  constexpr int MB = D / 32;          // 32-row blocks of O^T
  constexpr int PK = BC / 16;         // k-steps of the PV products
  constexpr int NF = PK * MB;         // V^T fragments per tile
  constexpr int kRing = 6;            // LDS tile slots
  using KL = Pad<D, false>;           // K: row reads
  using VL = Pad<D, true>;            // V: transpose reads
  constexpr int BRW = NW * kWQ;       // query rows per workgroup
  using KD = Dma<BC, D, false, NW>;
  using VD = Dma<BC, D, true, NW>;
  constexpr int SLOT = KD::kSlot + VD::kSlot;
  constexpr int C = KD::kPer + VD::kPer;  // DMA instructions per wave per tile
  static_assert(4 * C < 64, "vmcnt range");
  static_assert(C / 2 <= NF - 1 && C - C / 2 <= 2 * KS - 2, "DMA issue slots");
  static_assert(2 * KS == 2 * NF, "both phases hold the same number of products");
  __shared__ __attribute__((aligned(16))) char smem[kRing * SLOT];
  __shared__ uint64_t mbits[SPARSE ? 2 * kMaskWords : 1];  // kept mask blocks of the two mask rows
  __shared__ uint16_t mnext[SPARSE ? kMaskMaxT : 1];       // next kept block, kept flags per row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so loop control stays scalar
  const int c32 = lane & 31, g = lane >> 5;
  // Causal: workgroup p of a head runs the query blocks nqb-1-p and p one
  // after the other, so every workgroup has the same number of key tiles
  // (no long workgroup left running alone at the end of the grid).  The
  // grid covers the longest sequence; a shorter one leaves workgroups idle.
  const int per = (CAUSAL && !SPLIT) ? (a.nqb + 1) / 2 : a.nqb;
  const int nsp = SPLIT ? a.nsplit : 1;
  const int lb = xcd_remap(blockIdx.x, a.nblk);
  const int rng = lb % nsp;  // key range (split-KV)
  const int bh = (lb / nsp) / per;
  const int pb_ = (lb / nsp) % per;
  const HeadAt at = query_head(a.sq, bh, a.n);
  const int hcan = DROP ? canon_head(a.sq, bh) : 0;  // head index of the dropout counter
  const int n = at.n;           // this head's length
  const int qsr = a.sq.qsr;     // row strides (elements)
  const int ksr = a.sq.ksr;
  const uint16_t* __restrict__ Qg = reinterpret_cast<const uint16_t*>(a.q) + at.q;
  const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + at.kv;
  const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + at.kv;
  uint16_t* __restrict__ Og = reinterpret_cast<uint16_t*>(a.o) + at.q;
  float* __restrict__ Lg = a.lse + at.l;

  auto run = [&](const int qb) {
    const int q0 = qb * BRW;
    const int qw0 = q0 + w * kWQ;       // the wave's first query; block h starts at qw0 + 32h

    u32x4 qreg[2][KS];                  // Q^T fragments, in AGPRs
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const size_t r = (size_t)min(qw0 + 32 * h + c32, n - 1) * qsr + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) gload_agpr(qreg[h][ks], Qg + r + 16 * ks);
    }

    const int n_tiles = (n + BC - 1) / BC;
    int j_end = n_tiles;
    if constexpr (CAUSAL) j_end = min(n_tiles, (min(q0 + BRW, n) - 1) / BC + 1);
    int j_lo = 0;
    if constexpr (SPLIT) {  // this workgroup's chunk of the key tiles
      const int chunk = (j_end + nsp - 1) / nsp;
      j_lo = min(rng * chunk, j_end);
      j_end = min(j_lo + chunk, j_end);
    }
    // block-sparse: the workgroup spans one or two 128-query mask rows, each
    // wave lies in one of them; their kept entries go to LDS as bits once
    constexpr int TPB = kMaskBlock / BC;  // key tiles per mask block
    lds_u64* mb = (lds_u64*)mbits;
    lds_u16* mn = (lds_u16*)mnext;
    int mwave = 0;   // this wave's mask row: 0 or 1
    if constexpr (SPARSE) {
      const int t0 = q0 / kMaskBlock;
      const int t1 = min((q0 + BRW - 1) / kMaskBlock, (n - 1) / kMaskBlock);
      mask_bits_build(mb, a.mask + (size_t)t0 * a.mask_t, 1, a.mask_t, w, NW, lane);
      if (t1 != t0) mask_bits_build(mb + kMaskWords, a.mask + (size_t)t1 * a.mask_t, 1, a.mask_t, w, NW, lane);
      __syncthreads();
      mask_table_build(mn, mb, t1 != t0 ? kMaskWords : -1, a.mask_t, 64 * w + lane, NW * 64);
      __syncthreads();
      mwave = (qw0 / kMaskBlock == t0) ? 0 : 1;
    }
    // the next tile after j whose mask block either row keeps (j_end if none)
    auto next_tile = [&](int j) {
      ++j;
      if constexpr (SPARSE)
        if (j < j_end) j = min(max(j, TPB * mask_next(mn, j / TPB)), j_end);
      return j;
    };
    // tiles of this wave's queries that have allowed keys
    auto live = [&](int jt) {
      bool l = jt < j_end;
      if constexpr (CAUSAL) l = l && (jt * BC <= qw0 + kWQ - 1);
      if constexpr (SPARSE) l = l && mask_kept(mn, mwave, jt / TPB);
      return l;
    };
    // Element v of block h of tile jt holds key jt*BC + 4g + 8(v/4) + v%4; it
    // is allowed while 8(v/4) + v%4 is at most lim[h].
    auto limits = [&](int jt, int (&lim)[2]) {
      const bool lv = SPARSE ? live(jt) : true;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int last = n - 1;
        if constexpr (CAUSAL) last = min(last, qw0 + 32 * h + c32);
        if constexpr (SPLIT) last = min(last, j_end * BC - 1);
        lim[h] = lv ? last - jt * BC - 4 * g : -1;
      }
    };

    KD kd;
    VD vd;
    kd.init(w, lane);
    vd.init(w, lane);
    const int krow = KL::row_base(c32, g);
    const int vtr = KD::kSlot + VL::tr_base(lane);
    auto slot_next = [&](int so) { return so + SLOT == kRing * SLOT ? 0 : so + SLOT; };

    vm_wait<0>();  // Q loads done: from here vmcnt counts DMA only

    const int j_first = SPARSE ? next_tile(j_lo - 1) : j_lo;
    if (j_first >= j_end) {  // no key tile at all: O = 0, L = -inf
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int my_q = qw0 + 32 * h + c32;
        if (my_q < n) {
          if constexpr (SPLIT) {
            const size_t row = ((size_t)rng * a.nbh + bh) * a.n + my_q;
            for (int c = 4 * g; c < D; c += 8) *reinterpret_cast<f32x4*>(a.po + row * D + c) = f32x4{0.f, 0.f, 0.f, 0.f};
            if (g == 0) a.plse[row] = -INFINITY;
          } else {
            uint16_t* op = Og + (size_t)my_q * qsr;
            for (int c = 0; c < D; c += 8) *reinterpret_cast<u32x4*>(op + c) = u32x4{0u, 0u, 0u, 0u};
            if (g == 0) Lg[my_q] = -INFINITY;
          }
        }
      }
      return;
    }
    // Every iteration issues exactly C DMA instructions (past the last tile
    // they reload the first tile into a slot nobody reads), so the tile after
    // the next one has landed once vmcnt <= C at the barrier.
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
    dma_set();
    // A tile's DMA is split: instructions 0..kDB-1 are issued in the B
    // phase of one iteration, the rest in the A phase of the next (spreading
    // the address work of the four waves over the whole iteration)
    constexpr int kDB = C / 2;
    for (int t = 0; t < 3; ++t) {
#pragma unroll
      for (int i = 0; i < C; ++i) dma_tile(i);
      dma_advance();
    }
#pragma unroll
    for (int i = 0; i < kDB; ++i) dma_tile(i);

    f32x16 acc[2][MB];  // O^T of both blocks, in AGPRs
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[h][mb] = 0.0f;
    const float cs = a.c;  // scale * log2(e): scores in exp2 units
    const float inv_cs = 1.0f / cs;
    // S^T of both blocks for two tiles, register sets 0 and 1 by tile parity
    f32x16 s[2][2];
    // packed P^T (B operands of the PV products) for two tiles
    u32x4 pb[2][2][PK];
    constexpr int kPD = DROP ? 4 : 6;  // LDS fragments run kPD products ahead (registers permitting)
    u32x4 fr[kPD + 1];      // K row fragments (ring)
    u32x4 kq[kPD + 1];      // V^T fragments (ring)
    auto rd_k = [&](const lchar* rows, int ks) { return ld_row(rows + KL::row_off(0, ks)); };
    auto rd_v = [&](const lchar* vt, int f) {
      return ld_tr(vt + VL::tr_off(0, f / MB, 0, f % MB), vt + VL::tr_off(0, f / MB, 1, f % MB));
    };
    auto k_rows = [&](int so) { return lds_opaque(lds_ptr(smem) + so + krow); };
    auto v_cols = [&](int so) { return lds_opaque(lds_ptr(smem) + so + vtr); };
    auto prefetch_k = [&](int so) {
      const lchar* rows = k_rows(so);
#pragma unroll
      for (int ks = 0; ks < kPD && ks < KS; ++ks) fr[ks] = rd_k(rows, ks);
    };


    // S^T = K Q^T of both blocks for the tile in slot `so` into set Y (its
    // first kPD K fragments already in flight), with vec(u) = vector work
    // after product u = 2 ks + h.
    // (No VALU instruction writes their operands: K fragments come from LDS,
    // Q^T from memory, and the accumulators only from the products.)
    auto prod_s = [&](auto y_c, int so, auto&& vec) {
      constexpr int Y = decltype(y_c)::value;
      const lchar* rows = k_rows(so);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + kPD < KS) fr[(ks + kPD) % (kPD + 1)] = rd_k(rows, ks + kPD);
        const u32x4 f = fr[ks % (kPD + 1)];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (ks == 0) mfma32_vd<Tag, true, true, false>(s[Y][h], f, qreg[h][ks]);
          else mfma32_vd<Tag, false, true, false>(s[Y][h], f, qreg[h][ks]);
          vec(2 * ks + h);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    // Row statistics.  m_run[h] is the stale maximum every P of block h is
    // taken against (exp2 units, -inf until a row sees its first key); nmu is
    // -m_run, or 0 while m_run = -inf so that masked scores give exp2(-inf);
    // thr is the raw score above which a row's maximum has outgrown m_run by
    // more than the lazy margin.
    float m_run[2] = {-INFINITY, -INFINITY}, nmu[2] = {0.0f, 0.0f};
    float thr[2] = {-INFINITY, -INFINITY};
    float l_part[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};  // two partial sums per block (independent add chains)

    // the first tile's products; its P^T "predecessor" is zero
    vm_wait<C + kDB>();  // tiles 0 and 1 have landed (for this wave's share) ...
    __syncthreads();   // ... for every wave
    int j = j_first;
    int so = 0;        // slot of tile j
    int sp = 0;        // slot of the tile whose PV products run next (none yet: any landed slot)
    prefetch_k(so);
    prod_s(std::integral_constant<int, 0>{}, so, [](int) {});
    vgpr_drain(s[0]);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kk = 0; kk < PK; ++kk) pb[1][h][kk] = u32x4{0u, 0u, 0u, 0u};
    int jn = next_tile(j);
    int sn = slot_next(so);
    prefetch_k(sn);

    // Iteration i (tile j = set X, its successor jn = set Y, its predecessor
    // jp in slot sp):
    //   A: S^T of jn (matrix products into VGPRs)
    //      | mask, running-row maximum and t = S^T c - m of j
    //   barrier (the tile after jn has landed; every wave is past A)
    //   B: O^T += V^T P^T of jp (products into AGPRs)
    //      | P = exp2(t), row sums and packing of j, DMA
    // If a row's maximum outgrew the lazy margin in A, m is refreshed right
    // after A (l and the t values of j rescaled) and O^T right after B.  The
    // exponentials run beside the AGPR-destination products only: next to
    // products that write VGPRs they issue markedly slower.
    auto step = [&](auto x_c, auto mask_c) {
      constexpr int X = decltype(x_c)::value;
      constexpr int Y = 1 - X;
      constexpr bool MASK = decltype(mask_c)::value;
      int lim[2];
      if constexpr (MASK) limits(j, lim);
      // dropout bytes of tile j: the quad's four lanes (rows 4m .. 4m+3)
      // draw the four 4x4 blocks of keys 8a + 4g .. 8a + 4g + 3 (a = lane % 4)
      // and exchange words, so each lane ends with its own row's 16 bytes
      // in element order
      u32x4 kb[2];
      if constexpr (DROP) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 ctr = {(uint32_t)(qw0 + 32 * h + c32) >> 2, (uint32_t)(8 * j + g + 2 * (c32 & 3)),
                             (uint32_t)hcan, a.drop.offset};
          kb[h] = quad_transpose4(philox4x32_10(ctr, a.drop.k0, a.drop.k1), lane);
        }
      }
      // ---- A
      // Per element of tile j: mask and running maximum in the first half of
      // the products (so the refresh test is known early), t = S c - m
      // spread over all of them (after the element's mask).
      float mx[2] = {-INFINITY, -INFINITY};
      bool grow = false;
      constexpr int RM = 32 / KS;       // elements per slot, mask and maximum
      constexpr int R = 32 / (2 * KS);  // elements per slot, t
      // the first V^T fragments of tile jp are read during the last products
      constexpr int kPV = kPD < NF ? kPD : NF;
      const lchar* vtp = v_cols(sp);
      prod_s(std::integral_constant<int, Y>{}, sn, [&](int u) {
        if (u >= 2 * KS - kPV) kq[u - (2 * KS - kPV)] = rd_v(vtp, u - (2 * KS - kPV));
        if (u < KS) {
#pragma unroll
          for (int r = 0; r < RM; r += 2) {
            const int e = u * RM + r, h = e >> 4, v = e & 15;
            if constexpr (MASK) {
              s[X][h][v] = (8 * (v >> 2) + (v & 3) > lim[h]) ? -INFINITY : s[X][h][v];
              s[X][h][v + 1] = (8 * ((v + 1) >> 2) + ((v + 1) & 3) > lim[h]) ? -INFINITY : s[X][h][v + 1];
            }
            mx[h] = max3(mx[h], s[X][h][v], s[X][h][v + 1]);
          }
        }
        if (u == KS) grow = __builtin_amdgcn_ballot_w64(mx[0] > thr[0] || mx[1] > thr[1]) != 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int e = u * R + r, h = e >> 4, v = e & 15;
          s[X][h][v] = fmaf(s[X][h][v], cs, nmu[h]);
        }
#pragma unroll
        for (int q = kDB; q < C; ++q)
          if (u == 1 + (q - kDB) * (2 * KS - 2) / (C - kDB)) dma_tile(q);
      });
      dma_advance();
      // ---- B, first products (independent of the refresh and the barrier)
      const lchar* vt = v_cols(sp);
      auto pv = [&](int f, int h) { mfma32_acc<Tag>(acc[h][f % MB], kq[f % (kPD + 1)], pb[Y][h][f / MB]); };
      if (kPD < NF) kq[kPD % (kPD + 1)] = rd_v(vt, kPD);
      pv(0, 0);
      pv(0, 1);
      __builtin_amdgcn_sched_barrier(0);
      float alpha[2] = {1.0f, 1.0f};
      if (__builtin_expect(grow, 0)) {  // rare: refresh m for the rows whose maximum outgrew it
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float mt = half_max(mx[h]) * cs;
          const bool gr = mt > m_run[h] + kLazy;
          alpha[h] = gr ? fast_exp2(m_run[h] - mt) : 1.0f;
          const float nmu_new = gr ? -mt : nmu[h];
          const float delta = nmu_new - nmu[h];
          m_run[h] = gr ? mt : m_run[h];
          nmu[h] = nmu_new;
          thr[h] = (m_run[h] + kLazy) * inv_cs;
          l_part[h][0] *= alpha[h];
          l_part[h][1] *= alpha[h];
#pragma unroll
          for (int v = 0; v < 16; ++v) s[X][h][v] += delta;
        }
      }
      const int jnn = next_tile(jn);
      const int snn = slot_next(sn);
      vm_wait<C>();      // tile jnn has landed (for this wave's share) ...
      wg_barrier();      // ... for every wave; the slot refilled below is free
      constexpr int kPK = kPD < KS ? kPD : KS;
      const lchar* krn = k_rows(snn);
      // ---- B, the rest
      // element e (block e/16, row e%16) of tile j in two stages one slot
      // apart: P = exp2(t), then the row sum; each 8-element group is packed
      // once summed.  Slot u (2 .. 2NF-1) takes elements E(u-2) .. E(u-1)-1.
      auto stx = [&](int e) {
        const int h = e >> 4, v = e & 15;
        s[X][h][v] = fast_exp2(s[X][h][v]);
        asm volatile("" : "+v"(s[X][h][v]));
      };
      auto sty = [&](int e) {
        const int h = e >> 4, v = e & 15;
        l_part[h][v & 1] += s[X][h][v];
        asm volatile("" : "+v"(l_part[h][v & 1]));
        if ((v & 7) == 7) {
          if constexpr (DROP) pb[X][h][v >> 3] = pack8_keep<Tag>(s[X][h], v & 8, kb[h], a.drop.thr);
          else pb[X][h][v >> 3] = pack8<Tag>(s[X][h], v & 8);
          asm volatile("" : "+v"(pb[X][h][v >> 3]));
        }
      };
      constexpr int NS = 2 * NF - 2;  // slots carrying element work
      auto E = [](int k) { return 32 * k / NS; };
      auto slot_work = [&](int u) {  // u = 2 .. 2NF (2NF: the tail)
        const int k = u - 2;
        if (k < NS)
          for (int e = E(k); e < E(k + 1); ++e) stx(e);
        if (k >= 1)
          for (int e = E(k - 1); e < E(k); ++e) sty(e);
      };
#pragma unroll
      for (int f = 1; f < NF; ++f) {
        if (f + kPD < NF) kq[(f + kPD) % (kPD + 1)] = rd_v(vt, f + kPD);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          pv(f, h);
          slot_work(2 * f + h);
          // the first K fragments of tile jnn (landed: barrier above) are
          // read during the first products, for the next A phase
          const int u = 2 * f + h;
          if (u >= 2 && u < 2 + kPK) fr[u - 2] = rd_k(krn, u - 2);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = 0; q < kDB; ++q)
          if (f == 1 + (2 * q + 1) * (NF - 1) / (2 * kDB)) dma_tile(q);
      }
      slot_work(2 * NF);
      if (__builtin_expect(grow, 0)) {
        agpr_drain(acc[0]);
        agpr_drain(acc[1]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[h][mb] *= alpha[h];
      }
      sp = so;
      so = sn;
      sn = snn;
      j = jn;
      jn = jnn;
    };

    // Two iterations per trip keep the register sets in fixed roles.  The
    // sweep runs until the PV products of the last tile are done; iterations
    // past it see no tile (all keys masked, slots holding valid reloads).
    // Dense sweeps start with the iterations whose tile j has no masked key
    // for this wave (keys below its diagonal and inside the sequence), an
    // even number of them, without any per-element test; the rest run with
    // the mask.  The total is the same for every wave.
    int n_plain = 0;
    if constexpr (!SPARSE) {
      int jm = SPLIT ? min(n / BC, j_end) : n / BC;      // first tile reaching past the sequence (or range) end
      if constexpr (CAUSAL) jm = min(jm, qw0 / BC);     // first tile crossing the diagonal
      n_plain = max(jm - j_first, 0) & ~1;
    }
    for (int t = 0; t < n_plain; t += 2) {
      step(std::integral_constant<int, 0>{}, std::false_type{});
      step(std::integral_constant<int, 1>{}, std::false_type{});
    }
    // The iteration of tile j_end (the first past the last) runs the PV
    // products of the last tile; the trip containing it is the last.
    do {
      step(std::integral_constant<int, 0>{}, std::true_type{});
      step(std::integral_constant<int, 1>{}, std::true_type{});
    } while (j <= j_end);

    agpr_drain(acc[0]);
    agpr_drain(acc[1]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float l = half_sum(l_part[h][0] + l_part[h][1]);
      float inv = l > 0.0f ? 1.0f / l : 0.0f;
      if constexpr (DROP) inv *= a.drop.scale;  // kept probabilities scaled by 1 / (1 - p)
      const int my_q = qw0 + 32 * h + c32;
      if (my_q < n && SPLIT) {
        const size_t row = ((size_t)rng * a.nbh + bh) * a.n + my_q;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            f32x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = acc[h][mb][4 * r + i] * inv;
            *reinterpret_cast<f32x4*>(a.po + row * D + 32 * mb + 8 * r + 4 * g) = x;
          }
        if (g == 0) a.plse[row] = l > 0.0f ? m_run[h] * kLn2 + logf(l) : -INFINITY;
      } else if (my_q < n) {
        uint16_t* op = Og + (size_t)my_q * qsr;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            u32x2 pk;
            pk[0] = pack2<Tag>(acc[h][mb][4 * r] * inv, acc[h][mb][4 * r + 1] * inv);
            pk[1] = pack2<Tag>(acc[h][mb][4 * r + 2] * inv, acc[h][mb][4 * r + 3] * inv);
            *reinterpret_cast<u32x2*>(op + 32 * mb + 8 * r + 4 * g) = pk;
          }
        if (g == 0) Lg[my_q] = l > 0.0f ? m_run[h] * kLn2 + logf(l) : -INFINITY;
      }
    }
  };
  const int nqb = (n + BRW - 1) / BRW;  // this head's query blocks
  const int qa = nqb - 1 - pb_;         // the longer block first
  // blocks qa and pb_ (paired causal), or qa alone; none past the end of a
  // shorter sequence
  const int nrun = (CAUSAL && !SPLIT) ? (pb_ < qa ? 2 : pb_ == qa ? 1 : 0) : (qa >= 0 ? 1 : 0);
#pragma clang loop unroll(disable)
  for (int r = 0; r < nrun; ++r) {
    if (r) {
      vm_wait<0>();      // the first block's DMA and stores are done ...
      __syncthreads();   // ... and every wave is out of its LDS tiles
    }
    run(r ? pb_ : qa);
  }
}

// Merge of the split-KV partials of one row (v1-notes, "merging two
// vectors' softmax statistics", applied to nsplit parts): with the partial
// log-sum-exps L_s and outputs O_s (each normalised by its own sum),
// L = log sum_s e^{L_s} and O = sum_s e^{L_s - L} O_s.  D/4 threads per row,
// four columns each.
template <typename Tag, int D>
__global__ __launch_bounds__(kNT) void fwd_merge_kernel(FwdArgs a, long rows) {
  constexpr int TPR = D / 4;  // threads per row
  const long row = (long)blockIdx.x * (kNT / TPR) + threadIdx.x / TPR;
  if (row >= rows) return;
  const int c = 4 * (threadIdx.x % TPR);
  const int S = a.nsplit;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, a.plse[(size_t)s * rows + row]);
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    float wsum = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float wgt = expf(a.plse[(size_t)s * rows + row] - mx);
      wsum += wgt;
      const f32x4 x = *reinterpret_cast<const f32x4*>(a.po + ((size_t)s * rows + row) * D + c);
      o += wgt * x;
    }
    o *= 1.0f / wsum;
    lse = mx + logf(wsum);
  }
  u32x2 pk;
  pk[0] = pack2<Tag>(o[0], o[1]);
  pk[1] = pack2<Tag>(o[2], o[3]);
  *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.o) + (size_t)row * D + c) = pk;
  if (c == 0) a.lse[row] = lse;
}

template <typename Tag, int D>
hipError_t launch_split_d(bool causal, const FwdArgs& a, hipStream_t st) {
  timing_begin(kFwdSplit, st);
  if (causal) hipLaunchKernelGGL((fwd_kernel<Tag, D, true, false, true>), dim3(a.nblk), dim3(kNT), 0, st, a);
  else hipLaunchKernelGGL((fwd_kernel<Tag, D, false, false, true>), dim3(a.nblk), dim3(kNT), 0, st, a);
  hipError_t e = hipGetLastError();
  timing_end(kFwdSplit, st);
  if (e != hipSuccess) return e;
  const long rows = (long)a.nbh * a.n;
  constexpr int kRowsPerBlock = kNT / (D / 4);
  timing_begin(kFwdMerge, st);
  hipLaunchKernelGGL((fwd_merge_kernel<Tag, D>), dim3((rows + kRowsPerBlock - 1) / kRowsPerBlock), dim3(kNT), 0,
                     st, a, rows);
  e = hipGetLastError();
  timing_end(kFwdMerge, st);
  return e;
}

template <typename Tag, int D>
hipError_t launch_drop_d(bool causal, const FwdArgs& a, hipStream_t st) {
  timing_begin(kFwdDrop, st);
  if (causal) hipLaunchKernelGGL((fwd_kernel<Tag, D, true, false, false, true>), dim3(a.nblk), dim3(kNT), 0, st, a);
  else hipLaunchKernelGGL((fwd_kernel<Tag, D, false, false, false, true>), dim3(a.nblk), dim3(kNT), 0, st, a);
  hipError_t e = hipGetLastError();
  timing_end(kFwdDrop, st);
  return e;
}

// Waves per workgroup of the block-sparse forward (see fwd_kernel).
template <int D>
constexpr int sparse_waves() { return D == 64 ? 2 : 4; }

template <typename Tag, int D>
hipError_t launch_sparse_d(bool causal, const FwdArgs& a, hipStream_t st) {
  constexpr int SW = sparse_waves<D>();
  timing_begin(kFwd, st);
  if (causal)
    hipLaunchKernelGGL((fwd_kernel<Tag, D, true, true, false, false, SW>), dim3(a.nblk), dim3(64 * SW), 0, st, a);
  else hipLaunchKernelGGL((fwd_kernel<Tag, D, false, true, false, false, SW>), dim3(a.nblk), dim3(64 * SW), 0, st, a);
  hipError_t e = hipGetLastError();
  timing_end(kFwd, st);
  return e;
}

}  // namespace

hipError_t launch_fwd_sparse(Dt dt, int d, bool causal, int bh, FwdArgs a, hipStream_t st) {
  const int rows = kWQ * (d == 64 ? sparse_waves<64>() : sparse_waves<128>());
  a.nqb = (a.n + rows - 1) / rows;
  a.nblk = (causal ? (a.nqb + 1) / 2 : a.nqb) * bh;
  if (dt == Dt::BF16) return d == 64 ? launch_sparse_d<bf16_tag, 64>(causal, a, st)
                                     : launch_sparse_d<bf16_tag, 128>(causal, a, st);
  return d == 64 ? launch_sparse_d<f16_tag, 64>(causal, a, st) : launch_sparse_d<f16_tag, 128>(causal, a, st);
}

hipError_t launch_fwd_dropout(Dt dt, int d, bool causal, int bh, FwdArgs a, hipStream_t st) {
  a.nqb = (a.n + kBR - 1) / kBR;
  a.nblk = (causal ? (a.nqb + 1) / 2 : a.nqb) * bh;
  if (dt == Dt::BF16) return d == 64 ? launch_drop_d<bf16_tag, 64>(causal, a, st)
                                     : launch_drop_d<bf16_tag, 128>(causal, a, st);
  return d == 64 ? launch_drop_d<f16_tag, 64>(causal, a, st) : launch_drop_d<f16_tag, 128>(causal, a, st);
}

hipError_t launch_fwd_split(Dt dt, int d, bool causal, int bh, FwdArgs a, hipStream_t st) {
  a.nqb = (a.n + kBR - 1) / kBR;
  a.nbh = bh;
  a.nblk = a.nqb * bh * a.nsplit;
  if (dt == Dt::BF16) return d == 64 ? launch_split_d<bf16_tag, 64>(causal, a, st)
                                     : launch_split_d<bf16_tag, 128>(causal, a, st);
  return d == 64 ? launch_split_d<f16_tag, 64>(causal, a, st) : launch_split_d<f16_tag, 128>(causal, a, st);
}

}  // namespace fa
