// Fused exact-attention forward for gfx950, 16-bit inputs, two waves per
// SIMD (every dense 16-bit forward without dropout).
//
// The same computation as fwd_kernel (FlashAttention-2 notes, Algorithm 1,
// eqs. (10)-(15): online softmax over K/V tiles streamed through LDS, O and
// the row log-sum-exp written once), with a different split of the work:
//  * 8 waves x 32 query rows = 256 rows per workgroup, two waves per SIMD.
//    A lone wave per SIMD stalls on its own LDS, DMA and product-result
//    latencies; with two, one wave's matrix products run while the other
//    waits or works through its exponentials.
//  * 64-key K/V tiles in a ring of four LDS slots, filled by global->LDS
//    DMA two tiles ahead (K and V images of a slot in one run of blocks, so
//    four slots fit at d = 128) that only waves 0-3 issue; one barrier per
//    tile.
//  * Per tile and wave: S^T = K Q^T with Q^T in registers and K fragments
//    read as LDS rows; the running maximum is refreshed lazily (only when a
//    row's maximum outgrows it by more than 2^8 in exp2 units: every
//    contribution is then taken against the same stale maximum, and
//    L = m + ln l holds for any m); P = exp2(S c - m); O^T += V^T P^T with
//    V^T read by LDS transpose reads.  Fragments stream a fixed distance
//    ahead of their products.
//  * The waves of SIMD-mates are skewed by one phase: waves 0-3 run a
//    tile's S, softmax and PV products in order; waves 4-7 start each tile
//    with the previous tile's PV products, so one wave's exponentials
//    overlap the other's products instead of every wave reaching its
//    vector work at the same moment.  The slot a lagging wave still reads
//    is the fourth ring slot.
//  * Causal: tiles above a wave's rows are skipped (the wave still joins the
//    barriers and the DMA); only tiles crossing its diagonal or the sequence
//    end are masked element-wise; a workgroup runs a long and a short query
//    block of its head one after the other (balanced work).
//  * Every instance of the tile code holds the O^T accumulators in the same
//    registers: only the score products differ between masked and unmasked
//    tiles, and the softmax and PV code is shared (separate copies made the
//    compiler move the accumulators between register sets every tile).
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));

// c + a b on v_mfma_f32_32x32x16 (compiler-placed registers and hazards).
template <typename Tag>
__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (std::is_same<Tag, bf16_tag>::value)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8v, a), __builtin_bit_cast(f16x8v, b), c, 0,
                                                  0, 0);
}

constexpr int kNW = 8;            // waves per workgroup
constexpr int kWR = 32;           // query rows per wave
constexpr int kRows = kNW * kWR;  // query rows per workgroup
constexpr float kLazy2 = 8.0f;

// SPARSE (d = 64): block-sparse forward.  Four waves, 128 rows: a
// workgroup covers exactly one 128-row mask row, so it loads only that
// row's kept key tiles, and a three-slot ring (72 KB of LDS) lets two
// workgroups share a compute unit, two waves per SIMD as in the dense
// kernel; the waves are not skewed.
template <typename Tag, int D, bool CAUSAL, bool SPARSE = false>
__global__ __launch_bounds__((SPARSE ? 4 : kNW) * 64, SPARSE ? 2 : 1) void fwd2_kernel(FwdArgs a) {
  constexpr int NW = SPARSE ? 4 : kNW;  // waves per workgroup
  constexpr int ROWS = NW * kWR;        // query rows per workgroup
  constexpr int BC = 64;              // keys per tile
  constexpr int KS = D / 16;          // k-steps of the S^T products
  constexpr int MB = D / 32;          // 32-row blocks of O^T
  constexpr int KB = BC / 32;         // 32-key blocks per tile
  constexpr int PK = 2;               // 16-key steps per 32-key block
  constexpr int kRing = SPARSE ? 3 : 4;
  using KL = Pad<D, false>;
  using VL = Pad<D, true>;
  // dense: only waves 0-3 issue the DMA.  The lagging waves 4-7 are the
  // critical path (their chain of PV products, S products and softmax is
  // the longer one, and the leading waves wait for them at the barrier);
  // each DMA instruction costs the address unit ~30 cycles, so the
  // instructions queue after the barrier, and keeping the lagging waves out
  // of that queue shortens the iteration.  They see the data through the
  // barrier, which the issuing waves reach after their vm_wait.
  constexpr int NDMA = SPARSE ? NW : NW / 2;
  using KVD = DmaKV<BC, D, NDMA>;
  constexpr int SLOT = KVD::kSlot;
  constexpr int C = KVD::kPer;  // DMA instructions per wave per tile
  static_assert(2 * C < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem[kRing * SLOT];
  __shared__ uint64_t mbits[SPARSE ? kMaskWords : 1];  // kept mask blocks of the workgroup's mask row
  __shared__ uint16_t mnext[SPARSE ? kMaskMaxT : 1];   // next kept block

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, g = lane >> 5;
  const int per = CAUSAL ? (a.nqb + 1) / 2 : a.nqb;
  const int lb = xcd_remap(blockIdx.x, a.nblk);
  const int bh = lb / per;
  const int pb_ = lb % per;
  const HeadAt at = query_head(a.sq, bh, a.n);
  const int n = at.n;
  const int qsr = a.sq.qsr, ksr = a.sq.ksr;
  const uint16_t* __restrict__ Qg = reinterpret_cast<const uint16_t*>(a.q) + at.q;
  const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + at.kv;
  const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + at.kv;
  uint16_t* __restrict__ Og = reinterpret_cast<uint16_t*>(a.o) + at.q;
  float* __restrict__ Lg = a.lse + at.l;
  const float cs = a.c;

  auto run = [&](const int qb) {
    const int q0 = qb * ROWS;
    const int qw0 = q0 + w * kWR;  // the wave's first row
    const int my_q = qw0 + c32;

    u32x4 qreg[KS];  // Q^T fragments (B operands)
    {
      const uint16_t* qr = Qg + (size_t)min(my_q, n - 1) * qsr + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qreg[ks] = *reinterpret_cast<const u32x4*>(qr + 16 * ks);
    }
    const int n_tiles = (n + BC - 1) / BC;
    const int t_end = CAUSAL ? min(n_tiles, (min(q0 + ROWS, n) - 1) / BC + 1) : n_tiles;  // the workgroup's tiles
    const int t_wave = CAUSAL ? min(t_end, (min(qw0 + kWR, n) - 1) / BC + 1) : t_end;      // this wave's
    // tiles below t_plain have no masked key for this wave (below its
    // diagonal and inside the sequence)
    int t_plain = n / BC;
    if constexpr (CAUSAL) t_plain = min(t_plain, (qw0 + 1) / BC);

    // block-sparse: the kept entries of the workgroup's mask row, built in
    // LDS once; the sweep visits kept tiles only (the same ones for every
    // wave)
    constexpr int TPB = kMaskBlock / BC;  // key tiles per mask block
    lds_u16* mn = (lds_u16*)mnext;
    if constexpr (SPARSE) {
      lds_u64* mb = (lds_u64*)mbits;
      mask_bits_build(mb, a.mask + (size_t)(q0 / kMaskBlock) * a.mask_t, 1, a.mask_t, w, NW, lane);
      __syncthreads();
      mask_table_build(mn, mb, -1, a.mask_t, tid, NW * 64);
      __syncthreads();
    }
    auto next_tile = [&](int j) {
      ++j;
      if constexpr (SPARSE)
        if (j < t_end) j = min(max(j, TPB * mask_next(mn, j / TPB)), t_end);
      return j;
    };

    KVD kvd;
    kvd.init(w % NDMA, lane);
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds_ptr(smem);
    // tile jt's DMA into slot sl (past the end: a reload of tile 0 into a
    // slot nobody reads, so every issuing wave issues C instructions per
    // tile; the other waves issue none, and their vm_wait is a no-op)
    auto issue = [&](int jt, int sl) {
      if (w >= NDMA) return;
      const int tt = jt < t_end ? jt : 0;
      const uint16_t* kt = Kg + (size_t)tt * BC * ksr;
      const uint16_t* vt = Vg + (size_t)tt * BC * ksr;
      const int last = n - 1 - tt * BC;
      const uint32_t dst = lds_base + sl * SLOT + 1024 * w;
#pragma unroll
      for (int k = 0; k < KVD::kPer; ++k) kvd.issue_at(k, kt, vt, last, 2 * ksr, dst);
    };

    vm_wait<0>();  // Q loads done: from here vmcnt counts DMA only
    const int j0 = SPARSE ? next_tile(-1) : 0;  // the first two tiles
    const int j1 = next_tile(j0);
    issue(j0, 0);
    issue(j1, 1);

    f32x16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = 0.0f;
    float m_run = -INFINITY;  // exp2 units
    float nmu = 0.0f;         // -m_run, 0 while m_run = -inf
    float l_part[2] = {0.0f, 0.0f};
    const int krow = KL::row_base(c32, g);
    const int vtr = KVD::kBytesK + VL::tr_base(lane);

    // S^T of one tile into s (element v of block kb: key jt*BC + 32kb + 4g +
    // 8(v/4) + v%4); MASK: element test against the row's last key.  The
    // two blocks' product chains alternate, so consecutive products are
    // independent, and all K fragments are requested before the first.
    auto scores = [&](auto mask_c, int jt, int sl, f32x16 (&s)[KB]) {
      constexpr bool MASK = decltype(mask_c)::value;
      const lchar* kr = lds_opaque(lds_ptr(smem) + sl * SLOT + krow);
      // a stream of KS*KB fragments (k-step outer), each requested PD
      // fragments ahead of its product (at most PD + 1 LDS reads
      // outstanding, inside the wait counter's range)
      constexpr int NF = KS * KB;
      constexpr int PD = NF < 8 ? NF : 8;
      u32x4 kf[NF];
      const f32x16 zero = 0.0f;
#pragma unroll
      for (int f = 0; f < PD; ++f) kf[f] = ld_row(kr + KL::row_off(f % KB, f / KB));
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f + PD < NF) kf[f + PD] = ld_row(kr + KL::row_off((f + PD) % KB, (f + PD) / KB));
        __builtin_amdgcn_sched_barrier(0);
        const int kb = f % KB, ks = f / KB;
        s[kb] = mma<Tag>(kf[f], qreg[ks], ks ? s[kb] : zero);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (MASK) {
        int last = n - 1;
        if constexpr (CAUSAL) last = min(last, my_q);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int lim = last - jt * BC - 32 * kb - 4 * g;
#pragma unroll
          for (int v = 0; v < 16; ++v) s[kb][v] = (8 * (v >> 2) + (v & 3) > lim) ? -INFINITY : s[kb][v];
        }
      }
    };

    u32x4 pb[KB][PK];
    auto softmax = [&](int jt, int sl) {
      f32x16 s[KB];
      if (jt < t_plain) scores(std::false_type{}, jt, sl, s);
      else scores(std::true_type{}, jt, sl, s);
      // t = S c - m (exp2 units against the stale maximum; masked keys give
      // -inf).  The fma is the products' first (compiler-visible) reader, so
      // the compiler spaces it from them; the row maximum of t then runs as
      // asm v_max3 on VALU results.
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = fmaf(s[kb][v], cs, nmu);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; v += 2) mx = max3(mx, s[kb][v], s[kb][v + 1]);
      // a row that has seen no key yet (m = -inf, t the score itself) takes
      // its first maximum whatever it is
      const bool first = m_run == -INFINITY;
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(mx > kLazy2 || (first && mx > -INFINITY)) != 0, 0)) {
        // rare: some row outgrew the stale maximum by > 2^8 (the asm keeps the
        // compiler from flattening this block into every tile)
        asm volatile("s_nop 0");
        const float grow = half_max(mx);  // the row's growth (its maximum of t)
        const bool gr = first ? grow > -INFINITY : grow > kLazy2;
        const float alpha = gr ? (first ? 0.0f : fast_exp2(-grow)) : 1.0f;
        const float shift = gr ? grow : 0.0f;
        if (gr) {
          m_run = first ? grow : m_run + grow;
          nmu = -m_run;
        }
        l_part[0] *= alpha;
        l_part[1] *= alpha;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) s[kb][v] -= shift;
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(s[kb][v]);
          s[kb][v] = p;
          l_part[v & 1] += p;
        }
#pragma unroll
        for (int kk = 0; kk < PK; ++kk) pb[kb][kk] = pack8<Tag>(s[kb], 8 * kk);
      }
    };
    auto pv = [&](int sl) {
      const lchar* vt = lds_opaque(lds_ptr(smem) + sl * SLOT + vtr);
      // V^T fragments (16-key step outer, 32-row block inner), each
      // requested PV fragments ahead of its product (two reads each)
      constexpr int NV = KB * PK * MB;
      constexpr int PV = NV < 6 ? NV : 6;
      u32x4 vf[NV];
      auto rd_v = [&](int f) {
        const int q = f / MB, mb = f % MB;
        return ld_tr(vt + VL::tr_off(q / PK, q % PK, 0, mb), vt + VL::tr_off(q / PK, q % PK, 1, mb));
      };
#pragma unroll
      for (int f = 0; f < PV; ++f) vf[f] = rd_v(f);
#pragma unroll
      for (int f = 0; f < NV; ++f) {
        if (f + PV < NV) vf[f + PV] = rd_v(f + PV);
        __builtin_amdgcn_sched_barrier(0);
        const int q = f / MB, mb = f % MB;
        acc[mb] = mma<Tag>(vf[f], pb[q / PK][q % PK], acc[mb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (SPARSE) {
      int jq = next_tile(j1);  // the next tile to load
      int jt = j0;
      for (int it = 0; jt < t_end; ++it) {
        const int sl = it % kRing;
        vm_wait<C>();     // tile jt has landed (for this wave's share) ...
        wg_barrier();     // ... for every wave, and every wave is done with the previous tile
        issue(jq, (it + 2) % kRing);
        jq = next_tile(jq);
        if (jt < t_wave) {
          softmax(jt, sl);
          pv(sl);
        }
        jt = next_tile(jt);
      }
    } else if (w < NW / 2) {
      for (int jt = 0; jt < t_end; ++jt) {
        const int sl = jt % kRing;
        vm_wait<C>();     // tile jt has landed (for this wave's share; jt + 1 may be in flight) ...
        wg_barrier();     // ... for every wave, and every wave is done with tile jt - 2
        issue(jt + 2, (jt + 2) % kRing);
        if (jt >= t_wave) continue;
        softmax(jt, sl);
        pv(sl);
      }
    } else {
      // one phase behind: the previous tile's PV products first
      for (int jt = 0; jt < t_end; ++jt) {
        const int sl = jt % kRing;
        vm_wait<C>();
        wg_barrier();
        issue(jt + 2, (jt + 2) % kRing);
        if (jt > 0 && jt - 1 < t_wave) pv((jt - 1) % kRing);
        if (jt < t_wave) softmax(jt, sl);
      }
      if (t_end > 0 && t_end - 1 < t_wave) pv((t_end - 1) % kRing);
    }
    vm_wait<0>();  // the reloads issued past the last tile have landed

    const float l = half_sum(l_part[0] + l_part[1]);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (my_q < n) {
      uint16_t* op = Og + (size_t)my_q * qsr;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u32x2 pk;
          pk[0] = pack2<Tag>(acc[mb][4 * r] * inv, acc[mb][4 * r + 1] * inv);
          pk[1] = pack2<Tag>(acc[mb][4 * r + 2] * inv, acc[mb][4 * r + 3] * inv);
          *reinterpret_cast<u32x2*>(op + 32 * mb + 8 * r + 4 * g) = pk;
        }
      if (g == 0) Lg[my_q] = l > 0.0f ? m_run * kLn2 + logf(l) : -INFINITY;
    }
  };
  const int nqb = (n + ROWS - 1) / ROWS;
  const int qa = nqb - 1 - pb_;
  const int nrun = CAUSAL ? (pb_ < qa ? 2 : pb_ == qa ? 1 : 0) : (qa >= 0 ? 1 : 0);
#pragma clang loop unroll(disable)
  for (int r = 0; r < nrun; ++r) {
    if (r) {
      vm_wait<0>();     // the first block's DMA (reloads included) is done ...
      __syncthreads();  // ... and every wave is out of its LDS tiles
    }
    run(r ? pb_ : qa);
  }
}

template <typename Tag, int D>
hipError_t launch_d(bool causal, const FwdArgs& a, hipStream_t st) {
  timing_begin(kFwd, st);
  if (causal) hipLaunchKernelGGL((fwd2_kernel<Tag, D, true>), dim3(a.nblk), dim3(kNW * 64), 0, st, a);
  else hipLaunchKernelGGL((fwd2_kernel<Tag, D, false>), dim3(a.nblk), dim3(kNW * 64), 0, st, a);
  hipError_t e = hipGetLastError();
  timing_end(kFwd, st);
  return e;
}

template <typename Tag>
hipError_t launch_sparse64(bool causal, const FwdArgs& a, hipStream_t st) {
  timing_begin(kFwd, st);
  if (causal) hipLaunchKernelGGL((fwd2_kernel<Tag, 64, true, true>), dim3(a.nblk), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((fwd2_kernel<Tag, 64, false, true>), dim3(a.nblk), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  timing_end(kFwd, st);
  return e;
}

}  // namespace

hipError_t launch_fwd2_sparse(Dt dt, int d, bool causal, int bh, FwdArgs a, hipStream_t st) {
  if (d != 64) return hipErrorInvalidValue;
  constexpr int rows = 4 * kWR;
  a.nqb = (a.n + rows - 1) / rows;
  a.nblk = (causal ? (a.nqb + 1) / 2 : a.nqb) * bh;
  return dt == Dt::BF16 ? launch_sparse64<bf16_tag>(causal, a, st) : launch_sparse64<f16_tag>(causal, a, st);
}

hipError_t launch_fwd2(Dt dt, int d, bool causal, int bh, FwdArgs a, hipStream_t st) {
  a.nqb = (a.n + kRows - 1) / kRows;
  a.nblk = (causal ? (a.nqb + 1) / 2 : a.nqb) * bh;
  if (dt == Dt::BF16) return d == 64 ? launch_d<bf16_tag, 64>(causal, a, st) : launch_d<bf16_tag, 128>(causal, a, st);
  return d == 64 ? launch_d<f16_tag, 64>(causal, a, st) : launch_d<f16_tag, 128>(causal, a, st);
}

}  // namespace fa
