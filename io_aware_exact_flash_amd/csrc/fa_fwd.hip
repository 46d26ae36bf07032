// Fused exact-attention forward for gfx950, 16-bit inputs.
//
// Computes, per head, O = softmax(scale * Q K^T) V and the row log-sum-exp
// L = m + ln(l) in one pass over K and V (FlashAttention-2 notes,
// Algorithm 1 and eqs. (10)-(15)): each workgroup owns 128 query rows, keeps
// Q in registers, streams K/V tiles through LDS, and never writes the score
// or probability matrix anywhere.
//
// Work split (chosen for CDNA4, not taken from the pages' A100 design):
//  * 4 waves x 32 query rows.  Each wave computes S^T = K_j Q_w^T with
//    v_mfma_f32_32x32x16, so every query row is one lane column and the
//    running statistics (m, l), the exp(m_old - m_new) rescale of the
//    accumulator, and the final division are lane-local.
//  * The accumulator is O^T = V_j^T P^T: P^T comes straight out of the S^T
//    accumulator as the B operand; V_j^T is fetched from the row-major V
//    tile with LDS transpose reads (ds_read_b64_tr_b16).
//  * 64-key tiles, double-buffered in LDS with a register prefetch: one
//    barrier per tile; padded rows make every operand fetch a per-lane base
//    plus an immediate offset.
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
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

constexpr int kNT = 256;     // threads per workgroup
constexpr int kQW = 32;      // query rows per wave
constexpr int kBR = 128;     // query rows per workgroup
constexpr float kLazy = 8.0f;

template <typename Tag, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kNT, 2) void fwd_kernel(FwdArgs a) {
  constexpr int BC = 64;              // keys per tile
  constexpr int NKB = BC / 32;        // 32-key blocks per tile
  constexpr int KS = D / 16;          // k-steps over the head dimension
  constexpr int MB = D / 32;          // 32-wide output column blocks
  constexpr int PK = BC / 16;         // k-steps of the PV product
  using KL = Pad<D, false>;           // K: row reads
  using VL = Pad<D, true>;            // V: transpose reads
  constexpr int KT = KL::bytes(BC), VT = VL::bytes(BC), BUF = KT + VT;
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c32 = lane & 31, g = lane >> 5;
  const int n = a.n;

  const int lb = xcd_remap(blockIdx.x, a.nblk);
  const int bh = lb / a.nqb;
  const int qb = a.nqb - 1 - (lb % a.nqb);  // longest causal rows first
  const size_t hoff = (size_t)bh * n * D;
  const uint16_t* __restrict__ Q = reinterpret_cast<const uint16_t*>(a.q) + hoff;
  const uint16_t* __restrict__ K = reinterpret_cast<const uint16_t*>(a.k) + hoff;
  const uint16_t* __restrict__ V = reinterpret_cast<const uint16_t*>(a.v) + hoff;

  const int q0 = qb * kBR;
  const int qw0 = q0 + w * kQW;
  const int my_q = qw0 + c32;

  u32x4 qreg[KS];
  {
    const uint16_t* qp = Q + (size_t)min(my_q, n - 1) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
  }

  const int n_tiles = (n + BC - 1) / BC;
  int j_end = n_tiles;
  if constexpr (CAUSAL) j_end = min(n_tiles, (min(q0 + kBR, n) - 1) / BC + 1);
  const uint8_t* mrow = SPARSE ? a.mask + (size_t)(q0 / kMaskBlock) * a.mask_t : nullptr;
  auto next_tile = [&](int j) {
    ++j;
    if constexpr (SPARSE)
      while (j < j_end && !mrow[(j * BC) / kMaskBlock]) ++j;
    return j;
  };

  Stage<BC, D, kNT, false> sk;
  Stage<BC, D, kNT, true> sv;
  sk.init(tid);
  sv.init(tid);
  const int kread = KL::row_base(c32, g);
  const int vread = KT + VL::tr_base(lane);

  int j = SPARSE ? next_tile(-1) : 0;
  if (j < j_end) {
    sk.load(K + (size_t)j * BC * D, n - j * BC);
    sv.load(V + (size_t)j * BC * D, n - j * BC);
    sk.store(smem);
    sv.store(smem + KT);
  }
  settle(qreg);
  __syncthreads();

  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = 0.0f;
  float m_run = -INFINITY, l_part = 0.0f;
  const float cs = a.c;
  int buf = 0;

  while (j < j_end) {
    const int jn = next_tile(j);
    if (jn < j_end) {
      sk.load(K + (size_t)jn * BC * D, n - jn * BC);
      sv.load(V + (size_t)jn * BC * D, n - jn * BC);
    }
    const char* kb_ = smem + buf * BUF + kread;
    const char* vb_ = smem + buf * BUF + vread;
    const int k0 = j * BC;
    const bool wave_live = !CAUSAL || (k0 <= qw0 + kQW - 1);
    if (wave_live) {
      f32x16 s[NKB];
      const f32x16 zero = {};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma32<Tag>(ld_row(kb_ + KL::row_off(kb, 0)), qreg[0], zero);
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          s[kb] = mfma32<Tag>(ld_row(kb_ + KL::row_off(kb, ks)), qreg[ks], s[kb]);
      }
      const bool need_mask = (CAUSAL && (k0 + BC - 1 > qw0)) || (k0 + BC > n);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            int key = k0 + 32 * kb + 8 * (v >> 2) + 4 * g + (v & 3);
            bool dead = key >= n;
            if constexpr (CAUSAL) dead = dead || key > my_q;
            if (dead) s[kb][v] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
      mx = half_max(mx);
      const float m_new = fmaxf(m_run, mx * cs);
      const bool grow = m_new > m_run + kLazy;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
        if (grow) m_run = m_new;
        l_part *= alpha;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
      }
      const float mu = (m_run == -INFINITY) ? 0.0f : m_run;
      float rs = 0.0f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float p = fast_exp2(fmaf(s[kb][v], cs, -mu));
          s[kb][v] = p;
          rs += p;
        }
      l_part += rs;
#pragma unroll
      for (int kk = 0; kk < PK; ++kk) {
        const int kb = kk >> 1, h = kk & 1;
        const u32x4 pb = pack8<Tag>(s[kb], 8 * h);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const u32x4 av = ld_tr(vb_ + VL::tr_off(kb, h, 0, mb), vb_ + VL::tr_off(kb, h, 1, mb));
          oacc[mb] = mfma32<Tag>(av, pb, oacc[mb]);
        }
      }
    }
    if (jn < j_end) {
      char* nb = smem + (buf ^ 1) * BUF;
      sk.store(nb);
      sv.store(nb + KT);
    }
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  const float l = half_sum(l_part);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (my_q < n) {
    uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + hoff + (size_t)my_q * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 pk;
        pk[0] = pack2<Tag>(oacc[mb][4 * r] * inv, oacc[mb][4 * r + 1] * inv);
        pk[1] = pack2<Tag>(oacc[mb][4 * r + 2] * inv, oacc[mb][4 * r + 3] * inv);
        *reinterpret_cast<u32x2*>(op + 32 * mb + 8 * r + 4 * g) = pk;
      }
    if (g == 0) a.lse[(size_t)bh * n + my_q] = l > 0.0f ? m_run * kLn2 + logf(l) : -INFINITY;
  }
}

template <typename Tag, int D>
hipError_t launch_d(bool causal, bool sparse, int bh, const FwdArgs& a, hipStream_t st) {
  dim3 grid(a.nblk), block(kNT);
  timing_begin(kFwd, st);
  if (causal && sparse) hipLaunchKernelGGL((fwd_kernel<Tag, D, true, true>), grid, block, 0, st, a);
  else if (causal) hipLaunchKernelGGL((fwd_kernel<Tag, D, true, false>), grid, block, 0, st, a);
  else if (sparse) hipLaunchKernelGGL((fwd_kernel<Tag, D, false, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((fwd_kernel<Tag, D, false, false>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  timing_end(kFwd, st);
  return e;
}

}  // namespace

int fwd_query_block() { return kBR; }

hipError_t launch_fwd(Dt dt, int d, bool causal, bool sparse, int bh, FwdArgs a, hipStream_t st) {
  a.nqb = (a.n + kBR - 1) / kBR;
  a.nblk = a.nqb * bh;
  if (dt == Dt::BF16) return d == 64 ? launch_d<bf16_tag, 64>(causal, sparse, bh, a, st)
                                     : launch_d<bf16_tag, 128>(causal, sparse, bh, a, st);
  return d == 64 ? launch_d<f16_tag, 64>(causal, sparse, bh, a, st)
                 : launch_d<f16_tag, 128>(causal, sparse, bh, a, st);
}

}  // namespace fa
