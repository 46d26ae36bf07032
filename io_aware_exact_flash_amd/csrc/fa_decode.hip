// Exact attention of a few queries against a key/value cache (decoding),
// gfx950, 16-bit inputs.
//
// At a decoding step every sequence brings Nq new queries (usually one) per
// query head, and each attends to the L cached keys and values of its
// sequence (FlashAttention-2 notes, "impact on the KV cache": grouped K/V
// heads shrink the cache such a step has to read).  The work is one pass
// over the cache, so the pass is bound by HBM bandwidth, not by the matrix
// cores; the kernel is shaped to read every cached byte once:
//
//  * Row packing.  The G = H/Hkv query heads of a K/V head and their Nq
//    queries form G*Nq rows that are contiguous in a [B][H][Nq][d] tensor;
//    one wave takes 32 or 64 of them (row tile), so K/V tiles read from the
//    cache feed every query head of the group at once.
//  * Key splits.  The cache is cut into num_splits contiguous key ranges,
//    one workgroup (one wave) per (K/V head, row tile, range), enough
//    workgroups to keep every compute unit streaming; each range writes an
//    output normalised by its own softmax sum and its log-sum-exp, and a
//    merge pass combines the ranges (Flash Attention v1 notes: merging the
//    softmax statistics of two vectors, applied to num_splits parts).  With
//    one range the kernel writes the result directly.
//  * Streaming.  32-key K and V tiles move from HBM to LDS by global->LDS
//    DMA into a ring of two slots per wave (the next tile lands while the
//    current one is computed; four such waves per compute unit keep about
//    70 KB of loads in flight per unit).  Per tile: S^T = K Q^T on
//    v_mfma_f32_32x32x16 (every query row one lane column), online softmax
//    with a running maximum per row (FlashAttention-2 notes, eqs. (5)-(7),
//    (10)), and O^T += V^T P^T with V^T read by LDS transpose reads.
//  * Causal rule with fewer queries than keys: the queries are the last Nq
//    positions of a sequence of L tokens, so query i sees key j iff
//    j <= i + L - Nq (all L keys for the last query).
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));

// c + a b on v_mfma_f32_32x32x16 (operands in the layout of fa_device.hpp);
// the compiler places the registers and handles the hazards.
template <typename Tag>
__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (std::is_same<Tag, bf16_tag>::value)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8v, a), __builtin_bit_cast(f16x8v, b), c, 0,
                                                  0, 0);
}

// Wait until this wave's LDS reads have returned (before DMA refills a slot).
__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// RB: 32-row blocks per wave (1 or 2).
template <typename Tag, int D, int RB, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_decode_kernel(DecArgs a) {
  constexpr int BC = 32;              // keys per tile
  constexpr int KS = D / 16;          // k-steps of the S^T products
  constexpr int MB = D / 32;          // 32-row blocks of O^T
  constexpr int PK = BC / 16;         // k-steps of the PV products
  using KL = Pad<D, false>;           // K: row reads
  using VL = Pad<D, true>;            // V: transpose reads
  using KD = Dma<BC, D, false, 1>;
  using VD = Dma<BC, D, true, 1>;
  constexpr int SLOT = KD::kSlot + VD::kSlot;
  constexpr int C = KD::kPer + VD::kPer;  // DMA instructions per tile
  static_assert(2 * C < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem[2 * SLOT];

  const int lane = threadIdx.x;
  const int c32 = lane & 31, g = lane >> 5;
  const int lb = blockIdx.x;
  const int split = lb % a.nsplit;
  const int rt = (lb / a.nsplit) % a.nrt;
  const int bkv = lb / (a.nsplit * a.nrt);
  const int b = bkv / a.hkv, hk = bkv % a.hkv;
  // valid cache slots of this sequence (clamped to the cache's capacity)
  const int L = a.cache_lens ? min(max(a.cache_lens[b], 0), a.nk) : a.nk;
  const int R = a.grp * a.nq;                                        // rows of the group
  const long long grow0 = ((long long)b * a.h + (long long)hk * a.grp) * a.nq;  // its first row
  const int r0 = rt * 32 * RB;
  const uint16_t* __restrict__ Qg = reinterpret_cast<const uint16_t*>(a.q) + grow0 * D;
  const long long kvo = ((long long)b * a.hkv + hk) * a.nk * D;
  const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + kvo;
  const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + kvo;

  // Q^T fragments (B operands) of the wave's rows, and each row's key limit:
  // keys below lim are visible to it (lim <= 0: none)
  u32x4 qreg[RB][KS];
  int lim[RB];
#pragma unroll
  for (int h = 0; h < RB; ++h) {
    const int r = r0 + 32 * h + c32;
    const uint16_t* qr = Qg + (size_t)min(r, R - 1) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[h][ks] = *reinterpret_cast<const u32x4*>(qr + 16 * ks);
    const int i = r % a.nq;  // position among the sequence's new queries
    lim[h] = CAUSAL ? min(L, i + L - a.nq + 1) : L;
  }

  // this workgroup's key tiles
  const int n_tiles = (L + BC - 1) / BC;
  const int chunk = (n_tiles + a.nsplit - 1) / a.nsplit;
  const int j0 = min(split * chunk, n_tiles);
  const int j1 = min(j0 + chunk, n_tiles);

  KD kd;
  VD vd;
  kd.init(0, lane);
  vd.init(0, lane);
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds_ptr(smem);
  // tile jt into slot sl (rows past the cache end re-read its last row)
  auto issue = [&](int jt, int sl) {
    const uint16_t* kt = Kg + (size_t)jt * BC * D;
    const uint16_t* vt = Vg + (size_t)jt * BC * D;
    const int last = L - 1 - jt * BC;
    const uint32_t dst = lds_base + sl * SLOT;
#pragma unroll
    for (int k = 0; k < KD::kPer; ++k) kd.issue_at(k, kt, last, 2 * D, dst);
#pragma unroll
    for (int k = 0; k < VD::kPer; ++k) vd.issue_at(k, vt, last, 2 * D, dst + KD::kSlot);
  };

  f32x16 acc[RB][MB];  // O^T
#pragma unroll
  for (int h = 0; h < RB; ++h)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[h][mb] = 0.0f;
  float m[RB], l[RB];  // running maximum (exp2 units) and this lane's partial sum
#pragma unroll
  for (int h = 0; h < RB; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
  }
  const float cs = a.c;

  vm_wait<0>();  // the Q loads are done: from here vmcnt counts tile DMA only
  if (j0 < j1) issue(j0, 0);
  if (j0 + 1 < j1) issue(j0 + 1, 1);
  for (int jt = j0; jt < j1; ++jt) {
    const int sl = (jt - j0) & 1;
    if (jt + 1 < j1) vm_wait<C>();  // tile jt has landed (jt + 1 may still be in flight)
    else vm_wait<0>();
    const lchar* base = lds_ptr(smem) + sl * SLOT;

    // S^T = K Q^T; element v of block h is key jt*BC + 4g + 8(v/4) + v%4
    f32x16 s[RB];
    f32x16 zero = 0.0f;
    {
      const lchar* kr = lds_opaque(base + KL::row_base(c32, g));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kf = ld_row(kr + KL::row_off(0, ks));
#pragma unroll
        for (int h = 0; h < RB; ++h) s[h] = mma<Tag>(kf, qreg[h][ks], ks ? s[h] : zero);
      }
    }
    // online softmax per row (the two lane halves hold different keys of
    // the same rows: maxima and sums combine across them)
    u32x4 pb[RB][PK];
#pragma unroll
    for (int h = 0; h < RB; ++h) {
      const int lv = lim[h] - jt * BC - 4 * g;
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float x = (8 * (v >> 2) + (v & 3) < lv) ? s[h][v] * cs : -INFINITY;
        s[h][v] = x;
        mx = fmaxf(mx, x);
      }
      const float mnew = fmaxf(m[h], half_max(mx));
      const float alpha = mnew == -INFINITY ? 1.0f : fast_exp2(m[h] - mnew);
      const float sub = mnew == -INFINITY ? 0.0f : mnew;
      float ls = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(s[h][v] - sub);
        s[h][v] = p;
        ls += p;
      }
      l[h] = l[h] * alpha + ls;
      m[h] = mnew;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[h][mb] *= alpha;
#pragma unroll
      for (int kk = 0; kk < PK; ++kk) pb[h][kk] = pack8<Tag>(s[h], 8 * kk);
    }
    // O^T += V^T P^T
    {
      const lchar* vt = lds_opaque(base + KD::kSlot + VL::tr_base(lane));
#pragma unroll
      for (int kk = 0; kk < PK; ++kk)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const u32x4 vf = ld_tr(vt + VL::tr_off(0, kk, 0, mb), vt + VL::tr_off(0, kk, 1, mb));
#pragma unroll
          for (int h = 0; h < RB; ++h) acc[h][mb] = mma<Tag>(vf, pb[h][kk], acc[h][mb]);
        }
    }
    // the slot is refilled with tile jt + 2 once this wave's reads of it are back
    if (jt + 2 < j1) {
      lgkm_wait0();
      issue(jt + 2, sl);
    }
  }

  // epilogue: O = O^T / l (lane column = row), LSE = m ln 2 + ln l
#pragma unroll
  for (int h = 0; h < RB; ++h) {
    const float lt = half_sum(l[h]);
    const int r = r0 + 32 * h + c32;
    if (r >= R) continue;
    const long long row = grow0 + r;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const float lse = lt > 0.0f ? m[h] * kLn2 + logf(lt) : -INFINITY;
    if (a.nsplit == 1) {
      uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + row * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 pk;
          pk[0] = pack2<Tag>(acc[h][mb][4 * q4] * inv, acc[h][mb][4 * q4 + 1] * inv);
          pk[1] = pack2<Tag>(acc[h][mb][4 * q4 + 2] * inv, acc[h][mb][4 * q4 + 3] * inv);
          *reinterpret_cast<u32x2*>(op + 32 * mb + 8 * q4 + 4 * g) = pk;
        }
      if (g == 0) a.lse[row] = lse;
    } else {
      const size_t prow = (size_t)split * a.rows + row;
      float* pp = a.po + prow * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 x;
#pragma unroll
          for (int t = 0; t < 4; ++t) x[t] = acc[h][mb][4 * q4 + t] * inv;
          *reinterpret_cast<f32x4*>(pp + 32 * mb + 8 * q4 + 4 * g) = x;
        }
      if (g == 0) a.plse[prow] = lse;
    }
  }
}

// Merge of the key ranges of one row: with the ranges' log-sum-exps L_s and
// outputs O_s (each normalised by its own sum), L = log sum_s e^{L_s} and
// O = sum_s e^{L_s - L} O_s (a range without keys has L_s = -inf, weight 0).
// D/4 threads per row, four columns each.
template <typename Tag, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecArgs a) {
  constexpr int TPR = D / 4;
  const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (row >= a.rows) return;
  const int c = 4 * (threadIdx.x % TPR);
  const int S = a.nsplit;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, a.plse[(size_t)s * a.rows + row]);
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    float wsum = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float wgt = expf(a.plse[(size_t)s * a.rows + row] - mx);
      wsum += wgt;
      o += wgt * *reinterpret_cast<const f32x4*>(a.po + ((size_t)s * a.rows + row) * D + c);
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

template <typename Tag, int D, int RB>
hipError_t launch_rb(bool causal, const DecArgs& a, hipStream_t st) {
  const long long nblk = (long long)a.nbkv * a.nrt * a.nsplit;
  timing_begin(kDecode, st);
  if (causal) hipLaunchKernelGGL((fwd_decode_kernel<Tag, D, RB, true>), dim3(nblk), dim3(64), 0, st, a);
  else hipLaunchKernelGGL((fwd_decode_kernel<Tag, D, RB, false>), dim3(nblk), dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  timing_end(kDecode, st);
  if (e != hipSuccess || a.nsplit == 1) return e;
  constexpr int kRowsPerBlock = 256 / (D / 4);
  timing_begin(kDecodeMerge, st);
  hipLaunchKernelGGL((decode_merge_kernel<Tag, D>), dim3((a.rows + kRowsPerBlock - 1) / kRowsPerBlock), dim3(256), 0,
                     st, a);
  e = hipGetLastError();
  timing_end(kDecodeMerge, st);
  return e;
}

template <typename Tag, int D>
hipError_t launch_d(bool causal, DecArgs a, hipStream_t st) {
  const int R = a.grp * a.nq;
  if (R > 32) {
    a.nrt = (R + 63) / 64;
    return launch_rb<Tag, D, 2>(causal, a, st);
  }
  a.nrt = 1;
  return launch_rb<Tag, D, 1>(causal, a, st);
}

}  // namespace

int decode_row_tiles(long long rows_per_group) { return rows_per_group > 32 ? (int)((rows_per_group + 63) / 64) : 1; }

hipError_t launch_fwd_decode(Dt dt, int d, bool causal, DecArgs a, hipStream_t st) {
  if (dt == Dt::BF16) return d == 64 ? launch_d<bf16_tag, 64>(causal, a, st) : launch_d<bf16_tag, 128>(causal, a, st);
  return d == 64 ? launch_d<f16_tag, 64>(causal, a, st) : launch_d<f16_tag, 128>(causal, a, st);
}

}  // namespace fa
