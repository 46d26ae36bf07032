// Exact-attention forward for float32 inputs on gfx950.
//
// Same online-softmax pass as the 16-bit kernel (FlashAttention-2 notes,
// Algorithm 1), but every operand stays float32: the two contractions use
// v_mfma_f32_32x32x2_f32 and P is never rounded, so the result agrees with
// a float64 evaluation to float32 accuracy.  Float32 inputs are used for
// small problems where latency, not throughput, decides: a workgroup owns 32
// query rows, and its four waves take every fourth key tile each (own LDS
// buffers, no barriers in the sweep), keeping their own running max, sum and
// output; at the end the four partial states are merged with the
// statistics merge of the v1 notes (max, rescaled sums and outputs).
//
// Operands of v_mfma_f32_32x32x2_f32 (g = lane / 32, c = lane % 32):
//   A: lane holds A[c][g]   B: lane holds B[g][c]
//   C: lane holds column c, rows 8*(v/4) + 4*g + (v%4)
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

constexpr int kBC = 32;    // keys per tile
constexpr int kWaves = 4;  // waves per workgroup, each on every fourth key tile

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(64 * kWaves) void fwd_f32_kernel(FwdArgs a) {
  constexpr int LD = D + 1;  // padded LDS row (floats)
  constexpr int MB = D / 32;
  constexpr int TILE = kBC * LD;
  static_assert(kWaves * 64 * (MB * 16 + 2) <= kWaves * 2 * TILE, "merge area fits the tile buffers");
  __shared__ float smem[kWaves * 2 * TILE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c32 = lane & 31, g = lane >> 5;
  float* ks_ = smem + w * 2 * TILE;  // this wave's K and V tiles
  float* vs_ = ks_ + TILE;
  const int lb = xcd_remap(blockIdx.x, a.nblk);
  const int bh = lb / a.nqb;
  const HeadAt at = query_head(a.sq, bh, a.n);
  const int n = at.n;
  const int qb = (n + 31) / 32 - 1 - (lb % a.nqb);  // the longest blocks first
  if (qb < 0) return;                                // past a shorter sequence
  const int qsr = a.sq.qsr, ksr = a.sq.ksr;
  const float* __restrict__ Q = reinterpret_cast<const float*>(a.q) + at.q;
  const float* __restrict__ K = reinterpret_cast<const float*>(a.k) + at.kv;
  const float* __restrict__ V = reinterpret_cast<const float*>(a.v) + at.kv;
  const int q0 = qb * 32;
  const int my_q = q0 + c32;

  float qv[D / 2];
  {
    const float* qp = Q + (size_t)min(my_q, n - 1) * qsr;
#pragma unroll
    for (int t = 0; t < D / 2; ++t) qv[t] = qp[2 * t + g];
  }

  int j_end = (n + kBC - 1) / kBC;
  if constexpr (CAUSAL) j_end = min(j_end, (min(q0 + 32, n) - 1) / kBC + 1);
  const uint8_t* mrow = SPARSE ? a.mask + (size_t)(q0 / kMaskBlock) * a.mask_t : nullptr;

  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = 0.0f;
  float m_run = -INFINITY, l_part = 0.0f;
  const float cs = a.c;

  for (int j = w; j < j_end; j += kWaves) {
    const int k0 = j * kBC;
    if constexpr (SPARSE)
      if (!mrow[k0 / kMaskBlock]) continue;
    // The buffers are this wave's own: lanes write what other lanes of the
    // same wave read.  Wavefront-scope release/acquire fences around the
    // wave barrier order those LDS accesses in the memory model (the
    // barrier alone carries no memory semantics); at wave scope they cost
    // no instructions beyond the waits the accesses need anyway.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 16-byte loads (four columns per lane), scattered into the padded rows
    for (int e = 4 * lane; e < kBC * D; e += 4 * 64) {
      const int r = e / D, col = e % D;
      const int row = min(k0 + r, n - 1);
      const f32x4 kx = *reinterpret_cast<const f32x4*>(K + (size_t)row * ksr + col);
      const f32x4 vx = *reinterpret_cast<const f32x4*>(V + (size_t)row * ksr + col);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        ks_[r * LD + col + t] = kx[t];
        vs_[r * LD + col + t] = vx[t];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x16 s = 0.0f;
#pragma unroll
    for (int t = 0; t < D / 2; ++t)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks_[c32 * LD + 2 * t + g], qv[t], s, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int key = k0 + 8 * (v >> 2) + 4 * g + (v & 3);
      bool dead = key >= n;
      if constexpr (CAUSAL) dead = dead || key > my_q;
      if (dead) s[v] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
    mx = half_max(mx);
    const float m_new = fmaxf(m_run, mx * cs);
    const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
    const float mu = (m_new == -INFINITY) ? 0.0f : m_new;
    m_run = m_new;
    float rs = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float p = fast_exp2(fmaf(s[v], cs, -mu));
      s[v] = p;
      rs += p;
    }
    l_part = l_part * alpha + rs;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x16 acc = oacc[mb] * alpha;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        int key = 8 * (kk >> 2) + 4 * g + (kk & 3);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(vs_[key * LD + 32 * mb + c32], s[kk], acc, 0, 0, 0);
      }
      oacc[mb] = acc;
    }
  }

  // merge the four waves' states: m = max_w m_w, l = sum_w e^{m_w - m} l_w,
  // O = sum_w e^{m_w - m} O_w / l (m in exp2 units; a wave that saw no key
  // has m_w = -inf and weight 0)
  __syncthreads();  // every wave is done with its tiles: the LDS is reused
  constexpr int PART = MB * 16;
  float* part = smem;                            // [wave][lane][PART] partial O^T
  float* stat = smem + kWaves * 64 * PART;       // [wave][lane][2] m, partial l
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) part[(w * 64 + lane) * PART + 16 * mb + v] = oacc[mb][v];
  stat[(w * 64 + lane) * 2] = m_run;
  stat[(w * 64 + lane) * 2 + 1] = l_part;
  __syncthreads();
  if (w != 0) return;
  float mw[kWaves], alpha_w[kWaves];
  float mstar = -INFINITY;
#pragma unroll
  for (int u = 0; u < kWaves; ++u) {
    mw[u] = stat[(u * 64 + lane) * 2];
    mstar = fmaxf(mstar, mw[u]);
  }
  float lsum = 0.0f;
#pragma unroll
  for (int u = 0; u < kWaves; ++u) {
    alpha_w[u] = (mw[u] == -INFINITY) ? 0.0f : fast_exp2(mw[u] - mstar);
    lsum = fmaf(alpha_w[u], stat[(u * 64 + lane) * 2 + 1], lsum);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float o = 0.0f;
#pragma unroll
      for (int u = 0; u < kWaves; ++u) o = fmaf(alpha_w[u], part[(u * 64 + lane) * PART + 16 * mb + v], o);
      oacc[mb][v] = o;
    }
  m_run = mstar;
  const float l = half_sum(lsum);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (my_q < n) {
    float* op = reinterpret_cast<float*>(a.o) + at.q + (size_t)my_q * qsr;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 o4;
#pragma unroll
        for (int t = 0; t < 4; ++t) o4[t] = oacc[mb][4 * r + t] * inv;
        *reinterpret_cast<f32x4*>(op + 32 * mb + 8 * r + 4 * g) = o4;
      }
    if (g == 0) a.lse[at.l + my_q] = l > 0.0f ? m_run * kLn2 + logf(l) : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(bool causal, bool sparse, const FwdArgs& a, hipStream_t st) {
  dim3 grid(a.nblk), block(64 * kWaves);
  timing_begin(kFwdF32, st);
  if (causal && sparse) hipLaunchKernelGGL((fwd_f32_kernel<D, true, true>), grid, block, 0, st, a);
  else if (causal) hipLaunchKernelGGL((fwd_f32_kernel<D, true, false>), grid, block, 0, st, a);
  else if (sparse) hipLaunchKernelGGL((fwd_f32_kernel<D, false, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((fwd_f32_kernel<D, false, false>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  timing_end(kFwdF32, st);
  return e;
}

}  // namespace

hipError_t launch_fwd_f32(int d, bool causal, bool sparse, int bh, FwdArgs a, hipStream_t st) {
  a.nqb = (a.n + 31) / 32;
  a.nblk = a.nqb * bh;
  return d == 64 ? launch_d<64>(causal, sparse, a, st) : launch_d<128>(causal, sparse, a, st);
}

}  // namespace fa
