// C ABI of libflashattn.so: argument validation, shape bookkeeping and
// dispatch to the gfx950 kernels.  Every check runs before the first HIP
// call, so an invalid call never touches the device.
#include "../../include/flash_attn.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "fa_api_internal.hpp"
#include "fa_kernels.hpp"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
fa_status vfail(fa_status s, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  g_last_error = buf;
  return s;
}
fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(s, fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Problem {
  int B, H, N, d;
  fa_dtype dtype;
  bool empty;
  int bh;
};

// Shape/scalar checks shared by every entry point.
fa_status check_common(const char* fn, int B, int H, int N, int d, fa_dtype dtype, float scale,
                       int causal, bool backward, Problem* p) {
  if (B < 0 || H < 0 || N < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: negative size (B=%d H=%d N=%d)", fn, B, H, N);
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dtype);
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: scale must be finite and > 0 (got %g)", fn, (double)scale);
  if (causal != 0 && causal != 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: causal must be 0 or 1 (got %d)", fn, causal);
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "%s: head dimension %d not supported (64 or 128)", fn, d);
  if (backward && dtype == FA_F32)
    return fail(FA_ERR_UNSUPPORTED, "%s: float32 backward is not supported", fn);
  const long long bh = (long long)B * H;
  const long long blocks = bh * ((N + 31LL) / 32);
  if (blocks >= (1LL << 31))
    return fail(FA_ERR_UNSUPPORTED, "%s: problem too large (B*H*ceil(N/32) = %lld)", fn, blocks);
  p->B = B;
  p->H = H;
  p->N = N;
  p->d = d;
  p->dtype = dtype;
  p->bh = (int)bh;
  p->empty = (bh == 0 || N == 0);
  return FA_OK;
}

fa_status check_ptrs(const char* fn, const void* const* ptrs, const char* const* names, int count) {
  for (int i = 0; i < count; ++i) {
    if (!ptrs[i]) return fail(FA_ERR_INVALID_ARGUMENT, "%s: %s is null", fn, names[i]);
    if (!aligned16(ptrs[i]))
      return fail(FA_ERR_INVALID_ARGUMENT, "%s: %s is not 16-byte aligned", fn, names[i]);
  }
  return FA_OK;
}

// Grouped K/V heads: Hkv K/V heads serve H query heads, H / Hkv each.
fa_status check_heads(const char* fn, int H, int Hkv) {
  if (Hkv < 0) return fail(FA_ERR_INVALID_ARGUMENT, "%s: negative Hkv (%d)", fn, Hkv);
  if (H == 0 ? Hkv != 0 : (Hkv == 0 || H % Hkv != 0))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: H = %d query heads cannot share Hkv = %d K/V heads evenly", fn, H,
                Hkv);
  return FA_OK;
}

// Dropout: drop probability p in [0, 1) quantised to t / 256 with
// t = floor(256 p + 0.5) <= 255; kept values are scaled by 256 / (256 - t).
fa_status make_drop(const char* fn, float p, uint64_t seed, uint32_t offset, fa::Drop* d) {
  if (!(std::isfinite(p) && p >= 0.0f && p < 1.0f))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: dropout_p must lie in [0, 1) (got %g)", fn, (double)p);
  const double t = std::floor((double)p * 256.0 + 0.5);
  if (t > 255.0)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: dropout_p %g rounds to a drop threshold of 256/256", fn, (double)p);
  d->thr = (uint32_t)t;
  d->k0 = (uint32_t)seed;
  d->k1 = (uint32_t)(seed >> 32);
  d->offset = offset;
  d->scale = (float)(256.0 / (256.0 - t));
  return FA_OK;
}

// The kernels hold one row (or column) of the mask as bits in LDS: at most
// kMaskMaxEntries entries, i.e. N up to 128 * kMaskMaxEntries tokens.
constexpr int kMaskMaxEntries = 2048;

fa_status check_mask(const char* fn, const uint8_t* mask, int mask_block, int N) {
  if (!mask) return fail(FA_ERR_INVALID_ARGUMENT, "%s: block_mask is null", fn);
  if (mask_block != fa::kMaskBlockTokens)
    return fail(FA_ERR_UNSUPPORTED, "%s: mask_block %d not supported (must be 128)", fn, mask_block);
  if ((N + fa::kMaskBlockTokens - 1) / fa::kMaskBlockTokens > kMaskMaxEntries)
    return fail(FA_ERR_UNSUPPORTED, "%s: N = %d needs more than %d mask entries per row", fn, N, kMaskMaxEntries);
  return FA_OK;
}

fa_status hip_status(const char* fn, hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  return fail(FA_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
}

// Two float32 arrays with one entry per query row (D and the base-2 LSE;
// rows = B*H*N, or H*total for a packed batch), each followed by 256 spare
// bytes (16-byte loads of a ragged last tile may reach past the end) and
// 256-byte aligned.
size_t ws_array_bytes(long long rows) {
  size_t b = (size_t)rows * sizeof(float);
  return ((b + 255) & ~(size_t)255) + 256;
}
size_t workspace_bytes(long long rows) {
  if (rows <= 0) return 0;
  return 2 * ws_array_bytes(rows);
}
// Grouped K/V heads: when the dK/dV pass cuts each group of query heads into
// several ranges, the float32 partial dK and dV of every range follow
// ([hsplit][B*Hkv][N][d] each, 256-byte aligned).
size_t partial_bytes(long long bhkv, long long n, int d, int hsplit) {
  if (hsplit <= 1) return 0;
  const size_t b = (size_t)hsplit * (size_t)bhkv * (size_t)n * (size_t)d * sizeof(float);
  return (b + 255) & ~(size_t)255;
}
// rows: per-row entries; n: the longest sequence (sizes the partials)
size_t gqa_workspace_bytes(long long rows, long long bhkv, long long n, int d, int grp) {
  if (rows <= 0 || n <= 0) return 0;
  return workspace_bytes(rows) + 2 * partial_bytes(bhkv, n, d, fa::dkdv_head_splits(bhkv, n, grp));
}

// `seqs` null: dense [B][H][N][d] tensors with Hkv K/V heads; otherwise the
// (already validated) layout of a packed batch whose longest sequence is N.
fa_status run_fwd(const char* fn, int B, int H, int Hkv, int N, int d, fa_dtype dtype, const void* q,
                  const void* k, const void* v, float scale, int causal, const uint8_t* mask,
                  int mask_block, bool sparse, void* o, float* lse, hipStream_t stream,
                  const fa::Seqs* seqs = nullptr, const fa::Drop* drop = nullptr) {
  Problem p;
  fa_status s = check_common(fn, B, H, N, d, dtype, scale, causal, false, &p);
  if (s != FA_OK) return s;
  if (drop && dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "%s: float32 dropout is not supported", fn);
  if ((s = check_heads(fn, H, Hkv)) != FA_OK) return s;
  if (sparse && (s = check_mask(fn, mask, mask_block, N)) != FA_OK) return s;
  if (p.empty || (seqs && seqs->total == 0)) return FA_OK;
  const void* ptrs[] = {q, k, v, o, lse};
  const char* names[] = {"q", "k", "v", "o", "lse"};
  if ((s = check_ptrs(fn, ptrs, names, 5)) != FA_OK) return s;

  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.mask = sparse ? mask : nullptr;
  a.mask_t = (N + fa::kMaskBlockTokens - 1) / fa::kMaskBlockTokens;
  a.n = N;
  a.c = scale * 1.4426950408889634f;
  a.sq = seqs ? *seqs : fa::dense_seqs(H, Hkv, N, d);
  const fa::Dt dt = dtype == FA_BF16 ? fa::Dt::BF16 : fa::Dt::F16;
  hipError_t e;
  if (drop) {
    a.drop = *drop;
    e = fa::launch_fwd_dropout(dt, d, causal != 0, p.bh, a, stream);
  } else {
    if (dtype == FA_F32) e = fa::launch_fwd_f32(d, causal != 0, sparse, p.bh, a, stream);
    else if (sparse && d == 64) e = fa::launch_fwd2_sparse(dt, d, causal != 0, p.bh, a, stream);
    else if (sparse) e = fa::launch_fwd_sparse(dt, d, causal != 0, p.bh, a, stream);
    else e = fa::launch_fwd2(dt, d, causal != 0, p.bh, a, stream);
  }
  return hip_status(fn, e);
}

fa_status run_bwd(const char* fn, int B, int H, int Hkv, int N, int d, fa_dtype dtype, const void* q,
                  const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  float scale, int causal, const uint8_t* mask, int mask_block, bool sparse,
                  void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, hipStream_t stream,
                  const fa::Seqs* seqs = nullptr, const fa::Drop* drop = nullptr,
                  fa::WorkspaceFn get_ws = nullptr) {
  Problem p;
  fa_status s = check_common(fn, B, H, N, d, dtype, scale, causal, true, &p);
  if (s != FA_OK) return s;
  if ((s = check_heads(fn, H, Hkv)) != FA_OK) return s;
  if (sparse && (s = check_mask(fn, mask, mask_block, N)) != FA_OK) return s;
  if (p.empty || (seqs && seqs->total == 0)) return FA_OK;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv, ws};
  const char* names[] = {"q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "workspace"};
  // (a workspace from get_ws is checked once it has been supplied)
  if ((s = check_ptrs(fn, ptrs, names, get_ws ? 9 : 10)) != FA_OK) return s;
  const int grp = H / Hkv;
  const long long bhkv = (long long)B * Hkv;
  const int hsplit = fa::dkdv_head_splits(bhkv, N, grp);
  // per-row arrays: one per query row of every head (dense B*H*N, packed H*total)
  const long long lrows = seqs ? (long long)H * seqs->total : p.bh * (long long)N;
  const size_t need = gqa_workspace_bytes(lrows, bhkv, N, d, grp);
  if (get_ws) {
    if ((s = get_ws(fn, need, stream, &ws, &ws_bytes)) != FA_OK) return s;
    const void* wp[] = {ws};
    if ((s = check_ptrs(fn, wp, names + 9, 1)) != FA_OK) return s;
  }
  if (ws_bytes < need)
    return fail(FA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);

  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dvec = static_cast<float*>(ws);
  a.lt = reinterpret_cast<float*>(static_cast<char*>(ws) + ws_array_bytes(lrows));
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.mask = sparse ? mask : nullptr;
  a.mask_t = (N + fa::kMaskBlockTokens - 1) / fa::kMaskBlockTokens;
  a.n = N;
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  a.sq = seqs ? *seqs : fa::dense_seqs(H, Hkv, N, d);
  a.hsplit = hsplit;
  a.nbhkv = (int)bhkv;
  a.hkv = Hkv;
  if (hsplit > 1) {
    char* part = static_cast<char*>(ws) + workspace_bytes(lrows);
    a.pdk = reinterpret_cast<float*>(part);
    a.pdv = reinterpret_cast<float*>(part + partial_bytes(bhkv, N, d, hsplit));
  }
  const fa::Dt dt = dtype == FA_BF16 ? fa::Dt::BF16 : fa::Dt::F16;
  hipError_t e;
  if (drop) {
    a.drop = *drop;
    e = fa::launch_bwd_dropout(dt, d, causal != 0, p.bh, a, stream);
  } else {
    e = fa::launch_bwd(dt, d, causal != 0, sparse, p.bh, a, stream);
  }
  return hip_status(fn, e);
}

// Packed variable-length batches: q, o, dout, dq [total][H][d]; k, v, dk, dv
// [total][Hkv][d]; lse and the per-row workspace arrays [H][total].
fa_status check_varlen(const char* fn, int B, int H, int Hkv, int total, int max_seqlen, int d,
                       const int* cu, fa::Seqs* out) {
  if (total < 0 || max_seqlen < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: negative size (total=%d max_seqlen=%d)", fn, total, max_seqlen);
  fa_status s = check_heads(fn, H, Hkv);
  if (s != FA_OK) return s;
  if (B > 0 && !cu) return fail(FA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is null", fn);
  if (cu && (reinterpret_cast<uintptr_t>(cu) & 3u))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is not 4-byte aligned", fn);
  // the kernels form row offsets in bytes with 24-bit multiplies
  if ((long long)H * d * 2 >= (1LL << 24))
    return fail(FA_ERR_UNSUPPORTED, "%s: row stride H*d = %lld elements too large", fn, (long long)H * d);
  fa::Seqs q{};
  q.cu = cu;
  q.qsh = d;
  q.qsr = H * d;
  q.ksh = d;
  q.ksr = Hkv * d;
  q.lb = 0;
  q.lh = total;
  q.hq = H;
  q.grp = Hkv > 0 ? H / Hkv : 1;
  q.total = total;
  q.nb = B;
  *out = q;
  return FA_OK;
}

// Split-KV workspace: num_splits float32 [B*H][N][d] partial outputs, then
// num_splits float32 [B*H][N] partial log-sum-exps (256-byte aligned).
size_t splitkv_po_bytes(long long bh, long long n, int d, int splits) {
  const size_t b = (size_t)splits * (size_t)bh * (size_t)n * (size_t)d * sizeof(float);
  return (b + 255) & ~(size_t)255;
}
size_t splitkv_workspace_bytes(long long bh, long long n, int d, int splits) {
  if (bh <= 0 || n <= 0 || splits <= 0) return 0;
  return splitkv_po_bytes(bh, n, d, splits) + (size_t)splits * (size_t)bh * (size_t)n * sizeof(float);
}
constexpr int kMaxSplits = 64;

fa_status run_fwd_split(const char* fn, int B, int H, int N, int d, fa_dtype dtype, const void* q,
                        const void* k, const void* v, float scale, int causal, int splits, void* o,
                        float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  Problem p;
  fa_status s = check_common(fn, B, H, N, d, dtype, scale, causal, false, &p);
  if (s != FA_OK) return s;
  if (splits < 1 || splits > kMaxSplits)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: num_splits %d outside 1..%d", fn, splits, kMaxSplits);
  if (dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "%s: float32 split-KV forward is not supported", fn);
  if ((long long)p.bh * ((N + 255LL) / 256) * splits >= (1LL << 31))
    return fail(FA_ERR_UNSUPPORTED, "%s: problem too large for %d splits", fn, splits);
  if (p.empty) return FA_OK;
  const void* ptrs[] = {q, k, v, o, lse, ws};
  const char* names[] = {"q", "k", "v", "o", "lse", "workspace"};
  if ((s = check_ptrs(fn, ptrs, names, 6)) != FA_OK) return s;
  const size_t need = splitkv_workspace_bytes(p.bh, N, d, splits);
  if (ws_bytes < need)
    return fail(FA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);

  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.mask = nullptr;
  a.mask_t = 0;
  a.n = N;
  a.c = scale * 1.4426950408889634f;
  a.sq = fa::dense_seqs(H, H, N, d);
  a.nsplit = splits;
  a.po = static_cast<float*>(ws);
  a.plse = reinterpret_cast<float*>(static_cast<char*>(ws) + splitkv_po_bytes(p.bh, N, d, splits));
  hipError_t e = fa::launch_fwd_split(dtype == FA_BF16 ? fa::Dt::BF16 : fa::Dt::F16, d, causal != 0, p.bh, a,
                                      stream);
  return hip_status(fn, e);
}

// ---------------------------------------------------------------- KV-cache decoding
// Workspace of flash_attn_fwd_kvcache: with num_splits > 1, num_splits
// float32 partial outputs [B*H*Nq][d] then num_splits float32 partial
// log-sum-exps [B*H*Nq] (256-byte aligned); none with one range.
size_t kvcache_workspace_bytes(long long rows, int d, int splits) {
  if (rows <= 0 || splits <= 1) return 0;
  const size_t po = ((size_t)splits * (size_t)rows * (size_t)d * sizeof(float) + 255) & ~(size_t)255;
  return po + (size_t)splits * (size_t)rows * sizeof(float);
}

fa_status check_kvcache(const char* fn, int B, int H, int Hkv, int Nq, int Nk, int d, fa_dtype dtype, float scale,
                        int causal, int splits) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: negative size (B=%d H=%d Nq=%d Nk=%d)", fn, B, H, Nq, Nk);
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dtype);
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: scale must be finite and > 0 (got %g)", fn, (double)scale);
  if (causal != 0 && causal != 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: causal must be 0 or 1 (got %d)", fn, causal);
  if (splits < 1 || splits > kMaxSplits)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: num_splits %d outside 1..%d", fn, splits, kMaxSplits);
  fa_status s = check_heads(fn, H, Hkv);
  if (s != FA_OK) return s;
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "%s: head dimension %d not supported (64 or 128)", fn, d);
  if (dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "%s: float32 is not supported", fn);
  const long long rows = (long long)B * H * Nq;
  const long long grp_rows = Hkv > 0 ? (long long)(H / Hkv) * Nq : 0;
  const long long wgs = (long long)B * Hkv * fa::decode_row_tiles(grp_rows) * splits;
  if (rows * d >= (1LL << 40) || grp_rows >= (1LL << 30) || wgs >= (1LL << 31) ||
      (long long)B * Hkv * Nk * (long long)d >= (1LL << 40))
    return fail(FA_ERR_UNSUPPORTED, "%s: problem too large", fn);
  return FA_OK;
}

// ---------------------------------------------------------------- timing
struct Mark {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<hipEvent_t> g_event_pool;
std::vector<Mark> g_marks;
int g_open_kernel = -1;
hipEvent_t g_open_start = nullptr;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

const char* kKernelNames[fa::kNumKernels] = {"fwd",          "fwd_f32",   "bwd_pre",         "bwd_dkdv",
                                            "bwd_dq",       "fwd_split", "fwd_merge",       "bwd_dkdv_reduce",
                                            "fwd_dropout",  "bwd_dkdv_dropout", "bwd_dq_dropout", "fwd_decode",
                                            "fwd_decode_merge"};

}  // namespace

namespace fa {
fa_status fail_status(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(s, fmt, ap);
  va_end(ap);
  return s;
}

fa_status bwd_dense_with(const char* fn, int B, int H, int N, int d, fa_dtype dtype, const void* q, const void* k,
                         const void* v, const void* o, const void* dout, const float* lse, float scale, int causal,
                         void* dq, void* dk, void* dv, WorkspaceFn get_ws, hipStream_t stream) {
  return run_bwd(fn, B, H, H, N, d, dtype, q, k, v, o, dout, lse, scale, causal, nullptr, 0, false, dq, dk, dv,
                 nullptr, 0, stream, nullptr, nullptr, get_ws);
}

void timing_begin(int kernel, hipStream_t st) {
  std::lock_guard<std::mutex> g(g_timing_mu);
  if (!g_timing_on) return;
  g_open_start = take_event();
  g_open_kernel = kernel;
  if (g_open_start) hipEventRecord(g_open_start, st);
}
void timing_end(int kernel, hipStream_t st) {
  std::lock_guard<std::mutex> g(g_timing_mu);
  if (!g_timing_on || g_open_kernel != kernel || !g_open_start) return;
  hipEvent_t stop = take_event();
  if (!stop) return;
  hipEventRecord(stop, st);
  g_marks.push_back({kernel, g_open_start, stop});
  g_open_start = nullptr;
  g_open_kernel = -1;
}
}  // namespace fa

FA_EXPORT fa_status flash_attn_timing_enable(int enable) {
  std::lock_guard<std::mutex> g(g_timing_mu);
  g_timing_on = enable != 0;
  return FA_OK;
}

FA_EXPORT fa_status flash_attn_timing_collect(double* total_ms, int* launches, int n) {
  if ((!total_ms || !launches) && n > 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "flash_attn_timing_collect: null output array");
  std::lock_guard<std::mutex> g(g_timing_mu);
  for (int i = 0; i < n; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  fa_status st = FA_OK;
  for (const Mark& m : g_marks) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(m.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, m.start, m.stop);
    if (e != hipSuccess && st == FA_OK)
      st = fail(FA_ERR_HIP, "flash_attn_timing_collect: %s", hipGetErrorString(e));
    if (m.kernel < n && e == hipSuccess) {
      total_ms[m.kernel] += ms;
      launches[m.kernel] += 1;
    }
    g_event_pool.push_back(m.start);
    g_event_pool.push_back(m.stop);
  }
  g_marks.clear();
  return st;
}

FA_EXPORT const char* flash_attn_kernel_name(int kernel) {
  return (kernel >= 0 && kernel < fa::kNumKernels) ? kKernelNames[kernel] : "";
}

FA_EXPORT int flash_attn_abi_version(void) { return 1; }

FA_EXPORT fa_status flash_attn_fwd(int B, int H, int N, int d, fa_dtype dtype, const void* q,
                                   const void* k, const void* v, float scale, int causal, void* o,
                                   float* lse, hipStream_t stream) {
  return run_fwd("flash_attn_fwd", B, H, H, N, d, dtype, q, k, v, scale, causal, nullptr, 0, false, o,
                 lse, stream);
}

FA_EXPORT size_t flash_attn_fwd_splitkv_workspace_size(int B, int H, int N, int d, fa_dtype dtype,
                                                       int num_splits) {
  (void)dtype;
  if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
  return splitkv_workspace_bytes((long long)B * H, N, d, num_splits);
}

// Ranges that bring the forward to about two workgroups per compute unit
// (512 on a 256-CU MI355X) while every range keeps at least eight 32-key
// tiles; 1 when the plain forward already has that many workgroups.
FA_EXPORT int flash_attn_fwd_splitkv_num_splits(int B, int H, int N, int d, int causal) {
  (void)d;
  if (B <= 0 || H <= 0 || N <= 0) return 1;
  const long long nqb = (N + 255) / 256;
  const long long plain = (causal ? (nqb + 1) / 2 : nqb) * (long long)B * H;  // paired causal blocks
  if (plain >= 512) return 1;
  const long long split_wgs = nqb * (long long)B * H;  // split mode does not pair blocks
  long long s = (512 + split_wgs - 1) / split_wgs;
  const long long by_tiles = ((N + 31) / 32) / 8;
  if (s > by_tiles) s = by_tiles;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

FA_EXPORT fa_status flash_attn_fwd_splitkv(int B, int H, int N, int d, fa_dtype dtype, const void* q,
                                           const void* k, const void* v, float scale, int causal,
                                           int num_splits, void* o, float* lse, void* workspace,
                                           size_t workspace_bytes_, hipStream_t stream) {
  return run_fwd_split("flash_attn_fwd_splitkv", B, H, N, d, dtype, q, k, v, scale, causal, num_splits, o,
                       lse, workspace, workspace_bytes_, stream);
}

FA_EXPORT size_t flash_attn_bwd_workspace_size(int B, int H, int N, int d, fa_dtype dtype) {
  (void)d;
  (void)dtype;
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return workspace_bytes((long long)B * H * N);
}

FA_EXPORT fa_status flash_attn_bwd(int B, int H, int N, int d, fa_dtype dtype, const void* q,
                                   const void* k, const void* v, const void* o, const void* dout,
                                   const float* lse, float scale, int causal, void* dq, void* dk,
                                   void* dv, void* workspace, size_t workspace_bytes_,
                                   hipStream_t stream) {
  return run_bwd("flash_attn_bwd", B, H, H, N, d, dtype, q, k, v, o, dout, lse, scale, causal, nullptr,
                 0, false, dq, dk, dv, workspace, workspace_bytes_, stream);
}

FA_EXPORT fa_status flash_attn_blocksparse_fwd(int B, int H, int N, int d, fa_dtype dtype,
                                               const void* q, const void* k, const void* v,
                                               float scale, int causal, const uint8_t* block_mask,
                                               int mask_block, void* o, float* lse,
                                               hipStream_t stream) {
  return run_fwd("flash_attn_blocksparse_fwd", B, H, H, N, d, dtype, q, k, v, scale, causal, block_mask,
                 mask_block, true, o, lse, stream);
}

FA_EXPORT fa_status flash_attn_blocksparse_bwd(int B, int H, int N, int d, fa_dtype dtype,
                                               const void* q, const void* k, const void* v,
                                               const void* o, const void* dout, const float* lse,
                                               float scale, int causal, const uint8_t* block_mask,
                                               int mask_block, void* dq, void* dk, void* dv,
                                               void* workspace, size_t workspace_bytes_,
                                               hipStream_t stream) {
  return run_bwd("flash_attn_blocksparse_bwd", B, H, H, N, d, dtype, q, k, v, o, dout, lse, scale,
                 causal, block_mask, mask_block, true, dq, dk, dv, workspace, workspace_bytes_,
                 stream);
}

FA_EXPORT fa_status flash_attn_fwd_gqa(int B, int H, int Hkv, int N, int d, fa_dtype dtype, const void* q,
                                       const void* k, const void* v, float scale, int causal, void* o,
                                       float* lse, hipStream_t stream) {
  return run_fwd("flash_attn_fwd_gqa", B, H, Hkv, N, d, dtype, q, k, v, scale, causal, nullptr, 0, false, o,
                 lse, stream);
}

FA_EXPORT size_t flash_attn_bwd_gqa_workspace_size(int B, int H, int Hkv, int N, int d, fa_dtype dtype) {
  (void)dtype;
  if (B <= 0 || H <= 0 || N <= 0 || Hkv <= 0 || H % Hkv != 0 || (d != 64 && d != 128)) return 0;
  return gqa_workspace_bytes((long long)B * H * N, (long long)B * Hkv, N, d, H / Hkv);
}

FA_EXPORT fa_status flash_attn_bwd_gqa(int B, int H, int Hkv, int N, int d, fa_dtype dtype, const void* q,
                                       const void* k, const void* v, const void* o, const void* dout,
                                       const float* lse, float scale, int causal, void* dq, void* dk, void* dv,
                                       void* workspace, size_t workspace_bytes_, hipStream_t stream) {
  return run_bwd("flash_attn_bwd_gqa", B, H, Hkv, N, d, dtype, q, k, v, o, dout, lse, scale, causal, nullptr, 0,
                 false, dq, dk, dv, workspace, workspace_bytes_, stream);
}

FA_EXPORT fa_status flash_attn_varlen_fwd(int B, int H, int Hkv, int total, int max_seqlen, int d,
                                          fa_dtype dtype, const int* cu_seqlens, const void* q, const void* k,
                                          const void* v, float scale, int causal, void* o, float* lse,
                                          hipStream_t stream) {
  const char* fn = "flash_attn_varlen_fwd";
  fa::Seqs sq;
  fa_status s = check_varlen(fn, B, H, Hkv, total, max_seqlen, d, cu_seqlens, &sq);
  if (s != FA_OK) return s;
  return run_fwd(fn, B, H, Hkv, max_seqlen, d, dtype, q, k, v, scale, causal, nullptr, 0, false, o, lse, stream,
                 &sq);
}

FA_EXPORT size_t flash_attn_varlen_bwd_workspace_size(int B, int H, int Hkv, int total, int max_seqlen, int d,
                                                      fa_dtype dtype) {
  (void)dtype;
  if (B <= 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || total <= 0 || max_seqlen <= 0 || (d != 64 && d != 128))
    return 0;
  return gqa_workspace_bytes((long long)H * total, (long long)B * Hkv, max_seqlen, d, H / Hkv);
}

FA_EXPORT fa_status flash_attn_varlen_bwd(int B, int H, int Hkv, int total, int max_seqlen, int d,
                                          fa_dtype dtype, const int* cu_seqlens, const void* q, const void* k,
                                          const void* v, const void* o, const void* dout, const float* lse,
                                          float scale, int causal, void* dq, void* dk, void* dv, void* workspace,
                                          size_t workspace_bytes_, hipStream_t stream) {
  const char* fn = "flash_attn_varlen_bwd";
  fa::Seqs sq;
  fa_status s = check_varlen(fn, B, H, Hkv, total, max_seqlen, d, cu_seqlens, &sq);
  if (s != FA_OK) return s;
  return run_bwd(fn, B, H, Hkv, max_seqlen, d, dtype, q, k, v, o, dout, lse, scale, causal, nullptr, 0, false, dq,
                 dk, dv, workspace, workspace_bytes_, stream, &sq);
}

FA_EXPORT fa_status flash_attn_fwd_dropout(int B, int H, int N, int d, fa_dtype dtype, const void* q,
                                           const void* k, const void* v, float scale, int causal, float dropout_p,
                                           uint64_t seed, uint32_t offset, void* o, float* lse,
                                           hipStream_t stream) {
  const char* fn = "flash_attn_fwd_dropout";
  fa::Drop dr;
  fa_status s = make_drop(fn, dropout_p, seed, offset, &dr);
  if (s != FA_OK) return s;
  return run_fwd(fn, B, H, H, N, d, dtype, q, k, v, scale, causal, nullptr, 0, false, o, lse, stream, nullptr,
                 &dr);
}

FA_EXPORT fa_status flash_attn_bwd_dropout(int B, int H, int N, int d, fa_dtype dtype, const void* q,
                                           const void* k, const void* v, const void* o, const void* dout,
                                           const float* lse, float scale, int causal, float dropout_p,
                                           uint64_t seed, uint32_t offset, void* dq, void* dk, void* dv,
                                           void* workspace, size_t workspace_bytes_, hipStream_t stream) {
  const char* fn = "flash_attn_bwd_dropout";
  fa::Drop dr;
  fa_status s = make_drop(fn, dropout_p, seed, offset, &dr);
  if (s != FA_OK) return s;
  return run_bwd(fn, B, H, H, N, d, dtype, q, k, v, o, dout, lse, scale, causal, nullptr, 0, false, dq, dk, dv,
                 workspace, workspace_bytes_, stream, nullptr, &dr);
}

FA_EXPORT fa_status flash_attn_varlen_fwd_dropout(int B, int H, int Hkv, int total, int max_seqlen, int d,
                                                  fa_dtype dtype, const int* cu_seqlens, const void* q,
                                                  const void* k, const void* v, float scale, int causal,
                                                  float dropout_p, uint64_t seed, uint32_t offset, void* o,
                                                  float* lse, hipStream_t stream) {
  const char* fn = "flash_attn_varlen_fwd_dropout";
  fa::Seqs sq;
  fa::Drop dr;
  fa_status s = check_varlen(fn, B, H, Hkv, total, max_seqlen, d, cu_seqlens, &sq);
  if (s != FA_OK) return s;
  if ((s = make_drop(fn, dropout_p, seed, offset, &dr)) != FA_OK) return s;
  return run_fwd(fn, B, H, Hkv, max_seqlen, d, dtype, q, k, v, scale, causal, nullptr, 0, false, o, lse, stream,
                 &sq, &dr);
}

FA_EXPORT fa_status flash_attn_varlen_bwd_dropout(int B, int H, int Hkv, int total, int max_seqlen, int d,
                                                  fa_dtype dtype, const int* cu_seqlens, const void* q,
                                                  const void* k, const void* v, const void* o, const void* dout,
                                                  const float* lse, float scale, int causal, float dropout_p,
                                                  uint64_t seed, uint32_t offset, void* dq, void* dk, void* dv,
                                                  void* workspace, size_t workspace_bytes_, hipStream_t stream) {
  const char* fn = "flash_attn_varlen_bwd_dropout";
  fa::Seqs sq;
  fa::Drop dr;
  fa_status s = check_varlen(fn, B, H, Hkv, total, max_seqlen, d, cu_seqlens, &sq);
  if (s != FA_OK) return s;
  if ((s = make_drop(fn, dropout_p, seed, offset, &dr)) != FA_OK) return s;
  return run_bwd(fn, B, H, Hkv, max_seqlen, d, dtype, q, k, v, o, dout, lse, scale, causal, nullptr, 0, false, dq,
                 dk, dv, workspace, workspace_bytes_, stream, &sq, &dr);
}

FA_EXPORT size_t flash_attn_fwd_kvcache_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d, fa_dtype dtype,
                                                       int num_splits) {
  (void)dtype;
  (void)Nk;
  if (B <= 0 || H <= 0 || Nq <= 0 || (d != 64 && d != 128) || num_splits < 1 || num_splits > kMaxSplits) return 0;
  return kvcache_workspace_bytes((long long)B * H * Nq, d, num_splits);
}

// Ranges that give about four workgroups (one wave each) per compute unit
// of a 256-CU MI355X, each range keeping at least four 32-key tiles of the
// cache, at most 64.
FA_EXPORT int flash_attn_fwd_kvcache_num_splits(int B, int H, int Hkv, int Nq, int Nk, int d) {
  (void)d;
  if (B <= 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || Nq <= 0 || Nk <= 0) return 1;
  const long long wgs = (long long)B * Hkv * fa::decode_row_tiles((long long)(H / Hkv) * Nq);
  long long s = (1024 + wgs - 1) / wgs;
  const long long by_tiles = ((Nk + 31) / 32 + 3) / 4;
  if (s > by_tiles) s = by_tiles;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

FA_EXPORT fa_status flash_attn_fwd_kvcache(int B, int H, int Hkv, int Nq, int Nk, int d, fa_dtype dtype,
                                           const void* q, const void* k, const void* v, const int* cache_seqlens,
                                           float scale, int causal, int num_splits, void* o, float* lse,
                                           void* workspace, size_t workspace_bytes_, hipStream_t stream) {
  const char* fn = "flash_attn_fwd_kvcache";
  fa_status s = check_kvcache(fn, B, H, Hkv, Nq, Nk, d, dtype, scale, causal, num_splits);
  if (s != FA_OK) return s;
  const long long rows = (long long)B * H * Nq;
  if (rows == 0) return FA_OK;
  const void* ptrs[] = {q, o, lse};
  const char* names[] = {"q", "o", "lse"};
  if ((s = check_ptrs(fn, ptrs, names, 3)) != FA_OK) return s;
  if (Nk > 0) {
    const void* kv[] = {k, v};
    const char* kvn[] = {"k", "v"};
    if ((s = check_ptrs(fn, kv, kvn, 2)) != FA_OK) return s;
  }
  if (cache_seqlens && (reinterpret_cast<uintptr_t>(cache_seqlens) & 3u))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: cache_seqlens is not 4-byte aligned", fn);
  const size_t need = kvcache_workspace_bytes(rows, d, num_splits);
  if (need > 0) {
    if (!workspace) return fail(FA_ERR_INVALID_ARGUMENT, "%s: workspace is null", fn);
    if (workspace_bytes_ < need)
      return fail(FA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes_, need);
    if (!aligned16(workspace)) return fail(FA_ERR_INVALID_ARGUMENT, "%s: workspace is not 16-byte aligned", fn);
  }
  fa::DecArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cache_lens = cache_seqlens;
  a.h = H;
  a.hkv = Hkv;
  a.grp = H / Hkv;
  a.nq = Nq;
  a.nk = Nk;
  a.nbkv = B * Hkv;
  a.nsplit = num_splits;
  a.rows = rows;
  a.c = scale * 1.4426950408889634f;
  if (num_splits > 1) {
    a.po = static_cast<float*>(workspace);
    a.plse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      (((size_t)num_splits * (size_t)rows * (size_t)d * sizeof(float) + 255) &
                                       ~(size_t)255));
  }
  return hip_status(fn, fa::launch_fwd_decode(dtype == FA_BF16 ? fa::Dt::BF16 : fa::Dt::F16, d, causal != 0, a,
                                              stream));
}

FA_EXPORT const char* flash_attn_status_string(fa_status status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE_TOO_SMALL: return "FA_ERR_WORKSPACE_TOO_SMALL";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_UNKNOWN_STATUS";
}

FA_EXPORT const char* flash_attn_last_error(void) { return g_last_error.c_str(); }
