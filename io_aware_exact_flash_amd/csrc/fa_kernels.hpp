// Kernel argument blocks and host-side launchers shared by the kernel
// translation units and the C ABI in fa_api.cpp.  Nothing here is exported.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum class Dt : int { F32 = 0, F16 = 1, BF16 = 2 };

constexpr int kMaskBlockTokens = 128;  // tokens per block-mask entry

// Where the rows of one (batch, head) live.  Row t of head h of batch b of
// a per-token tensor starts at element
//     b * sb + h * sh + t * sr            (batched layouts), or
//     (cu[b] + t) * sr + h * sh           (packed variable-length batches);
// the per-row float arrays (LSE, D and the base-2 LSE) at
//     b * lb + h * lh + t   or   cu[b] + h * lh + t.
// Query-side tensors (q, o, dout, dq) and key-side tensors (k, v, dk, dv)
// each have their own strides; a K/V head serves grp consecutive query heads.
struct Seqs {
  const int* cu;         // [B+1] sequence starts of a packed batch (device), or nullptr
  long long qsb, qsh;    // query side: batch and head strides (elements)
  long long ksb, ksh;    // key side
  int qsr, ksr;          // row strides (elements, multiples of 8)
  long long lb, lh;      // per-row arrays: batch and head strides
  int hq;                // query heads per batch (H)
  int grp;               // query heads per K/V head (H / Hkv)
  int total;             // packed batches: rows in all (sequence bounds are clamped to it)
  int nb;                // packed batches: number of sequences
};

// Dense [B][H][N][d] tensors with Hkv K/V heads; LSE [B][H][N].
inline Seqs dense_seqs(int H, int Hkv, int N, int d) {
  Seqs s{};
  s.cu = nullptr;
  s.qsh = (long long)N * d;
  s.qsb = s.qsh * H;
  s.ksh = (long long)N * d;
  s.ksb = s.ksh * Hkv;
  s.qsr = d;
  s.ksr = d;
  s.lh = N;
  s.lb = (long long)N * H;
  s.hq = H;
  s.grp = Hkv > 0 ? H / Hkv : 1;
  return s;
}

// One query head (batch b, head h): element offsets of its rows, of its
// K/V head's rows and of its per-row arrays, and its length (n_max unless
// the batch is packed).
struct HeadAt {
  long long q, kv, l;
  int n;
};
__device__ __forceinline__ HeadAt head_at(const Seqs& s, int b, int h, int n_max);

// Linear head index -> (batch, head), `heads` heads per batch.  Dense
// batches enumerate heads batch-major.  Packed batches enumerate them
// head-major, so that the contiguous ranges of heads the workgroup
// remapping gives each XCD hold sequences of every length (balanced work).
__device__ __forceinline__ void split_bh(const Seqs& s, int bh, int heads, int& b, int& h) {
  if (s.cu) {
    b = bh % s.nb;
    h = bh / s.nb;
  } else {
    b = bh / heads;
    h = bh % heads;
  }
}
// Query head bh (over B x H).
__device__ __forceinline__ HeadAt query_head(const Seqs& s, int bh, int n_max) {
  int b, h;
  split_bh(s, bh, s.hq, b, h);
  return head_at(s, b, h, n_max);
}
// b*H + h of query head bh (the head index of the dropout counter).
__device__ __forceinline__ int canon_head(const Seqs& s, int bh) {
  int b, h;
  split_bh(s, bh, s.hq, b, h);
  return b * s.hq + h;
}
// The first query head of K/V head bh (over B x Hkv, hkv per batch).
__device__ __forceinline__ HeadAt group_head(const Seqs& s, int bh, int hkv, int n_max) {
  int b, hk;
  split_bh(s, bh, hkv, b, hk);
  return head_at(s, b, hk * s.grp, n_max);
}

__device__ __forceinline__ HeadAt head_at(const Seqs& s, int b, int h, int n_max) {
  HeadAt r;
  const int hk = s.grp == 1 ? h : h / s.grp;
  if (s.cu) {
    // clamped, so that inconsistent offsets cannot reach outside the tensors
    const int t0 = min(max(s.cu[b], 0), s.total);
    r.n = min(max(s.cu[b + 1] - t0, 0), min(n_max, s.total - t0));
    r.q = (long long)t0 * s.qsr + h * s.qsh;
    r.kv = (long long)t0 * s.ksr + hk * s.ksh;
    r.l = t0 + h * s.lh;
  } else {
    r.n = n_max;
    r.q = b * s.qsb + h * s.qsh;
    r.kv = b * s.ksb + hk * s.ksh;
    r.l = b * s.lb + h * s.lh;
  }
  return r;
}

// Dropout of the attention probabilities: element (query i, key j) of
// query head bh (b*H + h) is kept iff byte j%4 of word i%4 of
// Philox4x32-10(counter (i/4, j/4, bh, offset), key (k0, k1)) is at least
// thr (drop probability thr/256); kept probabilities are scaled by
// scale = 256 / (256 - thr).
struct Drop {
  uint32_t k0, k1;       // seed, low and high words
  uint32_t offset;
  uint32_t thr;          // 0 .. 255
  float scale;
};

// Forward: heads of up to N rows (N = the longest sequence when packed).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;            // [B*H*N] natural-log log-sum-exp
  const uint8_t* mask;   // [T][T] block mask or nullptr
  int mask_t;            // T = ceil(N / 128)
  int n;                 // tokens per head
  int nqb;               // query blocks per head
  int nblk;              // total workgroups
  float c;               // scale * log2(e)
  Seqs sq;               // layout of the tensors and of lse
  Drop drop;             // dropout kernels only
  // split-KV forward only (dense layout)
  int nsplit;            // key ranges per query row
  int nbh;               // B*H
  float* po;             // [nsplit][B*H][N][d] partial outputs, each normalised by its own l
  float* plse;           // [nsplit][B*H][N] partial log-sum-exp (-inf: no key in the range)
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;      // [B*H*N]
  float* dvec;           // [B*H*N] rowsum(dO o O), written by the pre-pass
  float* lt;             // [B*H*N] LSE * log2(e), +inf where LSE = -inf (pre-pass)
  void* dq;
  void* dk;
  void* dv;
  const uint8_t* mask;
  int mask_t;
  int n;
  int nblk_q;            // workgroups of the dQ pass
  int nqb;               // query blocks per head (dQ pass)
  int nblk_kv;           // workgroups of the dK/dV pass
  int nkb;               // key blocks per head (dK/dV pass)
  float scale;
  float c;               // scale * log2(e)
  // layout of the tensors, of lse and of the workspace arrays dvec and lt;
  // the dK/dV pass runs per K/V head and sums over the grp query heads that
  // share it
  Seqs sq;
  Drop drop;             // dropout kernels only
  // hsplit > 1: the group's query heads are cut into hsplit ranges swept by
  // separate workgroups, each writing scaled float32 partial dK, dV; a
  // reduction pass sums them into dk, dv
  int hsplit;
  int nbhkv;             // B*Hkv
  float* pdk;            // [hsplit][B*Hkv][N][d] (N = the longest sequence)
  float* pdv;            // [hsplit][B*Hkv][N][d]
  int hkv;               // K/V heads per batch
};

// Decoding against a key/value cache: q [B][H][nq][d], k, v [B][Hkv][nk][d]
// (nk cache slots, the first cache_lens[b] valid), o [B][H][nq][d], lse
// [B][H][nq].  The grp query heads of a K/V head and their nq queries are
// the group's grp*nq rows (contiguous in q, o and lse).
struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* cache_lens;  // [B] device, or nullptr (every sequence holds nk keys)
  int h, hkv, grp;        // query heads, K/V heads, query heads per K/V head
  int nq, nk;             // queries per head, cache slots per head
  int nbkv;               // B * Hkv
  int nrt;                // row tiles per group (set by the launcher)
  int nsplit;             // key ranges
  long long rows;         // B * H * nq
  float c;                // scale * log2(e)
  float* po;              // [nsplit][rows][d] partial outputs (nsplit > 1)
  float* plse;            // [nsplit][rows] partial log-sum-exps
};

// (K/V head, key block) units the dK/dV pass aims for before it cuts groups
// of query heads into ranges: four per compute unit of a 256-CU MI355X (a
// causal launch pairs two units per workgroup, so two workgroups per unit).
constexpr int kDkDvTargetUnits = 1024;
constexpr int kDkDvKeys = 128;  // keys per dK/dV unit

// Ranges the group of grp query heads is cut into (1 = no partials): enough
// units to fill the GPU, never more ranges than heads.  Depends on the shape
// only, so the workspace size can be computed before the call.
inline int dkdv_head_splits(long long bhkv, long long n, int grp) {
  if (grp <= 1 || bhkv <= 0 || n <= 0) return 1;
  const long long units = (n + kDkDvKeys - 1) / kDkDvKeys * bhkv;
  long long s = (kDkDvTargetUnits + units - 1) / units;
  if (s > grp) s = grp;
  return s < 1 ? 1 : (int)s;
}

// Kernel classes for the optional per-kernel timing hooks.
enum KernelId : int {
  kFwd = 0, kFwdF32 = 1, kBwdPre = 2, kBwdDkDv = 3, kBwdDq = 4, kFwdSplit = 5, kFwdMerge = 6,
  kBwdDkDvReduce = 7, kFwdDrop = 8, kBwdDkDvDrop = 9, kBwdDqDrop = 10, kDecode = 11, kDecodeMerge = 12,
  kNumKernels = 13
};

// Bracket one launch with events on its stream when timing is enabled
// (no-ops otherwise).  Defined in fa_api.cpp.
void timing_begin(int kernel, hipStream_t st);
void timing_end(int kernel, hipStream_t st);

// Launchers return hipGetLastError() after the launch.
// Block-sparse forward (a.mask set).
hipError_t launch_fwd_sparse(Dt dt, int d, bool causal, int bh, FwdArgs a, hipStream_t st);
// Dense forward at two waves per SIMD (no block mask, no dropout).
hipError_t launch_fwd2(Dt dt, int d, bool causal, int bh, FwdArgs a, hipStream_t st);
// Block-sparse forward at two waves per SIMD (d = 64; a.mask set).
hipError_t launch_fwd2_sparse(Dt dt, int d, bool causal, int bh, FwdArgs a, hipStream_t st);
hipError_t launch_fwd_f32(int d, bool causal, bool sparse, int bh, FwdArgs a, hipStream_t st);
// Split-KV forward (a.nsplit key ranges per row, partials in a.po / a.plse)
// followed by the merge into a.o / a.lse.
hipError_t launch_fwd_split(Dt dt, int d, bool causal, int bh, FwdArgs a, hipStream_t st);
hipError_t launch_bwd(Dt dt, int d, bool causal, bool sparse, int bh, BwdArgs a, hipStream_t st);
// Dropout variants (dense or packed layouts, no block mask): a.drop set.
hipError_t launch_fwd_dropout(Dt dt, int d, bool causal, int bh, FwdArgs a, hipStream_t st);
hipError_t launch_bwd_dropout(Dt dt, int d, bool causal, int bh, BwdArgs a, hipStream_t st);
// Decoding against a key/value cache (a.nsplit key ranges, merged when > 1).
hipError_t launch_fwd_decode(Dt dt, int d, bool causal, DecArgs a, hipStream_t st);
// Row tiles (workgroups per K/V head and key range) for groups of
// rows_per_group rows.
int decode_row_tiles(long long rows_per_group);

}  // namespace fa
