/*
 * flash_attn.h -- C ABI of the gfx950 exact-attention library (libflashattn.so)
 *
 * Exact softmax attention for one MI355X GPU:
 *     S = scale * Q K^T,  P = softmax_row(S),  O = P V,  LSE_i = ln sum_j exp(S_ij)
 * computed in one fused pass whose online-softmax statistics keep S and P
 * off HBM, with a backward pass that recomputes them from Q, K, V and LSE.
 *
 * Sources the operations follow (titles of the pages, with the section,
 * equation or algorithm):
 *   [FA2]  FlashAttention-2 reading notes (zhongzhuzhou.org): Algorithm 1
 *          (forward), Algorithm 2 (backward), eqs. (5)-(7) online softmax,
 *          eqs. (10)-(16) deferred normalisation and log-sum-exp, eq. (17)
 *          and eqs. (27)-(30) softmax Jacobian, "Causal mask optimisation",
 *          "MQA and GQA support", "Reproducibility notes" (FLOP convention).
 *   [FA1]  FlashAttention paper summary (zhaifeiyue.github.io/papers/
 *          2205.14135): Technique 1 (tiling), Technique 2 (recomputation,
 *          D_i = do_i . o_i), Block-Sparse FlashAttention.
 *   [WALK] FlashAttention walkthrough (bluuewhale.github.io/posts/
 *          flash-attention-en): "How Attention Is Computed" (scaled scores),
 *          "Block-Sparse FlashAttention" (mask M in {0,1}^{Tr x Tc}).
 *   [V1]   Flash Attention v1 notes (languisher.top/posts/flash-attention):
 *          merging the softmax statistics of two vectors (max, normaliser,
 *          rescaled numerators).
 *
 * Common conventions
 * ------------------
 * Layout.  Every per-token tensor (q, k, v, o, dout, dq, dk, dv) is a dense,
 *   contiguous [B][H][N][d] array of `dtype` elements (d innermost).  LSE is
 *   a dense [B][H][N] float32 array.  Queries and keys share one length N.
 * Pointers.  All tensor, mask and workspace pointers are DEVICE pointers,
 *   owned by the caller, 16-byte aligned, and must stay valid until the
 *   stream reaches the enqueued work.  The library never allocates or frees
 *   device memory and keeps no caller pointer after a call returns; the
 *   only device memory it holds is the static scratch array of
 *   flash_attn_bwd_noalloc (32 MiB per GPU, part of the loaded code object).
 * Streams.  Every call enqueues its kernels on `stream` (0 = null stream)
 *   and returns without synchronising.
 * Domain.  d in {64, 128}; N >= 0 (any value, no tile-multiple needed);
 *   B*H*ceil(N/32) < 2^31; scale finite and > 0; causal in {0, 1}
 *   (causal keeps key j for query i iff j <= i).  FA_F32 is accepted by the
 *   forward calls only; FA_F16 and FA_BF16 by all calls.  Arithmetic is
 *   float32 throughout (scores, statistics, accumulators); for 16-bit inputs
 *   the probabilities are rounded to the input type only as an operand of
 *   the P V product (and P, dS of the backward products).
 * Empty problems.  B*H*N == 0 returns FA_OK and launches nothing.
 * Rows with no allowed key (possible only with a block mask whose diagonal
 *   entry is 0) give O = 0, LSE = -inf and zero gradient contributions.
 * Errors.  Status codes only, never an abort.  All argument checks finish
 *   before any HIP call, so an invalid call has no effect on the device.  A
 *   failed kernel launch returns FA_ERR_HIP.  flash_attn_last_error() gives
 *   a thread-local description of the last non-OK status on the calling
 *   thread.  Faults inside kernels surface later, at the caller's
 *   synchronisation, as HIP errors.
 */
#ifndef FLASH_ATTN_H
#define FLASH_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, negative size, bad scale/flag */
  FA_ERR_UNSUPPORTED = 2,        /* valid but outside the supported domain (d, dtype, mask block) */
  FA_ERR_WORKSPACE_TOO_SMALL = 3,/* workspace smaller than the matching *_workspace_size() */
  FA_ERR_HIP = 4                 /* a HIP launch failed; see flash_attn_last_error() */
} fa_status;

typedef enum fa_dtype { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

/* Version of this ABI (incremented on any signature or semantic change). */
int flash_attn_abi_version(void);

/*
 * Forward pass [FA2 Algorithm 1; FA2 eqs. (10)-(15)].
 *   q, k, v  in   [B][H][N][d] dtype
 *   o        out  [B][H][N][d] dtype     O = softmax(scale Q K^T (masked)) V
 *   lse      out  [B][H][N]    float32   natural-log log-sum-exp of each row
 *                                         of scale Q K^T over allowed keys
 * causal = 1 masks keys after the query [FA2 "Causal mask optimisation"].
 */
fa_status flash_attn_fwd(int B, int H, int N, int d, fa_dtype dtype,
                         const void* q, const void* k, const void* v,
                         float scale, int causal,
                         void* o, float* lse, hipStream_t stream);

/*
 * Split-KV forward [V1 merging of softmax statistics, applied to num_splits
 * parts]: the result of flash_attn_fwd (same arguments and outputs, up to
 * float32 rounding order), computed by cutting every row block's key tiles
 * into num_splits contiguous ranges processed by separate workgroups, then
 * merging.  Meant for problems with too few query blocks to fill the GPU
 * (small B*H or short N).  Range s of row i yields its own output O_s
 * (normalised by its own sum) and log-sum-exp L_s (-inf if the range has no
 * allowed key); the merge writes LSE_i = ln sum_s e^{L_s} and
 * O_i = sum_s e^{L_s - LSE_i} O_s.
 *   num_splits  1 .. 64 (FA_ERR_INVALID_ARGUMENT outside).
 *   workspace   scratch, >= flash_attn_fwd_splitkv_workspace_size() bytes:
 *               num_splits float32 partial outputs [B][H][N][d] followed by
 *               num_splits float32 partial log-sum-exps [B][H][N].
 *               Contents on entry are ignored and left undefined.
 * dtype FA_F16 or FA_BF16 (FA_F32: FA_ERR_UNSUPPORTED).
 */
size_t flash_attn_fwd_splitkv_workspace_size(int B, int H, int N, int d, fa_dtype dtype,
                                             int num_splits);
/* A num_splits for flash_attn_fwd_splitkv: enough key ranges for about two
 * workgroups per compute unit (512 in all), at least eight 32-key tiles per
 * range, at most 64; 1 when the plain forward already fills the GPU.
 * Depends on the shape only; never fails (1 for empty shapes). */
int flash_attn_fwd_splitkv_num_splits(int B, int H, int N, int d, int causal);
fa_status flash_attn_fwd_splitkv(int B, int H, int N, int d, fa_dtype dtype,
                                 const void* q, const void* k, const void* v,
                                 float scale, int causal, int num_splits,
                                 void* o, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Device workspace bytes flash_attn_bwd / flash_attn_blocksparse_bwd need:
 * two float32 per query row (D_i = rowsum(dO o O) and the log-sum-exp in
 * base 2), each array rounded up to 256 bytes plus 256 spare bytes.
 * Returns 0 for empty problems; never fails.
 */
size_t flash_attn_bwd_workspace_size(int B, int H, int N, int d, fa_dtype dtype);

/*
 * Backward pass [FA2 Algorithm 2; FA2 eqs. (16), (17), (27)-(30);
 * FA1 Technique 2].
 *   q, k, v, o, dout  in   [B][H][N][d] dtype   (o, lse: the forward's outputs)
 *   lse               in   [B][H][N] float32
 *   dq, dk, dv        out  [B][H][N][d] dtype   gradients of sum(O o dout)
 *   workspace         scratch, >= flash_attn_bwd_workspace_size() bytes;
 *                     contents on entry are ignored and left undefined.
 * scale and causal must equal the forward's.  dtype FA_F32 is unsupported.
 */
fa_status flash_attn_bwd(int B, int H, int N, int d, fa_dtype dtype,
                         const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         float scale, int causal,
                         void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward pass without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * must not call hipMalloc, harnesses that forbid it).  Same arguments,
 * layouts, result and errors as flash_attn_bwd minus the workspace, which
 * here is a buffer the library holds: one static device array of 32 MiB per
 * GPU, held by each GPU the library runs on until the process ends, enough
 * for B*H*N up to about 4.1 million query rows.  Larger problems return
 * FA_ERR_UNSUPPORTED (use flash_attn_bwd).  The call allocates nothing; on
 * its first use on a device it looks up that device's copy of the array
 * (hipGetSymbolAddress).  `stream` (if not 0) must belong to the current
 * device (FA_ERR_INVALID_ARGUMENT otherwise).  All calls on one GPU share
 * the array: calls that overlap on one GPU (different streams, no ordering
 * between them) race and give undefined results.
 */
fa_status flash_attn_bwd_noalloc(int B, int H, int N, int d, fa_dtype dtype,
                                 const void* q, const void* k, const void* v,
                                 const void* o, const void* dout, const float* lse,
                                 float scale, int causal,
                                 void* dq, void* dk, void* dv, hipStream_t stream);

/*
 * Block-sparse forward [FA1 "Block-Sparse FlashAttention"; WALK
 * "Block-Sparse FlashAttention"]: as flash_attn_fwd, but key j is visible to
 * query i only if block_mask[i / mask_block][j / mask_block] != 0, and tiles
 * of zero mask blocks are skipped without being loaded.
 *   block_mask  in  device uint8 [T][T], T = ceil(N / mask_block), row-major,
 *               shared by every (batch, head); nonzero = keep.
 *   mask_block  tokens per mask entry; must be 128 (FA_ERR_UNSUPPORTED else).
 * N is limited to 128 * 2048 = 262144 tokens (T <= 2048; FA_ERR_UNSUPPORTED
 * beyond): the kernels keep tables of one row or column of the mask on chip.
 * causal may be combined with the mask (both must allow a key).
 */
fa_status flash_attn_blocksparse_fwd(int B, int H, int N, int d, fa_dtype dtype,
                                     const void* q, const void* k, const void* v,
                                     float scale, int causal,
                                     const uint8_t* block_mask, int mask_block,
                                     void* o, float* lse, hipStream_t stream);

/*
 * Block-sparse backward: the exact gradient of the masked attention above
 * (the pages give the sparse forward only; this is the gradient of the same
 * function), skipping the same zero tiles.  Arguments as flash_attn_bwd plus
 * the mask as in flash_attn_blocksparse_fwd.
 */
fa_status flash_attn_blocksparse_bwd(int B, int H, int N, int d, fa_dtype dtype,
                                     const void* q, const void* k, const void* v,
                                     const void* o, const void* dout, const float* lse,
                                     float scale, int causal,
                                     const uint8_t* block_mask, int mask_block,
                                     void* dq, void* dk, void* dv,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * Grouped K/V heads [FA2 "MQA and GQA support"]: flash_attn_fwd and
 * flash_attn_bwd with Hkv K/V heads shared by H query heads (Hkv = 1 is
 * multi-query attention, Hkv = H the plain calls).  H must be a multiple of
 * Hkv (H = 0 requires Hkv = 0; FA_ERR_INVALID_ARGUMENT otherwise).  Query
 * head i of a batch reads K/V head floor(i / (H / Hkv)): each run of H / Hkv
 * consecutive query heads forms one group, whose K/V head the kernels index
 * in place (K and V are never copied or broadcast).
 *   q, o, dout, dq   [B][H][N][d]   dtype
 *   lse              [B][H][N]      float32
 *   k, v, dk, dv     [B][Hkv][N][d] dtype
 * dK and dV of a K/V head are sums over the query heads of its group; the
 * dK/dV pass forms them by sweeping the group's heads into the same
 * accumulators.  When B*Hkv*ceil(N/128) is too small to fill the GPU, each
 * group is cut into up to H/Hkv ranges of heads swept by separate
 * workgroups, whose float32 partial sums a reduction pass adds up (fixed
 * order, so results are deterministic).  The backward workspace is
 * flash_attn_bwd_gqa_workspace_size() bytes: the flash_attn_bwd workspace
 * of the H query heads followed, when ranges are used, by the float32
 * partial dK and dV; it depends on the shape only and returns 0 for
 * empty or invalid shapes.  Other arguments, dtypes and errors as
 * flash_attn_fwd and flash_attn_bwd.
 */
fa_status flash_attn_fwd_gqa(int B, int H, int Hkv, int N, int d, fa_dtype dtype,
                             const void* q, const void* k, const void* v,
                             float scale, int causal,
                             void* o, float* lse, hipStream_t stream);
size_t flash_attn_bwd_gqa_workspace_size(int B, int H, int Hkv, int N, int d, fa_dtype dtype);
fa_status flash_attn_bwd_gqa(int B, int H, int Hkv, int N, int d, fa_dtype dtype,
                             const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse,
                             float scale, int causal,
                             void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Variable-length batches: B sequences of different lengths packed along
 * one token axis, each attended on its own (the per-head problem of
 * [FA2 Algorithm 1, Algorithm 2] for every sequence; grouped K/V heads as
 * in flash_attn_fwd_gqa).  Sequence b holds rows cu_seqlens[b] ..
 * cu_seqlens[b+1]-1; no attention crosses sequences, and the causal rule
 * (key j visible to query i iff j <= i) counts positions from the start
 * of each sequence.
 *   cu_seqlens      in  device int32 [B+1], 4-byte aligned: 0 = cu[0] <=
 *                       cu[1] <= ... <= cu[B] = total, every length <=
 *                       max_seqlen.  Not read on the host; the kernels
 *                       clamp each sequence into [0, total] and to
 *                       max_seqlen rows, so inconsistent offsets give
 *                       unspecified results but no access outside the
 *                       tensors.
 *   q, o, dout, dq  [total][H][d]   dtype (token-major: row stride H*d)
 *   k, v, dk, dv    [total][Hkv][d] dtype
 *   lse             [H][total]      float32
 * A batch of B sequences of equal length N in the [B][N][H][d] layout is
 * the packed batch with cu_seqlens = 0, N, 2N, ..., BN.  Domain as the
 * dense calls with N = max_seqlen, plus H*d < 2^23 (FA_ERR_UNSUPPORTED
 * otherwise); FA_F32 in the forward only.  Work is launched for
 * max_seqlen rows per sequence; shorter sequences leave workgroups idle.
 * The backward workspace is flash_attn_varlen_bwd_workspace_size() bytes
 * (the per-row arrays of H*total rows, then the grouped-head partial sums
 * when used); it returns 0 for empty or invalid shapes.
 */
fa_status flash_attn_varlen_fwd(int B, int H, int Hkv, int total, int max_seqlen, int d,
                                fa_dtype dtype, const int* cu_seqlens,
                                const void* q, const void* k, const void* v,
                                float scale, int causal,
                                void* o, float* lse, hipStream_t stream);
size_t flash_attn_varlen_bwd_workspace_size(int B, int H, int Hkv, int total, int max_seqlen, int d,
                                            fa_dtype dtype);
fa_status flash_attn_varlen_bwd(int B, int H, int Hkv, int total, int max_seqlen, int d,
                                fa_dtype dtype, const int* cu_seqlens,
                                const void* q, const void* k, const void* v,
                                const void* o, const void* dout, const float* lse,
                                float scale, int causal,
                                void* dq, void* dk, void* dv,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Dropout on the attention probabilities, fused into the passes [FA1
 * summary: matmul, softmax, dropout and mask fused into one kernel]:
 *   O = (P o Z) V / (1 - p'),  LSE as without dropout,
 * with Z in {0, 1} drawn, never stored, from the counter-based generator
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011): element (query i,
 * key j) of head h of batch b is kept iff byte j % 4 of word i % 4 of
 *   Philox4x32-10(counter = (i / 4, j / 4, b*H + h, offset),
 *                 key = (seed & 0xffffffff, seed >> 32))
 * is at least t = floor(256 dropout_p + 0.5), and p' = t / 256 (the drop
 * probability is quantised to 1/256).  The backward recomputes the same Z
 * from (seed, offset) and returns the exact gradient of that O:
 * dV = (P o Z)^T dO / (1 - p'), dS = P o (dP' o Z / (1 - p') - D) with
 * dP' = dO V^T and D = rowsum(dO o O).  dropout_p in [0, 1) with t <= 255
 * (FA_ERR_INVALID_ARGUMENT otherwise); dtype FA_F16 or FA_BF16.  Other
 * arguments, layouts and errors as flash_attn_fwd / flash_attn_bwd (same
 * workspace); seed, offset and dropout_p must equal the forward's.
 */
fa_status flash_attn_fwd_dropout(int B, int H, int N, int d, fa_dtype dtype,
                                 const void* q, const void* k, const void* v,
                                 float scale, int causal,
                                 float dropout_p, uint64_t seed, uint32_t offset,
                                 void* o, float* lse, hipStream_t stream);
fa_status flash_attn_bwd_dropout(int B, int H, int N, int d, fa_dtype dtype,
                                 const void* q, const void* k, const void* v,
                                 const void* o, const void* dout, const float* lse,
                                 float scale, int causal,
                                 float dropout_p, uint64_t seed, uint32_t offset,
                                 void* dq, void* dk, void* dv,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Dropout on packed variable-length batches (with grouped K/V heads): the
 * dropout above applied to flash_attn_varlen_fwd / flash_attn_varlen_bwd.
 * Positions i, j in the counter count from the start of each sequence and
 * the head index is b*H + h with b the sequence.  Arguments as the varlen
 * calls plus dropout_p, seed and offset; the same backward workspace.
 */
fa_status flash_attn_varlen_fwd_dropout(int B, int H, int Hkv, int total, int max_seqlen, int d,
                                        fa_dtype dtype, const int* cu_seqlens,
                                        const void* q, const void* k, const void* v,
                                        float scale, int causal,
                                        float dropout_p, uint64_t seed, uint32_t offset,
                                        void* o, float* lse, hipStream_t stream);
fa_status flash_attn_varlen_bwd_dropout(int B, int H, int Hkv, int total, int max_seqlen, int d,
                                        fa_dtype dtype, const int* cu_seqlens,
                                        const void* q, const void* k, const void* v,
                                        const void* o, const void* dout, const float* lse,
                                        float scale, int causal,
                                        float dropout_p, uint64_t seed, uint32_t offset,
                                        void* dq, void* dk, void* dv,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decoding against a key/value cache [FA2 "impact on the KV cache": a
 * decoding step attends a few new queries per head to every cached key and
 * value of the sequence; grouped K/V heads as in "MQA and GQA support"]:
 * exact attention of Nq queries per query head against the first L_b of the
 * Nk cache slots of sequence b,
 *   q      in   [B][H][Nq][d]  dtype
 *   k, v   in   [B][Hkv][Nk][d] dtype   (the cache; slots >= L_b are never read)
 *   cache_seqlens in  device int32 [B]: L_b (clamped to [0, Nk]), or NULL
 *          for L_b = Nk; 4-byte aligned
 *   o      out  [B][H][Nq][d]  dtype
 *   lse    out  [B][H][Nq]     float32
 * Query head h reads K/V head floor(h / (H / Hkv)).  Causal rule: the Nq
 * queries are the last Nq positions of the sequence, so query i sees key j
 * iff j <= i + L_b - Nq (the last query sees all L_b keys; with L_b < Nq
 * the first queries see none and give O = 0, LSE = -inf, as do all rows
 * when L_b = 0).  The cache is read once per K/V head: the H/Hkv query
 * heads of a group and their Nq queries are processed together, and the
 * key range is cut into num_splits parts (1..64) whose partial results a
 * merge pass combines as in flash_attn_fwd_splitkv.  Bound by HBM
 * bandwidth (the cache is read once); meant for Nq much smaller than Nk.
 *   workspace  >= flash_attn_fwd_kvcache_workspace_size() bytes (0 when
 *          num_splits = 1, then workspace may be NULL): num_splits float32
 *          partial outputs [B*H*Nq][d] then partial log-sum-exps [B*H*Nq].
 * flash_attn_fwd_kvcache_num_splits gives a split count for the shape
 * (about four single-wave workgroups per compute unit, at least four
 * 32-key tiles per split).  dtype FA_F16 or FA_BF16; other conventions and
 * errors as flash_attn_fwd.
 */
size_t flash_attn_fwd_kvcache_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d, fa_dtype dtype,
                                             int num_splits);
int flash_attn_fwd_kvcache_num_splits(int B, int H, int Hkv, int Nq, int Nk, int d);
fa_status flash_attn_fwd_kvcache(int B, int H, int Hkv, int Nq, int Nk, int d, fa_dtype dtype,
                                 const void* q, const void* k, const void* v, const int* cache_seqlens,
                                 float scale, int causal, int num_splits,
                                 void* o, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Per-kernel timing (diagnostics; not part of the method).  While enabled,
 * every kernel the library launches is bracketed by two HIP events recorded
 * on its launch stream.  flash_attn_timing_collect waits for the recorded
 * events, writes for each kernel class k < n the summed milliseconds and
 * launch count since the previous collect, and forgets them.  Kernel
 * classes: 0 forward (16-bit), 1 forward (float32), 2 backward D pre-pass,
 * 3 backward dK/dV pass, 4 backward dQ pass, 5 split-KV forward ranges,
 * 6 split-KV merge, 7 dK/dV range sum (grouped heads), 8 forward with
 * dropout, 9 dK/dV pass with dropout, 10 dQ pass with dropout, 11 KV-cache
 * decoding, 12 its merge pass; flash_attn_kernel_name(k) names them.
 * Events are created on first use and reused; no device memory is
 * allocated.  Process-wide, guarded by a mutex.
 */
fa_status flash_attn_timing_enable(int enable);
fa_status flash_attn_timing_collect(double* total_ms, int* launches, int n);
const char* flash_attn_kernel_name(int kernel);

/* Static name of a status code ("FA_OK", ...). */
const char* flash_attn_status_string(fa_status status);

/* Thread-local detail of the last non-OK status returned on this thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char* flash_attn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FLASH_ATTN_H */
