/*
 * fa.h -- C ABI of libfa.so: exact tiled attention on AMD MI355X (gfx950).
 *
 * What is computed.  For every batch b, query head h and query row i:
 *
 *     o[b,h,i,:] = sum_j softmax_j( scale * q[b,h,i,:] . k[b,g,j,:] ) * v[b,g,j,:]
 *     lse[b,h,i] = log sum_j exp( scale * q[b,h,i,:] . k[b,g,j,:] )
 *
 * with g = h / (Hq/Hkv) (grouped-query attention: consecutive query heads
 * share one key/value head), and j running over all keys, or over j <= i
 * under the causal mask.  This is softmax(Q K^T) V as written in the forum
 * comment on SRAM and GEMM tiling (item 45450456, paragraph on KV caching),
 * with the scale and mask between score and normalisation as listed in
 * "How Does Flash Attention Reduce Memory Traffic During Local Inference?",
 * section "Kernel Fusion Keeps More of the Attention Chain in One Execution
 * Path", and the GQA head sharing of "Optimizing memory requirements for
 * inference in large language models" (GQA paragraph).  The result is exact
 * up to floating-point rounding ("11.4d FlashAttention", comparison table):
 * it is computed tile by tile with a running softmax ("11.4d FlashAttention",
 * "Online Softmax") so no N x N score matrix is ever written to memory.
 *
 * Conventions shared by every entry point.
 *   - All tensor pointers are DEVICE memory owned by the caller.  The library
 *     reads/writes them asynchronously on `stream` (a hipStream_t; NULL = the
 *     null stream) and keeps no reference after the enqueued work completes.
 *     The caller keeps the buffers alive until then.
 *   - Tensors are dense row-major (C-contiguous) with the layouts given per
 *     call; bf16 tensors are passed as raw 16-bit storage (bfloat16).
 *     bf16 and fp32 tensor pointers must be 16-byte aligned; lse and seqlens
 *     4-byte aligned.
 *   - No call synchronises the host.  Faults inside a kernel surface at the
 *     caller's next synchronisation on `stream`.
 *   - Status codes (fa_status) are returned, never thrown.  All argument
 *     checks run on the host before any HIP call, so invalid arguments never
 *     touch the device.
 *   - Head dimension d must be 64 or 128 (FA_ERR_UNSUPPORTED otherwise), and
 *     the current device must be gfx950 (FA_ERR_UNSUPPORTED otherwise).  There
 *     is no silent fallback: the caller decides what to do.
 *   - Calls are thread-safe; the library holds no mutable global state other
 *     than a per-device architecture cache.
 *   - scale: any finite fp32 value whose softmax coefficient |scale|*log2(e)
 *     is finite in fp32 (|scale| below about 2.3e38; larger values return
 *     FA_ERR_INVALID_ARG).  The kernels form scale * (q . k) in fp32, so every
 *     scaled score of a visible (query, key) pair must also be finite in fp32;
 *     if one overflows, the outputs of that row are unspecified (NaN in
 *     practice).  Non-finite input values likewise give unspecified results.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, size <= 0, Hq % Hkv != 0, scale not
                             finite or |scale|*log2(e) not finite in fp32,
                             misaligned pointer, too-small workspace, a grid
                             of 2^31 or more workgroups (prefill: B*Hq*
                             ceil(N/128) for bf16, ceil(N/16) for fp32) */
  FA_ERR_UNSUPPORTED = 2, /* d not in {64,128}, or device is not gfx950 */
  FA_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
  FA_ERR_NO_MEMORY = 4,   /* stream-ordered workspace allocation failed */
  FA_ERR_TOO_LARGE = 5    /* fa_decode_noalloc: the sizes need more than its
                             fixed FA_DECODE_NOALLOC_SCRATCH_BYTES */
} fa_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* fa_strerror(int status);

/*
 * Prefill (bf16 in/out, fp32 accumulation and lse).
 *   q   [B, Hq,  N, d]  bf16      k, v [B, Hkv, N, d]  bf16
 *   o   [B, Hq,  N, d]  bf16 (written)
 *   lse [B, Hq,  N]     fp32 (written; may be NULL to skip)
 *   causal: 0 = every query sees every key; 1 = query i sees keys 0..i.
 *   scale: multiplies q.k before the mask and softmax (finite; any sign).
 * Work: one kernel launch on `stream`.
 */
int fa_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               void* stream);

/* Prefill with fp32 q/k/v/o (same layouts and semantics).  Scores, running max
 * and sums are formed in fp64 and the exponentials in fp32, so the result stays
 * within about 1e-6 of the exact one also for long rows and sharp softmaxes.
 * Work: one kernel launch on `stream` (16 query rows per workgroup, the keys
 * split over its waves and merged at the end). */
int fa_prefill_f32(const float* q, const float* k, const float* v, float* o,
                   float* lse, int B, int Hq, int Hkv, int N, int d, int causal,
                   float scale, void* stream);

/*
 * Packed variable-length prefill: chunked prefill against a cached prefix,
 * batches of prompts of different lengths, and a sliding (left) window.
 * Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key /
 * value rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1.  Its n_q queries are the
 * LAST n_q positions of its n_k keys: with off = n_k - n_q, causal row i sees
 * keys j <= i + off (bottom-right alignment, so a chunk of new tokens sees the
 * cached prefix and itself), and window_left = W >= 0 also drops keys
 * j < i + off - W (-1: no window).  Each row is the same exact softmax(scale
 * q k^T) v as fa_prefill over the keys it sees.  The retained cache a chunk
 * attends to, and windowing as one way a runtime limits it, follow "How Does
 * Flash Attention Reduce Memory Traffic During Local Inference?", section
 * "Reduced IO Is Not the Same as Eliminating KV Cache"; masking, its section
 * "Kernel Fusion Keeps More of the Attention Chain in One Execution Path".
 *   q, o          [total_q, Hq, d]   bf16 (token-major packed rows)
 *   k, v          [total_k, Hkv, d]  bf16
 *   lse           [Hq, total_q]      fp32, may be NULL
 *   cu_seqlens_q  [B+1]              int32, device memory, non-decreasing,
 *   cu_seqlens_k  [B+1]              int32  from 0 to total_q / total_k (values
 *                                    outside [0, total] are clamped on the
 *                                    device: never an out-of-bounds access)
 *   max_seqlen_q  >= every n_q (sizes the grid; rows of a longer sequence
 *                 beyond it are not computed)
 * A row that sees no key (causal with i + off < 0) gets o = 0, lse = -inf.
 * Tiles outside every row's [i + off - W, i + off] range are never loaded.
 * bf16 only; d in {64, 128}.  Work: one kernel launch on `stream`.
 */
int fa_prefill_varlen(const void* q, const void* k, const void* v, void* o,
                      float* lse, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, int B, int Hq, int Hkv,
                      int total_q, int total_k, int max_seqlen_q, int d,
                      int causal, int window_left, float scale, void* stream);

/*
 * Backward of fa_prefill (bf16): gradients of sum(o * dout) with respect to
 * q, k and v.  The attention probabilities are recomputed from q, k and the
 * forward's log-sum-exp rather than stored ("11.4d FlashAttention", section
 * "Recomputation"; its trade-offs section notes the extra FLOPs this costs).
 * With p = exp(scale q.k - lse) over the visible keys of each row:
 *     dv = p^T dout,  dp = dout v^T,  ds = p (dp - rowsum(dout * o)),
 *     dq = scale ds k,  dk = scale ds^T q
 * and, under GQA, a key/value head's dk, dv summed over its query heads.
 *   q, o, dout, dq  [B, Hq, N, d]   bf16 (dq written)
 *   k, v, dk, dv    [B, Hkv, N, d]  bf16 (dk, dv written)
 *   lse             [B, Hq, N]      fp32: the lse fa_prefill returned for the
 *                                   same q, k, v, causal and scale
 * causal and scale as passed to fa_prefill; d in {64, 128}.  workspace may
 * be NULL (obtained stream-ordered) or hold at least
 * fa_prefill_backward_workspace_bytes(B, Hq, N) bytes, 256-byte aligned.
 * Every output element is written by exactly one workgroup (no atomics), so
 * the results are deterministic.  Work: two kernel launches on `stream` (dQ
 * with the rows' rowsum(dout * o) terms, then dK/dV).
 */
int fa_prefill_backward(const void* q, const void* k, const void* v,
                        const void* o, const void* dout, const float* lse,
                        void* dq, void* dk, void* dv, int B, int Hq, int Hkv,
                        int N, int d, int causal, float scale, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Workspace bytes fa_prefill_backward needs (0 if the sizes are invalid). */
size_t fa_prefill_backward_workspace_bytes(int B, int Hq, int N);

/*
 * Decode: one new query token per sequence against its KV cache.  The cache
 * grows with the context and is retained by the caller between steps; this
 * call only reads it ("How Does Flash Attention Reduce Memory Traffic ...",
 * section "Reduced IO Is Not the Same as Eliminating KV Cache").  Each step
 * re-reads the whole cache of each sequence including the newest entry
 * (forum comment item 45450456, paragraph on KV caching).
 *   q       [B, Hq, d]              bf16
 *   kcache  [B, Hkv, maxlen, d]     bf16 (one contiguous maxlen x d slab per
 *   vcache  [B, Hkv, maxlen, d]     bf16  sequence and key/value head)
 *   seqlens [B]                     int32, device memory; sequence b attends
 *                                   to cache rows 0 .. seqlens[b]-1, which
 *                                   already include the new token.  Rows at or
 *                                   past seqlens[b] are never read.  Values
 *                                   are clamped to [0, maxlen] on the device;
 *                                   seqlens[b] == 0 gives o = 0.
 *   o       [B, Hq, d]              bf16 (written)
 * The key range is split into chunks whose partial results are merged by
 * their log-sum-exp weights.  fa_decode obtains that workspace stream-ordered
 * (hipMallocAsync / hipFreeAsync on `stream`); fa_decode_ws takes it from
 * the caller instead (at least fa_decode_workspace_bytes(...) bytes, 256-byte
 * aligned, device memory, not used concurrently by another call).
 * Work: two kernel launches on `stream`; the host never reads seqlens.
 */
int fa_decode(const void* q, const void* kcache, const void* vcache,
              const int32_t* seqlens, void* o, int B, int Hq, int Hkv,
              int maxlen, int d, float scale, void* stream);

int fa_decode_ws(const void* q, const void* kcache, const void* vcache,
                 const int32_t* seqlens, void* o, int B, int Hq, int Hkv,
                 int maxlen, int d, float scale, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Decode with fp32 q/caches/o (same layouts and semantics).  Scores, chunk
 * maxima, sums and P.V accumulate in fp64 over fp32 inputs; probabilities,
 * the chunks' partial outputs and the output are fp32, their log-sum-exps
 * fp64 (so the merge weights stay exact when |lse| is large): within about
 * 1e-5 of the exact result for unit-scale caches. */
int fa_decode_f32(const float* q, const float* kcache, const float* vcache,
                  const int32_t* seqlens, float* o, int B, int Hq, int Hkv,
                  int maxlen, int d, float scale, void* stream);

int fa_decode_f32_ws(const float* q, const float* kcache, const float* vcache,
                     const int32_t* seqlens, float* o, int B, int Hq, int Hkv,
                     int maxlen, int d, float scale, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Workspace bytes fa_decode_ws / fa_decode_f32_ws need for these sizes
 * (0 if the sizes are invalid). */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int maxlen, int d);

/*
 * fa_decode (bf16) for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, layouts, semantics and kernels as fa_decode,
 * and bit-identical results; the split-KV partials go to a fixed device array
 * of FA_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends.  The call allocates nothing (no hipMalloc,
 * hipMallocAsync or hipFree) and enqueues exactly the two kernels of
 * fa_decode_ws.
 *   Limit: the partials take (B*Hq*S*d*4 and B*Hq*S*4 bytes, each rounded up
 *   to 256) for the S key chunks the launcher picks; sizes beyond the array
 *   return FA_ERR_TOO_LARGE before any HIP call.  It always fits when
 *   fa_decode_workspace_bytes(B, Hq, Hkv, maxlen, d) <=
 *   FA_DECODE_NOALLOC_SCRATCH_BYTES (e.g. B 64, Hq 32, Hkv 8, maxlen 32768,
 *   d 128 uses 8.5 MB).
 *   Sharing: every call on one GPU uses that GPU's single array.  Calls on
 *   the same stream are ordered and safe; calls that can overlap on one GPU
 *   (other streams, other host threads) race on it and must be serialised by
 *   the caller.  Nothing in the array needs clearing between calls.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fa_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                      const int32_t* seqlens, void* o, int B, int Hq, int Hkv,
                      int maxlen, int d, float scale, void* stream);

/*
 * Decode against a paged KV cache.  The retained history stays available to
 * later tokens unless the runtime evicts, compresses, windows or offloads it
 * ("How Does Flash Attention Reduce Memory Traffic During Local Inference?",
 * section "Reduced IO Is Not the Same as Eliminating KV Cache"); a paged
 * cache is the storage such a runtime manages: fixed-size pages from one
 * pool, mapped to each sequence by a block table, so pages can be freed,
 * moved or shared without copying a sequence's whole history.  The attention
 * computed is exactly fa_decode's over the logical cache the table describes.
 *   q           [B, Hq, d]                        bf16
 *   kpages      [num_pages, Hkv, page_size, d]    bf16 page pool (page p holds
 *   vpages      [num_pages, Hkv, page_size, d]    bf16  page_size consecutive
 *                                                 cache entries of every KV head)
 *   block_table [B, max_pages]                    int32, device memory: entry
 *               i of row b is the pool page holding cache entries
 *               i*page_size .. (i+1)*page_size - 1 of sequence b.  Entries
 *               past the sequence's last page are never read; several rows
 *               may name the same page (shared prefixes).  Ids outside
 *               [0, num_pages) are a caller error and are clamped into the
 *               pool on the device (never an out-of-bounds read).
 *   seqlens     [B]                               int32, device memory, clamped
 *               to [0, max_pages * page_size]; 0 gives o = 0.
 *   o           [B, Hq, d]                        bf16 (written)
 * page_size must be a power of two in [16, 2^20]; max_pages * page_size must
 * fit in an int.  workspace may be NULL (then it is obtained stream-ordered,
 * as in fa_decode) or hold at least fa_decode_paged_workspace_bytes(...)
 * bytes, 256-byte aligned.  Work: two kernel launches on `stream`.
 */
int fa_decode_paged(const void* q, const void* kpages, const void* vpages,
                    const int32_t* block_table, const int32_t* seqlens, void* o,
                    int B, int Hq, int Hkv, int num_pages, int page_size,
                    int max_pages, int d, float scale, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace bytes fa_decode_paged needs (0 if the sizes are invalid). */
size_t fa_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int page_size,
                                       int max_pages, int d);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
