/*
 * prefill_attn.h -- C ABI of the MI355X (gfx950) prefill-attention library.
 *
 * One call computes causal scaled-dot-product self-attention over a batch of
 * variable-length prompts flattened into one token stream and, in the same
 * launch, writes every new token's K and V into a head-major KV cache.
 *
 * Sources (the pages that define the operation):
 *   [P1] "Prefill不是热身：大模型推理的真正瓶颈与优化核心" (www.mhpn.cn/news/2373630)
 *   [P2] "大模型推理优化：Prefill、Decode与KV Cache的工程实践" (www.zskr.cn/news/2334369)
 *   [P3] "大模型 Prompt Prefill 阶段的高效 Batching 与算子排布" (www.nxmr.cn/news/92962)
 *   [P4] "大语言模型推理核心：Prefill与Decode原理及工程优化" (www.yfxerp.com/news/184489)
 *   [P5] untitled page at www.zwxr.cn/news/300951
 *
 * Common conventions
 *   - bf16 tensors are passed as raw 16-bit patterns (uint16_t).
 *   - q, k, v, out: [N, H, D] contiguous, token-major, N = cu_seqlens[B].  The
 *     flattened [total_tokens, hidden] stream with hidden = H * D [P3 §2].
 *   - cu_seqlens: int32 [B + 1] in DEVICE memory, cu[0] = 0, non-decreasing;
 *     sequence b owns tokens cu[b] .. cu[b+1]-1 [P3 figure and §2].
 *   - Attention of sequence b, head h, query i (absolute position p_b + i,
 *     p_b = 0 for varlen):  out = sum_{j <= p_b + i} softmax_j(scale q.k_j) v_j
 *     over keys of sequence b only [P1 §3 and P4 §2.2 formula; P5 §1.1 causal
 *     visibility; P3 §2 no attention across requests].
 *   - head_dim D in {32, 64, 128}.  scale: any finite float (0 allowed); the
 *     usual value is 1/sqrt(D).  Scores |scale * q.k| up to 2^26 are supported
 *     (attention logits are many orders of magnitude smaller); beyond that the
 *     softmax weights may overflow.
 *   - All pointers are caller-owned device memory aligned to 16 bytes.  The
 *     library keeps no pointer after returning, allocates no memory, creates
 *     no stream and never synchronises the device (except in check mode,
 *     below).  Work is enqueued on `stream` (NULL = default stream); inputs
 *     must stay valid until it completes.  Calls are re-entrant.
 *   - Outputs (out, k_cache, v_cache) must not overlap q, k, v, cu_seqlens,
 *     prefix_lens or each other.
 *   - Errors detectable on the host are reported before anything is enqueued
 *     and leave every buffer untouched.  B == 0 or max_seqlen == 0 enqueues
 *     nothing and returns PA_OK.  Device faults surface at the caller's next
 *     synchronisation, as for any HIP launch.
 *   - Device-resident metadata (cu_seqlens, prefix_lens) is trusted in the
 *     default mode: a violated precondition (non-monotonic cu_seqlens, a
 *     length above max_seqlen, prefix + length above the cache capacity) is
 *     undefined behaviour.  In check mode (pa_set_check_mode(1) or the
 *     environment variable PA_CHECK=1 at load time) the library copies the
 *     metadata to the host on `stream`, waits for it, and returns
 *     PA_ERR_SEQLENS / PA_ERR_CAPACITY instead of launching.
 */
#ifndef PREFILL_ATTN_H
#define PREFILL_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL = 1,      /* a required pointer is NULL */
    PA_ERR_SHAPE = 2,     /* num_seqs < 0, num_heads < 1, max_seqlen < 0, cache_capacity < 1, num_kv_heads < 1 or not dividing num_heads, or a grid limit exceeded */
    PA_ERR_HEAD_DIM = 3,  /* head_dim not in {32, 64, 128} */
    PA_ERR_SCALE = 4,     /* scale is NaN or infinite */
    PA_ERR_ALIGN = 5,     /* a tensor pointer is not 16-byte aligned */
    PA_ERR_ALIAS = 6,     /* an output pointer equals an input or another output pointer */
    PA_ERR_SEQLENS = 7,   /* check mode: cu_seqlens[0] != 0, decreasing, or a length > max_seqlen */
    PA_ERR_CAPACITY = 8,  /* check mode: a prefix length < 0, prefix + length > cache_capacity, or a block id outside the pool */
    PA_ERR_HIP = 9,       /* a HIP runtime call failed; see pa_last_hip_error() */
    PA_ERR_WORKSPACE = 10, /* split-KV: workspace_bytes below prefill_attn_splitkv_workspace_size() */
    PA_ERR_NOALLOC_LIMIT = 11 /* no-allocation split-KV: the workspace the problem needs exceeds prefill_attn_splitkv_noalloc_limit() */
} pa_status;

/*
 * Varlen causal prefill with KV-cache write.
 *
 *   q, k, v      bf16 [N, H, D] device, read only.
 *   cu_seqlens   int32 [num_seqs + 1] device.
 *   num_seqs     B >= 0 (host).
 *   max_seqlen   host upper bound on every cu[b+1] - cu[b]; sizes the grid.
 *   num_heads    H >= 1; head_dim D in {32, 64, 128}.
 *   k_cache,     bf16 device, written only: sequence b's cache block is
 *   v_cache      [H, len_b, D] starting at element cu[b] * H * D, so the
 *                buffers hold N * H * D elements in total.  This is the
 *                per-layer cache layout [batch, heads, seq, head_dim] of
 *                [P2 §1.3] and [P4 §3.2], head-major as [P1 §3] advises,
 *                with one sequence per batch entry packed back to back.
 *                Prefill produces K and V of every prompt position
 *                [P5 §1.1]; Q is not cached [P2 §1.3].
 *   out          bf16 [N, H, D] device, written only (rounded to nearest even).
 *   scale        softmax scale applied to q.k.
 *   stream       HIP stream (NULL = default stream).
 */
pa_status prefill_attn_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *cu_seqlens, int32_t num_seqs,
                              int32_t max_seqlen, int32_t num_heads, int32_t head_dim,
                              uint16_t *k_cache, uint16_t *v_cache, uint16_t *out,
                              float scale, hipStream_t stream);

/*
 * Chunked prefill: each sequence already has prefix_lens[b] tokens in the
 * cache, and its new tokens (a prompt chunk, or a single decode token) attend
 * to that cached prefix and causally to each other [P3 §3 chunked prefill
 * co-scheduled with decode; P2 §2.2; P5 §1.2: the decoded token attends to
 * every cached position and to itself].  Query i of sequence b sits at
 * absolute position prefix_lens[b] + i and sees keys 0 .. prefix_lens[b] + i.
 *
 *   q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, head_dim, out,
 *   scale, stream      as for prefill_attn_varlen (new tokens only).
 *   k_cache, v_cache   bf16 [num_seqs, H, cache_capacity, D] device.  Positions
 *                      0 .. prefix_lens[b]-1 of sequence b are read; the new
 *                      tokens' K/V are written at positions prefix_lens[b] ..
 *                      prefix_lens[b] + len_b - 1; nothing else is touched.
 *                      With B = 1, prefix 0 and capacity = len, this layout is
 *                      byte-identical to the varlen cache block.
 *   cache_capacity     positions per (sequence, head) in the cache, >= 1.
 *   prefix_lens        int32 [num_seqs] device, 0 <= prefix_lens[b] and
 *                      prefix_lens[b] + len_b <= cache_capacity.
 *
 * The new tokens' own K/V are read from k and v, never from the cache, so no
 * work-group reads a cache position the same call writes, and repeating the
 * call with the same arguments writes identical bytes.
 */
pa_status prefill_attn_chunked(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const int32_t *cu_seqlens, int32_t num_seqs,
                               int32_t max_seqlen, int32_t num_heads, int32_t head_dim,
                               uint16_t *k_cache, uint16_t *v_cache,
                               int32_t cache_capacity, uint16_t *out, float scale,
                               hipStream_t stream, const int32_t *prefix_lens);

/*
 * Grouped K/V heads (grouped-query / multi-query attention) [P5 §2.4: fewer
 * K/V heads than query heads, 32 -> 8 in its example, shrink the KV cache in
 * proportion].  As prefill_attn_varlen / prefill_attn_chunked, except:
 *
 *   num_kv_heads   HK >= 1 dividing num_heads H.  Query head h reads K/V head
 *                  h / (H / HK): consecutive query heads share one K/V head
 *                  (HK = 1: one K/V head for all, multi-query).
 *   k, v           bf16 [N, HK, D] device.
 *   k_cache,       varlen: sequence b's block is [HK, len_b, D] starting at
 *   v_cache        element cu[b] * HK * D (N * HK * D elements in total);
 *                  chunked: [num_seqs, HK, cache_capacity, D].  Each K/V head
 *                  row is written once.
 *   q, out         bf16 [N, H, D] as before.
 *
 * With num_kv_heads == num_heads these are the calls above; errors as above,
 * plus PA_ERR_SHAPE when num_kv_heads < 1 or does not divide num_heads.
 */
pa_status prefill_attn_varlen_gqa(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                  const int32_t *cu_seqlens, int32_t num_seqs,
                                  int32_t max_seqlen, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, uint16_t *k_cache, uint16_t *v_cache,
                                  uint16_t *out, float scale, hipStream_t stream);
pa_status prefill_attn_chunked_gqa(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                   const int32_t *cu_seqlens, int32_t num_seqs,
                                   int32_t max_seqlen, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, uint16_t *k_cache, uint16_t *v_cache,
                                   int32_t cache_capacity, uint16_t *out, float scale,
                                   hipStream_t stream, const int32_t *prefix_lens);

/*
 * Varlen prefill writing an INT8 KV cache.  Attention is computed exactly as
 * prefill_attn_varlen_gqa (on the bf16 inputs); only the cache write differs:
 * K and V are quantised, Q is not [P2 §4.3: quantising the KV cache to INT8
 * halves its size and read traffic; scales may be per tensor, per channel or
 * per token].  Each (token, K/V head) row of D values gets one float scale:
 *     scale = amax / 127,  code = rint(x * (127 / amax)),  |code| <= 127,
 * in float32 with ties to even (a row whose amax is below 2^-100 is stored
 * as scale 0 and codes 0); the value it stands for is code * scale.
 *
 *   k_cache, v_cache   int8 device, written only, laid out as the bf16 varlen
 *                      cache: sequence b's [HK, len_b, D] block starts at
 *                      byte cu[b] * HK * D (N * HK * D bytes in total).
 *   k_scale, v_scale   float device, written only: sequence b's [HK, len_b]
 *                      block starts at element cu[b] * HK (N * HK floats).
 *   other arguments    as prefill_attn_varlen_gqa.
 *
 * Errors as prefill_attn_varlen_gqa; the scale pointers are outputs too
 * (PA_ERR_NULL, PA_ERR_ALIGN, PA_ERR_ALIAS apply to them).
 */
pa_status prefill_attn_varlen_int8(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                   const int32_t *cu_seqlens, int32_t num_seqs,
                                   int32_t max_seqlen, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int8_t *k_cache, int8_t *v_cache,
                                   float *k_scale, float *v_scale, uint16_t *out, float scale,
                                   hipStream_t stream);

/*
 * Varlen prefill writing an FP8 KV cache: as prefill_attn_varlen_int8 with
 * one-byte codes in the OCP 8-bit E4M3 format [P2 §4.3 lists low-precision
 * cache formats; the E4M3 encoding is this library's reading]: a sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, no
 * infinities, S.1111.111 NaN, largest finite magnitude 448.  Per (token, K/V
 * head) row:
 *     scale = amax / 448,  code = E4M3(x * (448 / amax)),
 * the product in float32, the code the nearest E4M3 value with ties to even
 * (a row whose amax is below 2^-100 gets scale 0 and the codes of x * 0,
 * zeros that keep x's sign); the value it stands for is E4M3 value * scale.
 * Layout, scales, arguments and errors as prefill_attn_varlen_int8.
 */
pa_status prefill_attn_varlen_fp8(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                  const int32_t *cu_seqlens, int32_t num_seqs,
                                  int32_t max_seqlen, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, uint8_t *k_cache, uint8_t *v_cache,
                                  float *k_scale, float *v_scale, uint16_t *out, float scale,
                                  hipStream_t stream);

/*
 * Split-KV chunked prefill.  Same result and cache writes as
 * prefill_attn_chunked_gqa, computed so that long key ranges do not serialise
 * on one work-group: in a chunked step a prompt chunk is batched with decode
 * rows [P3 §3; P2 §2.2], and a decode row reads every cached position of its
 * sequence [P5 §3.3], so a few long rows would otherwise leave most compute
 * units idle.  Each query block's keys are cut into segments of at least 1024
 * keys; every segment is an independent work item, and a block with more
 * than one segment is finished by an fp32 log-sum-exp merge of the segments'
 * partial results.  Enqueued on `stream`: a plan, one persistent attention
 * launch, a launch for the length-1 rows unless the attention launch runs
 * them beside the chunk's blocks (B > 1, max_seqlen > 1, at most two query
 * heads per K/V head), and the merge.  Rows differ from
 * prefill_attn_chunked_gqa only by floating-point rounding order.
 *
 *   num_tokens        N, the rows of q, k, v and out (host); cu_seqlens[B]
 *                     must not exceed it (check mode: PA_ERR_SEQLENS).
 *   workspace         device scratch memory, 16-byte aligned, of at least
 *                     prefill_attn_splitkv_workspace_size(...) bytes, owned by
 *                     the caller; its contents on entry do not matter and on
 *                     return are unspecified.  Calls that overlap in time
 *                     (other streams) need separate workspaces.
 *   other arguments   as prefill_attn_chunked_gqa.
 *
 * Errors as prefill_attn_chunked_gqa, plus PA_ERR_NULL for a NULL workspace,
 * PA_ERR_ALIGN, PA_ERR_ALIAS if the workspace equals another pointer,
 * PA_ERR_SHAPE for num_tokens < 0 or cache_capacity * head_dim >= 2^32 (one
 * (sequence, K/V head) row of the cache must span fewer than 2^32 elements;
 * 33.5M positions at D = 128), and PA_ERR_WORKSPACE when workspace_bytes is
 * too small.  B == 0, max_seqlen == 0 or num_tokens == 0 enqueue nothing.
 */
pa_status prefill_attn_chunked_splitkv(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                       const int32_t *cu_seqlens, int32_t num_seqs,
                                       int32_t max_seqlen, int32_t num_tokens,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       uint16_t *k_cache, uint16_t *v_cache,
                                       int32_t cache_capacity, uint16_t *out, float scale,
                                       hipStream_t stream, const int32_t *prefix_lens,
                                       void *workspace, size_t workspace_bytes);

/*
 * prefill_attn_chunked_splitkv without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It allocates nothing: the plan,
 * partial results and counters live in a fixed array of
 * prefill_attn_splitkv_noalloc_limit() bytes (128 MiB) that the library holds
 * on each GPU it runs on until the process ends.  The array of the current
 * device is used (its address is looked up on the first call on a device).
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero: each call's plan writes
 * what the call reads).  Calls that overlap in time on one GPU (other
 * streams, other threads) race on it and must be serialised by the caller.
 * Check mode's host-side metadata checks are not run (they copy metadata to
 * host memory).
 *
 * Arguments, results and errors as prefill_attn_chunked_splitkv, without
 * workspace and workspace_bytes; PA_ERR_NOALLOC_LIMIT when
 * prefill_attn_splitkv_workspace_size(num_seqs, num_tokens, num_heads,
 * head_dim, cache_capacity) exceeds the array (nothing is enqueued).
 */
pa_status prefill_attn_chunked_splitkv_noalloc(const uint16_t *q, const uint16_t *k,
                                               const uint16_t *v, const int32_t *cu_seqlens,
                                               int32_t num_seqs, int32_t max_seqlen,
                                               int32_t num_tokens, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               uint16_t *k_cache, uint16_t *v_cache,
                                               int32_t cache_capacity, uint16_t *out, float scale,
                                               hipStream_t stream, const int32_t *prefix_lens);

/* Bytes of the per-GPU array prefill_attn_chunked_splitkv_noalloc uses. */
size_t prefill_attn_splitkv_noalloc_limit(void);

/*
 * Split-KV chunked prefill over a paged KV cache [P2 §4.2 and P5 §3.4: the
 * cache is cut into fixed 16-token blocks that need not be contiguous, a
 * block table maps each request's logical blocks to physical ones, and
 * requests with a common prefix can point at the same blocks; P4 §4.1 shows
 * a block as a small tokens x heads x head_dim array].  Same computation as
 * prefill_attn_chunked_splitkv; only where cache positions live differs.
 *
 *   k_cache, v_cache     bf16 [num_blocks, HK, 16, D] device: block n holds 16
 *                        consecutive positions of one request, head-major.
 *   block_table          int32 [num_seqs, max_blocks_per_seq] device: position
 *                        j of sequence b is row j % 16 of block
 *                        block_table[b][j / 16].  Every block a sequence
 *                        touches (positions below prefix_lens[b] + len_b)
 *                        must be in [0, num_blocks); the blocks receiving new
 *                        tokens must not be shared with another sequence of
 *                        the call.  Entries past those are not read.
 *   num_blocks           blocks in the pool (>= 1).
 *   max_blocks_per_seq   columns of block_table (>= 1); the capacity per
 *                        sequence is 16 * max_blocks_per_seq positions.
 *   workspace            prefill_attn_splitkv_workspace_size(num_seqs,
 *                        num_tokens, num_heads, head_dim,
 *                        16 * max_blocks_per_seq) bytes at least.
 *   other arguments      as prefill_attn_chunked_splitkv.
 *
 * Errors as prefill_attn_chunked_splitkv, plus PA_ERR_NULL for a NULL block
 * table, PA_ERR_SHAPE for num_blocks or max_blocks_per_seq < 1, PA_ERR_ALIAS
 * if block_table equals an output or the workspace; check mode also returns
 * PA_ERR_CAPACITY for a block id outside the pool.
 */
pa_status prefill_attn_chunked_splitkv_paged(
    const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *cu_seqlens,
    int32_t num_seqs, int32_t max_seqlen, int32_t num_tokens, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, uint16_t *k_cache, uint16_t *v_cache,
    int32_t num_blocks, const int32_t *block_table, int32_t max_blocks_per_seq, uint16_t *out,
    float scale, hipStream_t stream, const int32_t *prefix_lens, void *workspace,
    size_t workspace_bytes);

/*
 * Workspace bytes prefill_attn_chunked_splitkv needs for these sizes (host
 * values only; 0 for invalid arguments).  It grows with num_tokens * num_heads
 * * head_dim * segments, segments being at most 64 and at most
 * ceil(cache_capacity / 1024).
 */
size_t prefill_attn_splitkv_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                           int32_t num_heads, int32_t head_dim,
                                           int32_t cache_capacity);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *pa_status_string(int status);

/* Turn check mode on (1) or off (0); returns the previous setting.  Process-wide. */
int pa_set_check_mode(int on);

/* hipError_t of the last PA_ERR_HIP returned on the calling thread (0 if none). */
int pa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PREFILL_ATTN_H */
