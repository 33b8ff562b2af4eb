/*
 * attn.h -- C ABI of libattn.so: fused scaled-dot-product attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations are those of the blog post "从零实现 vLLM (1.3)：如何加速
 * Attention 计算": O = softmax(s * Q K^T) V (section Attention 的计算过程,
 * with the scale of the 标准实现方法 second step), computed in one pass over
 * K/V tiles with the online-softmax state (m, d', o') of sections
 * FlashAttention 的最终实现 and 计算流程(1-Pass 算法与分块), so that the logits
 * and probabilities never reach device memory.  Argument names follow the
 * calls in the page's Attention 源码分析 section (store_kvcache,
 * flash_attn_varlen_func, flash_attn_with_kvcache).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array argument is a DEVICE pointer to a packed, row-major array
 *   owned by the caller.  The library never allocates, frees or retains
 *   memory, keeps no global mutable state, and is safe to call from several
 *   host threads on different streams.
 * - stream is a hipStream_t passed as void* (NULL = the default stream).
 *   Calls are asynchronous on that stream and never synchronise the host.
 *   Kernels launch on the current HIP device (hipSetDevice), whose compute
 *   unit count sizes the persistent grids; the arrays and the stream must
 *   belong to that device.
 * - Host-side argument validation runs before any HIP call.  On failure the
 *   call returns a nonzero status and launches nothing.  Launch failures
 *   return ATTN_ERR_HIP.  No C++ exception crosses the ABI.
 * - Values that live in device memory (cu_seqlens, block tables, slot
 *   mappings, cache lengths) are preconditions the host cannot check without
 *   a sync.  The kernels bound every access by the sizes passed here: a
 *   block id outside [0, num_blocks) reads as zero rows in decode and in the
 *   fp32 prefill, and as physical block 0 in the bf16/fp16 prefill; a slot
 *   outside the cache is skipped; a sequence range outside [0, total) is
 *   clipped.  Bad metadata gives wrong numbers, never an out-of-bounds
 *   access.
 * - dtype codes: ATTN_F32 (IEEE binary32), ATTN_BF16 (bfloat16) and ATTN_F16
 *   (IEEE binary16).
 * - Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 */
#ifndef ATTN_MI355X_ATTN_H
#define ATTN_MI355X_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL                    */
    ATTN_ERR_SHAPE = 2,       /* a size is negative/zero or sizes disagree      */
    ATTN_ERR_UNSUPPORTED = 3, /* valid, but not a supported dtype/head_dim/... */
    ATTN_ERR_WORKSPACE = 4,   /* decode workspace missing or too small          */
    ATTN_ERR_HIP = 5          /* the HIP runtime reported an error              */
};

enum attn_dtype { ATTN_F32 = 0, ATTN_BF16 = 1, ATTN_F16 = 2 };

/* Status code -> static, human-readable string (never NULL). */
const char *attn_status_str(int status);

/* Library version, major*10000 + minor*100 + patch. */
int attn_version(void);

/*
 * kv_store_slots -- the store_kvcache step of the page's Attention 源码分析
 * section, run before attention in both prefill and decode.
 *
 * For every token t in [0, num_tokens) with slot = slot_mapping[t] >= 0:
 *     k_cache[slot / block_size][slot % block_size][g][:] = k[t][g][:]
 *     v_cache[slot / block_size][slot % block_size][g][:] = v[t][g][:]
 * for all KV heads g.  Negative slots are skipped (padding tokens); slots at
 * or beyond num_blocks * block_size are skipped too.  Bit-exact copy.
 *
 *   k, v          [num_tokens, num_kv_heads, head_dim]     dtype, 16-B aligned
 *   k_cache,
 *   v_cache       [num_blocks, block_size, num_kv_heads, head_dim], dtype
 *   slot_mapping  [num_tokens] int32; slots must be distinct (two tokens
 *                 writing one slot race and the result is either of them)
 *   dtype         ATTN_BF16, ATTN_F16 or ATTN_F32 (rows are copied bit for bit)
 * num_tokens == 0 is a no-op returning ATTN_OK.
 */
int kv_store_slots(const void *k, const void *v, void *k_cache, void *v_cache,
                   const int32_t *slot_mapping, int num_tokens, int num_kv_heads,
                   int head_dim, int num_blocks, int block_size, int dtype,
                   void *stream);

/*
 * attn_prefill_varlen -- variable-length prefill (the page's Prefill section,
 * flash_attn_varlen_func), including the prefix-cache case.
 *
 * Sequences are packed without padding.  Sequence b owns query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (Lq_b of them) and Lk_b =
 * cu_seqlens_k[b+1] - cu_seqlens_k[b] keys.  For each query row i of
 * sequence b and query head h:
 *     O[i][h][:] = sum_{j in J} softmax_j(s * q_i . k_j) v_j
 * with J = { j < Lk_b : !causal or j <= i + Lk_b - Lq_b }, i.e. the causal
 * mask is aligned to the END of the sequence, so that with a prefix cache
 * (Lq_b < Lk_b, queries are the newest tokens) query i sits at absolute
 * position Lk_b - Lq_b + i.  A row with an empty J is written as zeros.
 *
 * K/V source:
 *   block_table == NULL: k, v are packed [total_k, num_kv_heads, head_dim];
 *       key j of sequence b is row cu_seqlens_k[b] + j.  max_blocks_per_seq,
 *       num_blocks and block_size are ignored.
 *   block_table != NULL (prefix cache): k, v are the paged caches
 *       [num_blocks, block_size, num_kv_heads, head_dim]; key j of sequence
 *       b is slot block_table[b * max_blocks_per_seq + j / block_size]
 *       * block_size + j % block_size.  total_k is ignored; Lk_b still comes
 *       from cu_seqlens_k.  Table entries past ceil(Lk_b / block_size) are
 *       never read.  num_blocks * block_size must fit a 32-bit int (else
 *       ATTN_ERR_SHAPE).
 *
 *   q            [total_q, num_q_heads, head_dim], in_dtype
 *   o            [total_q, num_q_heads, head_dim], out_dtype (written only
 *                for rows that belong to a sequence)
 *   cu_seqlens_q, cu_seqlens_k  [batch + 1] int32, nondecreasing, from 0
 *   max_seqlen_q, max_seqlen_k  upper bounds of Lq_b, Lk_b (host ints; they
 *                size the launch, rows beyond max_seqlen_q are not computed)
 *   softmax_scale  s > 0 and finite (usually 1/sqrt(head_dim)), with
 *                s * log2(e) at least FLT_MIN; anything else (0, negative,
 *                non-finite, subnormal) is rejected with ATTN_ERR_SHAPE
 *   causal       nonzero = causal mask as above
 *
 * Supported: in_dtype ATTN_BF16 or ATTN_F16 with head_dim 128 (16-bit
 * matrix cores, P rounded to the input type, fp32 softmax state; out_dtype
 * ATTN_F32 or the input type) and in_dtype ATTN_F32 with head_dim 64 or 128
 * (fp32 throughout; out_dtype ATTN_F32 or ATTN_BF16); conversions round to
 * nearest even;
 * num_q_heads a multiple of num_kv_heads; block_size a multiple of 64 when
 * paged.  Pointers must be 16-byte aligned; k and v may be NULL when
 * block_table is NULL and total_k is 0 (no key anywhere; every row is 0).
 */
int attn_prefill_varlen(const void *q, const void *k, const void *v, void *o,
                        const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                        int batch, int max_seqlen_q, int max_seqlen_k,
                        int total_q, int total_k,
                        int num_q_heads, int num_kv_heads, int head_dim,
                        float softmax_scale, int causal,
                        const int32_t *block_table, int max_blocks_per_seq,
                        int num_blocks, int block_size,
                        int in_dtype, int out_dtype, void *stream);

/*
 * attn_prefill_padded -- the same attention as attn_prefill_varlen for a
 * padded batch (the page's Prefill section contrasts the padded layout of
 * a batch with its varlen packing by cu_seqlens; the two give the same
 * outputs on the valid rows).  Sequence b holds seqlens_q[b] queries at
 * rows 0 .. of q[b] and seqlens_k[b] keys at rows 0 .. of k[b] and v[b]
 * (lengths are clipped to [0, max_seqlen_*]); the causal mask is aligned to
 * the sequence end as in attn_prefill_varlen.  Padded rows are not read as
 * keys, and output rows at or past seqlens_q[b] are left unchanged.  The
 * varlen kernels run in place on the padded tensors: nothing is packed or
 * copied.
 *
 *   q, o           [batch, max_seqlen_q, num_q_heads, head_dim]
 *   k, v           [batch, max_seqlen_k, num_kv_heads, head_dim]
 *   seqlens_q,
 *   seqlens_k      [batch] int32 device arrays
 *
 * Supported: as attn_prefill_varlen with contiguous K/V; batch *
 * max_seqlen_q and batch * max_seqlen_k below 2^31.  k and v may be NULL
 * when max_seqlen_k is 0 (no sequence has a key; every valid row is 0).
 * Errors as attn_prefill_varlen.
 */
int attn_prefill_padded(const void *q, const void *k, const void *v, void *o,
                        const int32_t *seqlens_q, const int32_t *seqlens_k,
                        int batch, int max_seqlen_q, int max_seqlen_k,
                        int num_q_heads, int num_kv_heads, int head_dim,
                        float softmax_scale, int causal, int in_dtype, int out_dtype,
                        void *stream);

/*
 * attn_decode_workspace_bytes -- bytes of device workspace attn_decode_paged
 * needs for these sizes (0 if the sizes are invalid).  Layout: partial
 * slots S = 1024 + batch, each with num_q_heads rows of head_dim fp32
 * values; then, 256-byte aligned, 2 fp32 words per (slot, head) (m, d');
 * then, 256-byte aligned, two int32 per sequence.  The size
 * does not depend on max_blocks_per_seq, block_size or split_tokens, which
 * are validated as in attn_decode_paged.  Nothing needs clearing between
 * calls: every word the combine reads is written by the same call.
 */
size_t attn_decode_workspace_bytes(int batch, int num_q_heads, int num_kv_heads,
                                   int head_dim, int max_blocks_per_seq,
                                   int block_size, int split_tokens);

/*
 * attn_decode_paged -- single-token decode against a paged KV cache (the
 * page's Decode section, flash_attn_with_kvcache with q.unsqueeze(1)).
 *
 * For each sequence b and query head h, with L = cache_seqlens[b] (the
 * context length INCLUDING the token just stored by kv_store_slots):
 *     O[b][h][:] = sum_{j < L} softmax_j(s * q[b][h] . k_j) v_j
 * where key j is cache slot block_table[b * max_blocks_per_seq +
 * j / block_size] * block_size + j % block_size.  With one query per
 * sequence the causal mask hides nothing.  L == 0 gives a zero row; L is
 * clipped to max_blocks_per_seq * block_size.
 *
 * The keys of every sequence are cut into items of split_tokens keys (0 =
 * the library's choice, 32; else a positive multiple of 32).  The items of
 * all sequences, in order, are dealt in equal contiguous runs to persistent
 * workgroups (one per compute unit), each serving every KV head of its
 * keys.  A workgroup keeps the online state (m, d', unnormalised o') across
 * the items of one sequence it reads and stores one partial per sequence it
 * touches; a second kernel merges the partials with the same rescaling the
 * online recurrence uses.  The result does not depend on how the runs fall,
 * up to floating-point rounding order.
 *
 *   q             [batch, num_q_heads, head_dim], in_dtype
 *   k_cache,
 *   v_cache       [num_blocks, block_size, num_kv_heads, head_dim], in_dtype
 *   o             [batch, num_q_heads, head_dim], out_dtype
 *   cache_seqlens [batch] int32
 *   block_table   [batch, max_blocks_per_seq] int32
 *   softmax_scale s > 0, as for attn_prefill_varlen (else ATTN_ERR_SHAPE)
 *   workspace     device scratch of at least attn_decode_workspace_bytes()
 *                 bytes, 256-byte aligned, not shared with a concurrent call
 *
 * Supported: in_dtype ATTN_BF16 or ATTN_F16, head_dim 128, num_q_heads /
 * num_kv_heads <= 16, block_size a multiple of 64; out_dtype ATTN_F32 or
 * the input type.
 * Errors: ATTN_ERR_NULL for a null pointer; ATTN_ERR_SHAPE for non-positive
 * sizes, num_q_heads not a multiple of num_kv_heads or a bad scale;
 * ATTN_ERR_UNSUPPORTED outside the supported set (also split_tokens not a
 * multiple of 32, unaligned pointers); ATTN_ERR_WORKSPACE for a missing,
 * small or unaligned workspace; ATTN_ERR_HIP if the device query or a
 * launch fails.  Nothing is launched unless the status is ATTN_OK.
 */
int attn_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                      void *o, const int32_t *cache_seqlens,
                      const int32_t *block_table, int batch, int num_q_heads,
                      int num_kv_heads, int head_dim, int max_blocks_per_seq,
                      int num_blocks, int block_size, float softmax_scale,
                      int split_tokens, int in_dtype, int out_dtype,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments (minus workspace),
 * semantics, kernels and results as attn_decode_paged; the workspace is a
 * scratch array of 32 MiB built into the library, one per GPU, resolved on
 * the first call on each device and held until the process ends.
 *
 * Limit: the call's workspace must fit that scratch.  It is laid out as in
 * attn_decode_workspace_bytes but for the runs this device uses (its
 * compute units divided by the blocks of up to 8 KV heads: 256 on a
 * 256-CU MI355X with 8 KV heads) instead of the 1024 any device may use, so
 * at head_dim 128 on that GPU: batch <= 1759 at 32 query heads, 752 at 64,
 * 248 at 128.  Larger calls return ATTN_ERR_WORKSPACE and launch nothing.  Nothing in the scratch needs clearing (every word the
 * merge reads is written by the same call).  All calls on one GPU share its
 * scratch: calls that overlap in time on one GPU (different streams, or
 * host threads without ordering) race and give wrong results; serialise
 * them, e.g. on one stream.  No hipMalloc, hipFree or allocating library
 * call is made.  Errors as attn_decode_paged, plus ATTN_ERR_HIP if the
 * scratch address cannot be resolved.
 */
int attn_decode_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              void *o, const int32_t *cache_seqlens,
                              const int32_t *block_table, int batch, int num_q_heads,
                              int num_kv_heads, int head_dim, int max_blocks_per_seq,
                              int num_blocks, int block_size, float softmax_scale,
                              int split_tokens, int in_dtype, int out_dtype, void *stream);

/*
 * attn_unfused_workspace_bytes -- bytes of device workspace
 * attn_prefill_unfused needs (0 if the sizes are invalid): the logits X as
 * fp32, then (256-byte aligned) the probabilities A as bf16, each laid out
 * [batch, num_q_heads, max_seqlen_q, ldx] with ldx = max_seqlen_k rounded
 * up to a multiple of 64, plus 64.
 */
size_t attn_unfused_workspace_bytes(int batch, int num_q_heads, int max_seqlen_q,
                                    int max_seqlen_k);

/*
 * attn_prefill_unfused -- the page's standard, unfused method (section
 * 标准实现方法) as a measured baseline for attn_prefill_varlen: three kernels,
 *     X = softmax_scale * Q K^T          (written to the workspace, fp32)
 *     A = softmax(X) row by row          (3-pass safe softmax, masked keys
 *                                         get weight 0; written as bf16)
 *     O = A V
 * with the same arguments, semantics (varlen packing, GQA, end-aligned
 * causal mask, zero rows for queries with no visible key) and output as
 * attn_prefill_varlen with block_table == NULL.  X and A are formed for
 * every (query, key) pair of each sequence, as the standard method does, so
 * they cost HBM traffic of about 12 bytes per pair and head.
 *
 *   workspace    at least attn_unfused_workspace_bytes(batch, num_q_heads,
 *                max_seqlen_q, max_seqlen_k) bytes, 256-byte aligned;
 *                contents on entry are ignored
 *
 * Supported: in_dtype ATTN_BF16, head_dim 128, contiguous K/V, out_dtype
 * ATTN_F32 or ATTN_BF16, batch * num_q_heads <= 65535, 16-byte aligned
 * pointers.  Errors as attn_prefill_varlen, plus ATTN_ERR_WORKSPACE for a
 * missing, small or unaligned workspace.  Nothing is launched unless the
 * status is ATTN_OK.  Asynchronous on stream; allocates nothing.
 */
int attn_prefill_unfused(const void *q, const void *k, const void *v, void *o,
                         const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                         int batch, int max_seqlen_q, int max_seqlen_k,
                         int total_q, int total_k, int num_q_heads, int num_kv_heads,
                         int head_dim, float softmax_scale, int causal, int in_dtype,
                         int out_dtype, void *workspace, size_t workspace_bytes,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_ATTN_H */
