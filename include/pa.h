/*
 * pa.h — C ABI of the paged-attention library (libpa.so) for AMD Instinct MI355X (gfx950).
 *
 * Attention over a paged, block-structured KV cache, and the cache operations around it:
 *   pa_store_kv        scatter new keys/values into cache slots (slot_mapping)
 *   pa_copy_blocks     duplicate physical blocks of both cache planes
 *   pa_prefill_varlen  varlen causal attention (chunked, optional sliding window)
 *   pa_decode          grouped-query decode, one query per sequence, split-K
 *   pa_prefill_varlen_with_store, pa_decode_with_store
 *                      the store of the new tokens and the attention in one call
 *   pa_cascade_decode  decode of a batch that shares a prefix of cached blocks
 *   pa_cascade_prefill_varlen
 *                      prefill of query chunks that share a prefix of cached blocks
 *   pa_decode_no_alloc pa_decode with its scratch in the library (no workspace argument)
 *   pa_*_workspace_size, pa_status_string, pa_last_error
 * Options: ALiBi slopes (alibi_slopes arguments) and an FP8 (E4M3) cache with a kv_scale
 * (pa_cache_desc.dtype / kv_scale).
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers, caller-allocated and caller-owned; the
 *     library never allocates, frees or keeps them.  Index arrays are int32.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls only
 *     enqueue work on it and never synchronise; the result is ready when the stream is.
 *   - Scalars are checked on the host before any HIP call; a failed check returns a
 *     non-zero pa_status and pa_last_error() names the argument.  Device contents (slot
 *     values, table entries, lengths) are preconditions that are not checked.
 *   - Zero work (no tokens, no sequences, zero-length sequences) is PA_OK and a no-op.
 *
 * Cache layout (vLLM learning book, "05. Attention Backends", section 3, FlashAttention
 * backend get_kv_cache_shape): one contiguous buffer
 *     kv_cache[2][num_blocks][block_size][num_kv_heads][head_size]
 * plane 0 holds keys, plane 1 values; element (p, b, o, g, d) is at linear index
 * (((p*num_blocks + b)*block_size + o)*num_kv_heads + g)*head_size + d.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,   /* null pointer with work to do, bad size or count        */
    PA_ERR_UNSUPPORTED = 2,   /* head size, block size, dtype or group size not built     */
    PA_ERR_WORKSPACE = 3,     /* decode workspace missing or smaller than required        */
    PA_ERR_LAUNCH = 4         /* the HIP runtime reported an error at launch              */
} pa_status;

typedef enum pa_dtype {
    PA_F32 = 0,               /* float32 cache, q/k/v and output                          */
    PA_BF16 = 1,              /* bfloat16 cache, q/k/v and output; fp32 accumulation      */
    PA_FP8_E4M3 = 2           /* 8-bit float cache holding value / kv_scale; q/k/v and
                                 output bfloat16; fp32 accumulation (see below)           */
} pa_dtype;

/* Description of the caller's cache.  head_size in {64, 128}; block_size a power of two in
 * [1, 256] for PA_F32 and in [16, 256] for PA_BF16 and PA_FP8_E4M3; num_blocks*block_size
 * < 2^31.
 *
 * PA_FP8_E4M3 (vllm-npu 0.4.2 diff, torch_sdpa.py forward: the store and decode calls take
 * kv_cache_dtype and kv_scale; vLLM learning book, "05. Attention Backends", section 5: the
 * cache planes viewed as an FP8 dtype): one byte per element, the E4M3 format of the OCP 8-bit
 * floating-point specification (sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, largest finite 448).  The store writes e4m3(x * r), r = fp32(1 / kv_scale),
 * rounded to nearest even and saturated to +-448; attention reads e4m3 * kv_scale.  kv_scale
 * must be finite and > 0 for such a cache and is ignored otherwise.  Every call supports it;
 * pa_prefill_varlen_with_store then runs the store before the attention instead of inside
 * it, so the attention reads the quantized new rows like any other cached row. */
typedef struct pa_cache_desc {
    void*   kv_cache;
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_size;
    int32_t dtype;            /* a pa_dtype value */
    float   kv_scale;         /* PA_FP8_E4M3 only */
} pa_cache_desc;

/*
 * pa_store_kv — write token t's key and value rows into its cache slot.
 *
 * MinivLLM API docs, "Attention" page, section store_kvcache (and its example); vLLM
 * learning book, section 10 question 2: slot = physical_block * block_size + offset, so
 * cache[0][slot / block_size][slot % block_size][:][:] = key[t] and plane 1 = value[t].
 * A negative slot (-1 padding) skips the token.  The copy is bitwise (for PA_FP8_E4M3 each
 * element is quantized as the cache description states).
 *
 *   key, value    [num_tokens][num_kv_heads][head_size], contiguous, cache dtype (bfloat16
 *                 for PA_FP8_E4M3)
 *   slot_mapping  [num_tokens] int32
 * Preconditions: every non-negative slot < num_blocks*block_size and no slot repeats
 * (a repeated slot is a write race).
 */
int pa_store_kv(const pa_cache_desc* cache, const void* key, const void* value,
                const int32_t* slot_mapping, int32_t num_tokens, void* stream);

/*
 * pa_copy_blocks — for each pair (src, dst): cache[:, dst] = cache[:, src], both planes.
 *
 * vllm-npu 0.4.2 diff, torch_sdpa.py / xformers.py backend, copy_blocks(kv_caches,
 * src_to_dists) (copy-on-write forks; the pages give the signature only).
 *   block_pairs  [num_pairs][2] int32 (src, dst)
 * Preconditions: ids in [0, num_blocks); dst values unique and not among the src values,
 * so every copy reads the pre-call contents.
 */
int pa_copy_blocks(const pa_cache_desc* cache, const int32_t* block_pairs, int32_t num_pairs,
                   void* stream);

/*
 * pa_prefill_varlen — attention for packed query chunks over keys already in the cache.
 *
 * MinivLLM API docs, section flash_attention_prefill (packed varlen queries, cu_seqlens,
 * online softmax, GQA); HF transformers continuous_batching input_ouputs.py,
 * build_attention_mask (bottom-right causal diagonal when seqlen_q < seqlen_k, sliding
 * window); vLLM learning book section 5 (varlen call with block_table).
 *
 * Sequence s owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1]) and has
 * seqlen_k = cu_seqlens_k[s+1] - cu_seqlens_k[s] keys, logical key j at
 * block_table[s*max_blocks_per_seq + j/block_size], offset j % block_size.  Row i sits at
 * position p = seqlen_k - seqlen_q + i and attends keys j in [lo, p] with
 * lo = max(0, p - sliding_window + 1) when sliding_window > 0, else 0.  Query head h reads
 * KV head h / (num_heads / num_kv_heads).  out = softmax(scale * q.K^T) V per row and head;
 * a row with no key (p < 0) is written as zeros.
 *
 *   out, query    [cu_seqlens_q[num_seqs]][num_heads][head_size], contiguous, cache dtype
 *   block_table   [num_seqs][max_blocks_per_seq] int32 (entries outside a sequence's live
 *                 key range are never read and may be -1)
 *   cu_seqlens_q, cu_seqlens_k  [num_seqs + 1] int32, non-decreasing, starting at 0
 *   max_seqlen_q  >= every seqlen_q (sizes the grid); max_seqlen_k >= every seqlen_k
 *   scale         final multiplier of q.K^T (e.g. 1/sqrt(head_size)), finite and > 0
 *   alibi_slopes  NULL, or [num_heads] float32 ALiBi slopes: the score of query head h at
 *                 position p for key j gets alibi_slopes[h] * (j - p) added after the scale
 *                 (vllm-npu 0.4.2 diff, torch_sdpa.py / xformers.py, _make_alibi_bias)
 * Keys must already be stored (pa_store_kv first).  The K/V tiles are read only inside
 * each row's live range, so cache slots outside it may hold anything, NaN included.
 */
int pa_prefill_varlen(const pa_cache_desc* cache, void* out, const void* query,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                      int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                      int32_t num_heads, float scale, int32_t sliding_window,
                      const float* alibi_slopes, void* stream);

/*
 * pa_prefill_varlen_with_store — pa_store_kv of the batch's new tokens, then
 * pa_prefill_varlen, as one call.
 *
 * vLLM learning book, "05. Attention Backends", section 5 (FlashAttentionImpl.forward) and
 * the section-10 question on how K/V reach the cache: the attention kernel itself writes the
 * new tokens' K/V at their slot_mapping slots, saving the separate store launch.  Here, for
 * bf16 caches, the prefill kernel takes the new keys straight from key/value (they are the
 * last seqlen_q keys of each sequence) and writes them to the cache as it goes; float32 and
 * FP8 caches run the store and the attention back to back.
 *
 *   key, value    [num_tokens][num_kv_heads][head_size], row t = query row t, cache dtype
 *                 (bfloat16 for PA_FP8_E4M3)
 *   slot_mapping  [num_tokens] int32: the cache slot of each row's token
 *   num_tokens    == cu_seqlens_q[num_seqs] (the rows of query, key and value)
 * Other arguments as pa_prefill_varlen.  Precondition (as in the paged layout everywhere):
 * the slot of the new token at key position j of sequence s is the block-table position of
 * j (in particular not negative), so attending the stored cache and attending key/value give
 * the same keys.  Result and cache contents then equal pa_store_kv followed by
 * pa_prefill_varlen.  Outside it, a negative slot leaves its token unstored and the rows that
 * attend that key see the given key/value row (bf16 cache) or the cache's old contents at the
 * key's position (float32 and FP8 caches, which run the store first).
 */
int pa_prefill_varlen_with_store(const pa_cache_desc* cache, void* out, const void* query,
                                 const void* key, const void* value, const int32_t* slot_mapping,
                                 int32_t num_tokens, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                 int32_t max_seqlen_k, int32_t num_heads, float scale,
                                 int32_t sliding_window, const float* alibi_slopes, void* stream);

/*
 * pa_decode_workspace_size — bytes of device workspace pa_decode needs for these sizes
 * (0 when the batch is too small to be split, and for float32 caches).  With
 * partition_size 0 the size depends on how many decode workgroups the current device
 * holds at once; query it on the device that runs the decode.
 */
size_t pa_decode_workspace_size(const pa_cache_desc* cache, int32_t num_seqs,
                                int32_t num_heads, int32_t max_seq_len,
                                int32_t sliding_window, int32_t partition_size);

/*
 * pa_decode — one query token per sequence over its cached keys (split-K + merge).
 *
 * MinivLLM API docs, section paged_attention_decode (query [batch][heads][dim],
 * block_tables, context_lens valid keys per sequence); vLLM learning book section 7
 * (split-KV for long-context decode).  Sequence s attends keys [lo, n) with
 * n = seq_lens[s] (the keys stored so far, the new token's included) and
 * lo = max(0, n - sliding_window) when sliding_window > 0, else 0: the seqlen_q = 1 case
 * of pa_prefill_varlen.  The 32-key steps of all sequences, in order, are cut into equal
 * chunks, one per workgroup; a sequence cut by chunk boundaries leaves a partial softmax
 * state per piece in the workspace, merged afterwards with a log-sum-exp rescale.
 * partition_size 0 = automatic (as many chunks as the device runs at once, of at least
 * 128 keys); otherwise a multiple of 32: chunks of at least that many keys.
 *
 *   out, query   [num_seqs][num_heads][head_size], contiguous, cache dtype
 *   block_table  [num_seqs][max_blocks_per_seq] int32
 *   seq_lens     [num_seqs] int32, each in [0, max_seq_len]
 *   alibi_slopes NULL, or [num_heads] float32 ALiBi slopes (as pa_prefill_varlen, with the
 *                query at position seq_lens[s] - 1)
 *   workspace    16-byte aligned device buffer of >= pa_decode_workspace_size(...) bytes
 *                (may be NULL when that is 0); its contents need no initialisation
 * A sequence with seq_lens[s] == 0 gets a zero output row.
 */
int pa_decode(const pa_cache_desc* cache, void* out, const void* query,
              const int32_t* block_table, int32_t max_blocks_per_seq,
              const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
              int32_t num_heads, float scale, int32_t sliding_window,
              const float* alibi_slopes, int32_t partition_size, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * pa_decode_with_store — pa_store_kv of each sequence's new token, then pa_decode, as one
 * call (same source as pa_prefill_varlen_with_store).  key, value [num_seqs][num_kv_heads]
 * [head_size] and slot_mapping [num_seqs]: the token just produced by each sequence, which
 * seq_lens already counts.  Other arguments as pa_decode.  With a bf16 cache it is one partition
 * launch (plus the merge): the workgroup holding a sequence's last key takes that key's K/V from
 * key/value rather than the cache, and writes the rows to slot_mapping[s].  With a float32 or FP8
 * cache the store kernel runs first, then the decode kernels.  Precondition as
 * pa_prefill_varlen_with_store: slot_mapping[s] is the block-table position of key
 * seq_lens[s] - 1; a sequence with seq_lens[s] == 0 has no new token and takes a negative slot.
 * Outside it, a negative slot leaves the token unstored and the query sees the given row (bf16)
 * or the cache's old contents (float32, FP8).
 */
int pa_decode_with_store(const pa_cache_desc* cache, void* out, const void* query, const void* key,
                         const void* value, const int32_t* slot_mapping, const int32_t* block_table,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t max_seq_len, int32_t num_heads, float scale, int32_t sliding_window,
                         const float* alibi_slopes, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * pa_cascade_decode_workspace_size — bytes of device workspace pa_cascade_decode needs
 * (the split of the own keys as pa_decode_workspace_size, plus the prefix pass's states:
 * num_seqs * num_heads * (head_size + 2) floats per prefix chunk).  0 for float32 caches.
 */
size_t pa_cascade_decode_workspace_size(const pa_cache_desc* cache, int32_t num_seqs,
                                        int32_t num_heads, int32_t max_seq_len,
                                        int32_t common_prefix_len, int32_t partition_size);

/*
 * pa_cascade_decode — decode of a batch whose sequences share their first common_prefix_len
 * keys through the same physical blocks (a prefix-cache hit, such as one system prompt).
 *
 * vLLM learning book, "05. Attention Backends", section 8 (Cascade Attention), the cascade
 * fields of section 4 (use_cascade, common_prefix_len) and self-check question 4: attention
 * over the shared prefix is taken once for all queries of the batch, whose K/V is then read
 * once instead of once per sequence; each sequence then attends only its own keys, and the
 * two parts are combined by log-sum-exp.  The result equals pa_decode without a window or
 * ALiBi (up to rounding).
 *
 *   common_prefix_len  a multiple of block_size, at most max_seq_len; 0 runs pa_decode
 *   (other arguments as pa_decode; bf16 caches only: a float32 cache is PA_ERR_UNSUPPORTED)
 * Preconditions on device data (not checked): every seq_lens[s] >= common_prefix_len, and
 * entries [0, common_prefix_len / block_size) of every block-table row are the same
 * physical blocks; the prefix is read through row 0.
 * Runs the prefix kernel, then the partition (+ merge) kernels of pa_decode on the keys
 * after the prefix, whose first piece of each sequence starts from the prefix's state.
 * When it pays: the saving is the prefix's re-reads, which the device's last-level cache
 * (256 MB) already serves cheaply for short prefixes.  Measured on MI355X (32/8 heads, head
 * size 128, bf16, own keys U[0, 3072]): cascade beats pa_decode for prefixes of 4096 keys
 * from 16 sequences, 2048 keys from 64, 1024 keys only at 256; with 512-key prefixes pa_decode
 * is faster up to 256 sequences.  Both give the same attention, so a caller may pick by that.
 */
int pa_cascade_decode(const pa_cache_desc* cache, void* out, const void* query,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                      int32_t num_heads, float scale, int32_t common_prefix_len,
                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * pa_cascade_prefill_varlen_workspace_size — bytes of device workspace pa_cascade_prefill_varlen
 * needs: the prefix pass's states, num_tokens * num_heads * (head_size + 2) floats per prefix
 * chunk (0 for float32 caches and for common_prefix_len 0).
 */
size_t pa_cascade_prefill_varlen_workspace_size(const pa_cache_desc* cache, int32_t num_tokens,
                                                int32_t num_heads, int32_t common_prefix_len);

/*
 * pa_cascade_prefill_varlen — varlen causal attention (as pa_prefill_varlen, no window) of a
 * batch whose sequences share their first common_prefix_len keys through the same physical
 * blocks, with query chunks of any length (chunked prefill, mixed prefill/decode batches).
 *
 * vLLM learning book, "05. Attention Backends", section 8 (Cascade Attention), the cascade
 * fields of section 4 FlashAttentionMetadata (common_prefix_len, cu_prefix_query_lens,
 * prefix_kv_lens, suffix_kv_lens) and self-check question 4: the shared segment is attended
 * by every query row of the batch together (the prefix's K/V read once for all of them), each
 * sequence's rows then attend its own keys from common_prefix_len on under the causal rule,
 * and the two parts are combined by log-sum-exp.  The result equals pa_prefill_varlen (up to
 * rounding).  Runs the prefix pass (the packed query rows as one block against the prefix),
 * then the prefill kernel over the own keys, folding the prefix states into each row.
 *
 *   common_prefix_len  a multiple of block_size, at most max_seqlen_k; 0 runs pa_prefill_varlen
 *   num_tokens         the packed query rows, == cu_seqlens_q[num_seqs] (sizes the prefix pass)
 *   workspace          16-byte aligned, >= pa_cascade_prefill_varlen_workspace_size(...) bytes;
 *                      contents need no initialisation
 *   (other arguments as pa_prefill_varlen; bf16 or FP8 caches, no ALiBi)
 * Preconditions on device data (not checked): every sequence's first query row sits at or
 * after the prefix's last key (seqlen_k - seqlen_q >= common_prefix_len - 1), and entries
 * [0, common_prefix_len / block_size) of every block-table row are the same physical blocks
 * (the prefix is read through row 0).
 */
int pa_cascade_prefill_varlen(const pa_cache_desc* cache, void* out, const void* query,
                              const int32_t* block_table, int32_t max_blocks_per_seq,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                              int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_heads, float scale,
                              int32_t common_prefix_len, int32_t num_tokens, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * pa_decode_no_alloc — pa_decode with no workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It calls no allocating routine.  The split's partial states go to a
 * scratch array that the library keeps in device memory, PA_DECODE_NO_ALLOC_SCRATCH_BYTES
 * (32 MiB) on each GPU it runs on, held from the library's load on that GPU until the
 * process ends.  Its device address is looked up once per device, on the first call with
 * that device current.
 *
 * Arguments and results as pa_decode (the caller still passes every input and output); the
 * call runs on the current device, which must be the device of the tensors and the stream.
 * Sizes whose split needs more scratch than the maximum (pa_decode_workspace_size(...)
 * > PA_DECODE_NO_ALLOC_SCRATCH_BYTES: e.g. many heads with a small partition_size) return
 * PA_ERR_WORKSPACE before any launch; pa_decode with a caller-owned workspace serves them.
 * Every call on one GPU shares that GPU's array and leaves its contents behind (the kernels
 * need none cleared): calls that overlap on one GPU (concurrent streams, or host threads)
 * race on it and give wrong results, so a caller serialises them.
 */
#define PA_DECODE_NO_ALLOC_SCRATCH_BYTES (32u << 20)
int pa_decode_no_alloc(const pa_cache_desc* cache, void* out, const void* query,
                       const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                       int32_t num_heads, float scale, int32_t sliding_window,
                       const float* alibi_slopes, int32_t partition_size, void* stream);

/* Fixed text for a status code. */
const char* pa_status_string(int status);

/* Detail of the most recent non-OK return on the calling thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
