/*
 * mi_attn.h -- C ABI of libmi_attn: multi-head scaled-dot-product attention on
 * AMD Instinct MI355X (gfx950).
 *
 * Two operations, both computing, for every batch item b, query head h and query
 * row i,
 *
 *     out[b,h,i,:] = sum_{j in J} softmax_J(scale * q[b,h,i,:] . k[b,kh,j,:]) * v[b,kh,j,:]
 *
 * where kh = h / (q_heads / kv_heads) (contiguous groups of query heads share one
 * K/V head) and J is the key set of the row (causal prefix, valid length, window).
 * A row whose key set is empty, or whose query position lies at or past the item's
 * valid length (a padded row), is written as zeros.
 *
 * Sources (docs.rs pages):
 *   - ferrum-kernels 0.8.7, trait `Backend`, Required Methods: `flash_attention`
 *     (q, k, v, out, batch, q_len, kv_len, pos_offset, config) -- the prefill call;
 *     `qk_norm_rope` -- head-major [heads, tokens, head_dim] layout, token i at
 *     position pos_offset + i; `kv_cache_append_head_major` -- cache layout
 *     [kv_heads, capacity, head_dim]; `flash_attention_batched_per_cache` -- the
 *     batched decode call: per-item kv_lens in a device buffer, scale, sliding_window
 *     (0 = full causal, w > 0 = the last w valid positions).
 *   - ripvec-core 0.8.3, trait `Driver`, Required Methods: `fused_scale_mask_softmax`
 *     (softmax(scores * scale + mask) per head), `fused_scale_mask_softmax_windowed`
 *     (|query_pos - key_pos| > window/2 masked), `build_attn_mask` (per-item key
 *     padding), `unpad_from_batch` (padded rows are discarded).
 *   - realizar 0.8.5, `src/gguf/inference/cached/attention.rs`:
 *     `parallel_multihead_attention_gpu_cached` (scale 1/sqrt(head_dim) applied to
 *     the scores before the softmax) and `batched_causal_softmax` (rows normalised
 *     only when their exponential sum is positive).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers to contiguous row-major arrays, 16-byte
 *     aligned.  The caller owns every buffer; the library keeps no pointer after a call
 *     returns and allocates no device memory.
 *   - `dtype` is MI_ATTN_BF16, MI_ATTN_F16 or MI_ATTN_F32 and applies to q, k, v and out
 *     alike (and to the new rows and caches of the decode calls).  bf16 and fp16 inputs
 *     are multiplied on matrix cores with fp32 accumulation; the softmax runs in fp32;
 *     16-bit outputs are rounded to nearest even.  fp16 follows the `_f16` twins of the
 *     ripvec-core `Driver` page (`fused_scale_mask_softmax_f16` and the others: half
 *     storage, fp32 reductions).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue work and
 *     never synchronise; errors raised while the kernels run surface at the caller's
 *     next synchronisation of that stream.
 *   - Return value: a mi_attn_status.  On failure nothing is enqueued and
 *     attn_last_error() holds "<call>: <reason>" for the calling thread.
 *   - head_dim must be 32, 64 or 128 (else MI_ATTN_ERR_UNSUPPORTED; there is no slow
 *     fallback).
 */
#ifndef MI_ATTN_H
#define MI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MI_ATTN_VERSION 7

typedef enum { MI_ATTN_F32 = 0, MI_ATTN_BF16 = 1, MI_ATTN_F16 = 2 } mi_attn_dtype;

typedef enum {
    MI_ATTN_OK = 0,
    MI_ATTN_ERR_INVALID = 1,     /* bad pointer, size, alignment, or relation between sizes */
    MI_ATTN_ERR_UNSUPPORTED = 2, /* valid request the library does not implement           */
    MI_ATTN_ERR_HIP = 3          /* the HIP runtime refused a launch                       */
} mi_attn_status;

/*
 * attn_prefill -- attention of q_len query rows against kv_len keys per (item, head).
 * Follows `flash_attention` of the ferrum-kernels `Backend` page, with the mask kinds
 * of the ripvec-core `Driver` page.
 *
 *   q    [batch, q_heads,  q_len,  head_dim]
 *   k, v [batch, kv_heads, kv_len, head_dim]
 *   out  [batch, q_heads,  q_len,  head_dim]   written in full (padded rows = 0)
 *   q_heads % kv_heads == 0; query head h reads K/V head h / (q_heads / kv_heads).
 *   pos_offset  absolute position of query row 0 (row i sits at pos_offset + i; key j
 *               at position j); requires pos_offset >= 0 and pos_offset + q_len <= kv_len.
 *   seq_lens    NULL, or DEVICE int32 [batch]: valid key count of each item (values are
 *               clamped to [0, kv_len]).  Keys j >= seq_lens[b] are ignored and query
 *               rows at positions >= seq_lens[b] are padding (written as 0).  Values
 *               past the valid length may be anything, NaN included.
 *   window      0: no band.  causal != 0: a query at p sees keys p - window < j <= p.
 *               causal == 0: a query at p sees keys with |p - j| <= window / 2.
 *   causal      nonzero: keys j > p are masked.
 *   scale       multiplies q.k before the softmax, used exactly as given (1/sqrt(head_dim)
 *               is the usual value).
 *   batch == 0 or q_len == 0 is a valid empty call (nothing is enqueued).
 */
int attn_prefill(const void* q, const void* k, const void* v, void* out, int batch, int q_heads,
                 int kv_heads, int q_len, int kv_len, int head_dim, int pos_offset,
                 const int32_t* seq_lens, int window, int causal, float scale, int dtype,
                 void* stream);

/*
 * attn_prefill_token_major -- attn_prefill with every tensor token-major: the layout
 * the heads come in from the QKV projection and go out in to the output projection.
 * On the ferrum-kernels `Backend` page, `flash_attention` sits between two layout
 * conversions: `qk_norm_rope` (Required Methods) turns token-major [tokens, heads,
 * head_dim] inputs head-major, and `transpose_head_to_token` (Required Methods) turns the
 * head-major output back token-major for the output projection; the ripvec-core
 * `Driver` page's `attn_reshape` does the latter for [batch, num_heads, seq, head_dim].
 * This call reads and writes the token-major tensors in place, so neither conversion
 * exists.
 *
 *   q, out  [batch, q_len,  q_heads,  head_dim]
 *   k, v    [batch, kv_len, kv_heads, head_dim]
 *   Every other argument, and every rule, is attn_prefill's.
 */
int attn_prefill_token_major(const void* q, const void* k, const void* v, void* out, int batch, int q_heads,
                             int kv_heads, int q_len, int kv_len, int head_dim, int pos_offset,
                             const int32_t* seq_lens, int window, int causal, float scale, int dtype,
                             void* stream);

/*
 * attn_prefill_varlen -- attn_prefill on an unpadded batch: the items' tokens are
 * concatenated, token-major, with cu_seqlens marking the item boundaries.  Follows
 * `prepare_batch_unpadded` of the ripvec-core `Driver` page (tokens concatenated flat,
 * cu_seqlens for the attention boundaries) and reads and writes the [tokens, hidden]
 * layout directly, where the pages pad around the per-head products and transpose
 * afterwards (`fused_pad_qkv_split_f16`, `fused_reshape_unpad_f16`; ferrum-kernels
 * `Backend`, `transpose_head_to_token`).  Keys are the item's own tokens (self-attention,
 * query i of an item at position i).
 *
 *   q, out     [tokens, q_heads,  head_dim]   token-major: row t is token t's hidden vector
 *   k, v       [tokens, kv_heads, head_dim]
 *   cu_seqlens DEVICE int32 [batch + 1]: item b is tokens [cu_seqlens[b], cu_seqlens[b+1]).
 *              Must be non-decreasing from cu_seqlens[0] >= 0, with cu_seqlens[batch] <=
 *              tokens; an item of length 0 is empty.  The host does not read it.
 *   max_seqlen the longest item (sizes the launch).  An item longer than that is treated
 *              as its first max_seqlen tokens; its later rows of out are not written.
 *   window, causal, scale, dtype as for attn_prefill.  Rows of out between items' tokens
 *   do not exist: every token row of an item is written.
 *   batch == 0 or max_seqlen == 0 is a valid empty call.
 */
int attn_prefill_varlen(const void* q, const void* k, const void* v, void* out, const int32_t* cu_seqlens,
                        int batch, int max_seqlen, int q_heads, int kv_heads, int head_dim, int window, int causal,
                        float scale, int dtype, void* stream);

/*
 * attn_decode -- one query token per (item, query head) against a head-major KV cache.
 * Follows `flash_attention_batched_per_cache` and `kv_cache_append_head_major` of the
 * ferrum-kernels `Backend` page, with the per-item caches stacked in one allocation.
 *
 *   q        [batch, q_heads, head_dim]
 *   k_cache  [batch, kv_heads, capacity, head_dim]  slots [0, kv_len) hold keys
 *   v_cache  [batch, kv_heads, capacity, head_dim]
 *   out      [batch, q_heads, head_dim]
 *   1 <= kv_len <= capacity.  Slots at or past an item's length are never read.
 *   kv_lens  NULL: every item has kv_len keys and its query sits at pos_offset
 *            (0 <= pos_offset < kv_len), seeing keys j <= pos_offset.
 *            DEVICE int32 [batch]: item b has kv_lens[b] keys (clamped to [0, kv_len])
 *            and its query sits at kv_lens[b] - 1 (pos_offset is then unused); an item
 *            with no keys gets zeros.  kv_len is the largest length any item may have.
 *   window   0: all causal keys; w > 0: only the last w positions p - w < j <= p.
 *   workspace, workspace_bytes  DEVICE scratch of at least
 *            attn_decode_workspace_bytes(batch, q_heads, kv_heads, kv_len, head_dim)
 *            bytes, 16-byte aligned (else MI_ATTN_ERR_INVALID), not used by anything else
 *            until the call's kernels finish (the call holds partial softmax states in it).
 *            May be NULL when that size is 0.
 *   batch == 0 is a valid empty call.
 */
int attn_decode(const void* q, const void* k_cache, const void* v_cache, void* out, int batch,
                int q_heads, int kv_heads, int kv_len, int capacity, int head_dim, int pos_offset,
                const int32_t* kv_lens, int window, float scale, int dtype, void* workspace,
                size_t workspace_bytes, void* stream);

/* Bytes of the device scratch attn_decode_noalloc keeps per GPU. */
#define MI_ATTN_NOALLOC_SCRATCH_BYTES (4u << 20)

/*
 * attn_decode_noalloc -- attn_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call allocates nothing (no hipMalloc, no
 * allocating library routine).  The split decode's partial states go to a scratch array
 * of MI_ATTN_NOALLOC_SCRATCH_BYTES the library holds in device memory, one per GPU, from
 * the library's load until the process ends; its device address is looked up once per
 * GPU, on the first call with that GPU current (a host-side symbol query, no stream work).
 *
 *   Every argument and rule is attn_decode's, on the current device.  Sizes whose
 *   partial states need more than the scratch holds (attn_decode_workspace_bytes >
 *   MI_ATTN_NOALLOC_SCRATCH_BYTES) are refused with MI_ATTN_ERR_UNSUPPORTED.
 *   Every call on one GPU uses that GPU's one scratch array, which keeps the last call's
 *   partial states (nothing in it needs to start at zero).  Calls on one stream are
 *   ordered; calls whose kernels overlap on one GPU (different streams) race on it.
 */
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, int batch,
                        int q_heads, int kv_heads, int kv_len, int capacity, int head_dim, int pos_offset,
                        const int32_t* kv_lens, int window, float scale, int dtype, void* stream);

/*
 * attn_decode_per_cache -- attn_decode over one separately allocated cache per item.
 * Follows `flash_attention_batched_per_cache` of the ferrum-kernels `Backend` page
 * (Provided Methods): M decode caches, each [kv_heads, capacity, head_dim] head-major,
 * attended in one launch, with per-item lengths in a device buffer and a common
 * sliding window.
 *
 *   q         [batch, q_heads, head_dim]
 *   k_caches  DEVICE array of `batch` DEVICE pointers (8-byte aligned array); entry b
 *             points at item b's K cache [kv_heads, capacity, head_dim], 16-byte aligned
 *   v_caches  the same for V
 *   out       [batch, q_heads, head_dim]
 *   kv_lens   DEVICE int32 [batch], required: item b has kv_lens[b] keys (clamped to
 *             [0, capacity]) in slots [0, kv_lens[b]) and its query sits at
 *             kv_lens[b] - 1; an item with no keys gets zeros.
 *   window    0: all causal keys; w > 0: only the last w positions.
 *   workspace as for attn_decode, sized attn_decode_workspace_bytes(batch, q_heads,
 *             kv_heads, capacity, head_dim).
 *   The pointed-to caches are read only.  The pointer arrays, the caches and kv_lens
 *   are device memory the host does not inspect: a wrong pointer in them faults on the
 *   device, it is not reported by the call.
 */
int attn_decode_per_cache(const void* q, const void* const* k_caches, const void* const* v_caches, void* out,
                          int batch, int q_heads, int kv_heads, int capacity, int head_dim,
                          const int32_t* kv_lens, int window, float scale, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * attn_decode_append -- append the new token's K and V rows to each item's cache, then
 * attend its query over the cache including them, in one launch.  Fuses
 * `kv_cache_append_batched_per_cache` (each item's head-major row goes into its own
 * cache at the offset read from cache_lens[i]) with `flash_attention_batched_per_cache`
 * of the ferrum-kernels `Backend` page; `split_qkv_norm_rope_into_cache` on the same
 * page is the same idea of dropping the separate append dispatch.
 *
 *   q           [batch, q_heads, head_dim]  the new token's queries
 *   k_new, v_new [batch, kv_heads, head_dim] the new token's keys and values
 *   k_caches, v_caches  DEVICE arrays of `batch` DEVICE pointers to item caches
 *               [kv_heads, capacity, head_dim]; slot cache_lens[b] of every kv head of
 *               item b is overwritten with the new row, nothing else is written.
 *   cache_lens  DEVICE int32 [batch], required: the number of tokens already in each
 *               cache (the caller owns this bookkeeping and advances it after the call).
 *               Item b's query sits at position cache_lens[b] and sees the keys
 *               [0, cache_lens[b]] (the new one included), or the last `window` of them.
 *               An item with no room (cache_lens[b] < 0 or >= capacity) is left
 *               untouched and gets zeros.
 *   out, window, scale, dtype, workspace as for attn_decode_per_cache.
 *   Two items must not share a cache.  The caller must not read or write the caches
 *   until the call's kernels finish.
 */
int attn_decode_append(const void* q, const void* k_new, const void* v_new, void* const* k_caches,
                       void* const* v_caches, void* out, int batch, int q_heads, int kv_heads, int capacity,
                       int head_dim, const int32_t* cache_lens, int window, float scale, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_append_qkv -- attn_decode_append reading the new token's query, key and
 * value from one fused row per item, as a fused QKV projection writes it.  The row layout
 * is that of `split_qkv` on the ferrum-kernels `Backend` page (Required Methods): per
 * token [q_dim + 2 * kv_dim] with q_dim = q_heads * head_dim and kv_dim = kv_heads *
 * head_dim, the query heads first, then the key heads, then the value heads;
 * `split_qkv_norm_rope_into_cache` (Provided Methods) on the same page consumes such a
 * row and writes its K/V straight into the cache.  Here the row's parts enter as given:
 * a caller that normalises or rotates q and k does so before the call.
 *
 *   qkv         [batch, q_heads + 2 * kv_heads, head_dim], 16-byte aligned: item b's row
 *               holds its q heads, then its kv_heads key rows, then its kv_heads value rows
 *   k_caches, v_caches, out, batch, q_heads, kv_heads, capacity, head_dim, cache_lens,
 *   window, scale, dtype, workspace: as for attn_decode_append (the workspace query is the
 *   same).  Errors as for attn_decode_append; a null qkv with batch > 0 is
 *   MI_ATTN_ERR_INVALID.
 */
int attn_decode_append_qkv(const void* qkv, void* const* k_caches, void* const* v_caches, void* out, int batch,
                           int q_heads, int kv_heads, int capacity, int head_dim, const int32_t* cache_lens,
                           int window, float scale, int dtype, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Scratch bytes attn_decode needs for these sizes (0 when it needs none): the split
 * decode's partial states [batch, q_heads, splits, head_dim + 2] fp32 when the launch plan
 * cuts each key range into splits.  The caller allocates them, as the pages' backends
 * leave allocation to the caller (ripvec-core `Driver` page: drivers handle memory
 * allocation; ferrum-kernels `Backend` page, `flash_attention_batched_per_cache`: the
 * caller owns the buffers).  kv_heads is an argument because the plan splits per
 * (item, kv head).  Pure host function; returns 0 for sizes attn_decode would reject.
 * For attn_decode_per_cache and attn_decode_append pass capacity as kv_len. */
size_t attn_decode_workspace_bytes(int batch, int q_heads, int kv_heads, int kv_len, int head_dim);

/* Message of the calling thread's last failed call ("" if none), "<call>: <reason>":
 * the operation and why it was refused, after realizar `cached/attention.rs`, whose
 * GPU paths fail with `UnsupportedOperation { operation, reason }`, and the `Result`
 * errors of the ripvec-core `Driver` and ferrum-kernels `Backend` methods.  The pointer
 * stays valid until that thread's next call into the library. */
const char* attn_last_error(void);

/* MI_ATTN_VERSION of the built library. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MI_ATTN_H */
