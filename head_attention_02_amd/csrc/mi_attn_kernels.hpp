// mi_attn_kernels.hpp -- kernel argument blocks and host-side launchers (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mi_attn {

// One prefill problem, as validated by attn_prefill or attn_prefill_varlen.
struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    const int32_t* seq_lens;  // device [batch] or nullptr
    // Unpadded (varlen) layout: device [batch + 1] token offsets; q and out are then
    // [tokens, q_heads, D] and k, v [tokens, kv_heads, D] (token-major), item b holds
    // tokens [cu_seqlens[b], cu_seqlens[b+1]) and q_len is the longest item.  nullptr:
    // the padded head-major layout [batch, heads, len, D].
    const int32_t* cu_seqlens;
    int batch, q_heads, kv_heads, q_len, kv_len;
    int pos_offset, window, causal;
    float scale;
    int n_qtiles;             // grid.x
    int f16;                  // 16-bit inputs: 0 = bf16, 1 = fp16 (matrix-core kernels)
    // Padded layout only: 1 = token-major, q and out [batch, q_len, q_heads, D] and k, v
    // [batch, kv_len, kv_heads, D]; 0 = head-major [batch, heads, len, D].
    int token_major;
};

// Where one (item, query head)'s rows live and how many there are (element offsets and
// strides; the same code serves both layouts).
struct ItemRows {
    size_t q_base;    // row 0 of (item, query head) in q and out
    size_t kv_base;   // row 0 of (item, kv head) in k and v
    int q_rs, kv_rs;  // elements from one row to the next
    int q_len;        // query rows of the item
    int kv_valid;     // keys of the item (seq_lens applied)
};

__device__ __forceinline__ ItemRows item_rows(const PrefillArgs& a, int b, int h, int kvh, int D) {
    ItemRows r;
    if (a.cu_seqlens) {
        const int t0 = a.cu_seqlens[b];
        const int n = min(max(a.cu_seqlens[b + 1] - t0, 0), a.q_len);
        r.q_rs = a.q_heads * D;
        r.kv_rs = a.kv_heads * D;
        r.q_base = (size_t)t0 * r.q_rs + (size_t)h * D;
        r.kv_base = (size_t)t0 * r.kv_rs + (size_t)kvh * D;
        r.q_len = n;
        r.kv_valid = n;
    } else if (a.token_major) {
        r.q_rs = a.q_heads * D;
        r.kv_rs = a.kv_heads * D;
        r.q_base = (size_t)b * a.q_len * r.q_rs + (size_t)h * D;
        r.kv_base = (size_t)b * a.kv_len * r.kv_rs + (size_t)kvh * D;
        r.q_len = a.q_len;
        r.kv_valid = a.seq_lens ? min(max(a.seq_lens[b], 0), a.kv_len) : a.kv_len;
    } else {
        r.q_rs = D;
        r.kv_rs = D;
        r.q_base = ((size_t)b * a.q_heads + h) * (size_t)a.q_len * D;
        r.kv_base = ((size_t)b * a.kv_heads + kvh) * (size_t)a.kv_len * D;
        r.q_len = a.q_len;
        r.kv_valid = a.seq_lens ? min(max(a.seq_lens[b], 0), a.kv_len) : a.kv_len;
    }
    return r;
}

// One decode problem, as validated and planned by attn_decode.
struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* ws;                // [batch, q_heads, splits, head_dim + 2] partial states
    const int32_t* kv_lens;   // device [batch] or nullptr
    int batch, q_heads, kv_heads, kv_len, capacity;
    int pos_offset, window;
    float scale;
    int splits, split_len;    // key-range split of each (item, kv head)
    int head_groups;          // query-head groups per kv head (grid.y = kv_heads * head_groups)
    // Per-item caches (attn_decode_per_cache, attn_decode_append): device arrays of
    // `batch` pointers, each to one item's [kv_heads, capacity, head_dim] cache; k and v
    // are then unused.  nullptr: the stacked caches k, v.
    const void* const* k_ptrs;
    const void* const* v_ptrs;
    // attn_decode_append: the new token's rows [batch, kv_heads, head_dim]; kv_lens then
    // holds the cache lengths before the append.  nullptr: no append.
    const void* k_new;
    const void* v_new;
};

// Each launcher enqueues on `stream` and returns the launch status.
hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, hipStream_t stream);
// head dims 32 and 64 (called by launch_prefill_bf16)
hipError_t launch_prefill_bf16_narrow(const PrefillArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, int head_dim, hipStream_t stream);
// dtype: an mi_attn_dtype value (the element format of q, the caches and out)
hipError_t launch_decode(const DecodeArgs& a, int head_dim, int heads_per_group, int dtype,
                         hipStream_t stream);

// Decode launch plan shared by the call and the workspace query.
struct DecodePlan {
    int splits, split_len, heads_per_group, head_groups;
};
DecodePlan plan_decode(int batch, int q_heads, int kv_heads, int kv_len, int head_dim);

}  // namespace mi_attn
