// mi_attn_kernels.hpp -- kernel argument blocks and host-side launchers (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tile_plan.hpp"

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

// Where one (item, query head)'s rows live and how many there are: the device side of
// plan::item_rows, reading the item's token range or valid length.
__device__ __forceinline__ plan::Rows item_rows(const PrefillArgs& a, int b, int h, int kvh, int D) {
    if (a.cu_seqlens)
        return plan::item_rows(plan::kUnpadded, b, h, kvh, D, a.q_heads, a.kv_heads, a.q_len, a.kv_len,
                               a.cu_seqlens[b], a.cu_seqlens[b + 1], false, 0);
    const plan::Layout lay = a.token_major ? plan::kTokenMajor : plan::kHeadMajor;
    return plan::item_rows(lay, b, h, kvh, D, a.q_heads, a.kv_heads, a.q_len, a.kv_len, 0, 0, a.seq_lens != nullptr,
                           a.seq_lens ? a.seq_lens[b] : 0);
}

// Whether a prefill grid runs its q-tiles last to first (plan::map_block): a causal mask
// puts the most keys into the last tiles, and per-item lengths (padding or unpadded items)
// leave the last tiles only to the longest items.
__device__ __forceinline__ bool last_tiles_first(const PrefillArgs& a) {
    return a.causal != 0 || a.seq_lens != nullptr || a.cu_seqlens != nullptr;
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
    // Elements from one item's queries to the next item's (q_heads * head_dim, or the
    // fused QKV row's length for attn_decode_append_qkv), and from one item's new K/V
    // rows to the next item's (kv_heads * head_dim, or the fused row's length).
    int q_rs, new_rs;
};

// Each launcher enqueues on `stream` and returns the launch status.
hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, hipStream_t stream);
// head dims 32 and 64 (called by launch_prefill_bf16)
hipError_t launch_prefill_bf16_narrow(const PrefillArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, int head_dim, hipStream_t stream);
// dtype: an mi_attn_dtype value (the element format of q, the caches and out)
hipError_t launch_decode(const DecodeArgs& a, int head_dim, int heads_per_group, int dtype,
                         hipStream_t stream);

// Decode launch plan shared by the call and the workspace query (plan::decode_plan with
// the grid target the split kernel is tuned for).
plan::DecodePlan plan_decode(int batch, int q_heads, int kv_heads, int kv_len, int head_dim);

}  // namespace mi_attn
