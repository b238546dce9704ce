// abi.hip -- the extern "C" entry points of libmi_attn: argument validation, launch
// planning and dispatch to the gfx950 kernels.  Declarations and their documentation
// are in include/mi_attn.h.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>
#include <mutex>

#include "mi_attn.h"
#include "mi_attn_kernels.hpp"

namespace {

thread_local char g_error[512];

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return status;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool supported_head_dim(int d) { return d == 32 || d == 64 || d == 128; }

}  // namespace

namespace {

int prefill_padded(const char* fn, int token_major, const void* q, const void* k, const void* v, void* out,
                   int batch, int q_heads, int kv_heads, int q_len, int kv_len, int head_dim, int pos_offset,
                   const int32_t* seq_lens, int window, int causal, float scale, int dtype, void* stream) {
    g_error[0] = '\0';
    if (dtype != MI_ATTN_BF16 && dtype != MI_ATTN_F32 && dtype != MI_ATTN_F16)
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
    if (batch < 0 || q_len < 0 || kv_len < 0)
        return fail(MI_ATTN_ERR_INVALID, "%s: negative size (batch %d, q_len %d, kv_len %d)", fn, batch,
                    q_len, kv_len);
    if (q_heads < 1 || kv_heads < 1)
        return fail(MI_ATTN_ERR_INVALID, "%s: q_heads (%d) and kv_heads (%d) must be >= 1", fn, q_heads,
                    kv_heads);
    if (q_heads % kv_heads != 0)
        return fail(MI_ATTN_ERR_INVALID, "%s: q_heads (%d) is not a multiple of kv_heads (%d)", fn, q_heads,
                    kv_heads);
    if (pos_offset < 0 || (long)pos_offset + q_len > kv_len)
        return fail(MI_ATTN_ERR_INVALID, "%s: pos_offset (%d) + q_len (%d) exceeds kv_len (%d)", fn,
                    pos_offset, q_len, kv_len);
    if (window < 0) return fail(MI_ATTN_ERR_INVALID, "%s: window (%d) is negative", fn, window);
    if (!std::isfinite(scale)) return fail(MI_ATTN_ERR_INVALID, "%s: scale is not finite", fn);
    if (!supported_head_dim(head_dim))
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: head_dim %d is not one of 32, 64, 128", fn, head_dim);
    if (batch == 0 || q_len == 0) return MI_ATTN_OK;
    if (!q || !k || !v || !out) return fail(MI_ATTN_ERR_INVALID, "%s: null tensor pointer", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(MI_ATTN_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
    if (seq_lens && ((uintptr_t)seq_lens & 3u))
        return fail(MI_ATTN_ERR_INVALID, "%s: seq_lens must be 4-byte aligned", fn);
    if ((long)q_heads > 65535 || (long)batch > 65535)
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: q_heads and batch must be <= 65535", fn);

    mi_attn::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.seq_lens = seq_lens;
    a.batch = batch;
    a.q_heads = q_heads;
    a.kv_heads = kv_heads;
    a.q_len = q_len;
    a.kv_len = kv_len;
    a.pos_offset = pos_offset;
    a.window = window;
    a.causal = causal ? 1 : 0;
    a.scale = scale;
    a.token_major = token_major;
    hipStream_t s = (hipStream_t)stream;
    a.f16 = dtype == MI_ATTN_F16;
    hipError_t e = dtype != MI_ATTN_F32 ? mi_attn::launch_prefill_bf16(a, head_dim, s)
                                        : mi_attn::launch_prefill_f32(a, head_dim, s);
    if (e != hipSuccess) return fail(MI_ATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return MI_ATTN_OK;
}


// ---- the no-allocation decode's scratch ----------------------------------------------------
//
// Device memory for the split decode's partial states, in the library's code object: each
// GPU the library runs on holds its own copy from the code object's load until the process
// ends, so attn_decode_noalloc allocates nothing.  In host code `scratch` names only a
// host-side stand-in; its device address on the current GPU comes from
// hipGetSymbolAddress, once per device, and only that address reaches the kernels.  The
// split kernel writes every partial state it covers before the combine pass reads it, so
// nothing in the scratch has to start at zero.
constexpr size_t kScratchBytes = MI_ATTN_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

int scratch_for_current_device(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MI_ATTN_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: device %d is past the %d devices the library tracks", fn, dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MI_ATTN_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed: %s", fn,
                        hipGetErrorString(e));
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return MI_ATTN_OK;
}

}  // namespace

extern "C" {

int attn_version(void) { return MI_ATTN_VERSION; }

const char* attn_last_error(void) { return g_error; }


int attn_prefill(const void* q, const void* k, const void* v, void* out, int batch, int q_heads,
                 int kv_heads, int q_len, int kv_len, int head_dim, int pos_offset,
                 const int32_t* seq_lens, int window, int causal, float scale, int dtype,
                 void* stream) {
    return prefill_padded("attn_prefill", 0, q, k, v, out, batch, q_heads, kv_heads, q_len, kv_len, head_dim,
                          pos_offset, seq_lens, window, causal, scale, dtype, stream);
}

int attn_prefill_token_major(const void* q, const void* k, const void* v, void* out, int batch, int q_heads,
                             int kv_heads, int q_len, int kv_len, int head_dim, int pos_offset,
                             const int32_t* seq_lens, int window, int causal, float scale, int dtype,
                             void* stream) {
    return prefill_padded("attn_prefill_token_major", 1, q, k, v, out, batch, q_heads, kv_heads, q_len, kv_len,
                          head_dim, pos_offset, seq_lens, window, causal, scale, dtype, stream);
}

int attn_prefill_varlen(const void* q, const void* k, const void* v, void* out, const int32_t* cu_seqlens,
                        int batch, int max_seqlen, int q_heads, int kv_heads, int head_dim, int window, int causal,
                        float scale, int dtype, void* stream) {
    g_error[0] = '\0';
    const char* fn = "attn_prefill_varlen";
    if (dtype != MI_ATTN_BF16 && dtype != MI_ATTN_F32 && dtype != MI_ATTN_F16)
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
    if (batch < 0 || max_seqlen < 0)
        return fail(MI_ATTN_ERR_INVALID, "%s: negative size (batch %d, max_seqlen %d)", fn, batch, max_seqlen);
    if (q_heads < 1 || kv_heads < 1)
        return fail(MI_ATTN_ERR_INVALID, "%s: q_heads (%d) and kv_heads (%d) must be >= 1", fn, q_heads,
                    kv_heads);
    if (q_heads % kv_heads != 0)
        return fail(MI_ATTN_ERR_INVALID, "%s: q_heads (%d) is not a multiple of kv_heads (%d)", fn, q_heads,
                    kv_heads);
    if (window < 0) return fail(MI_ATTN_ERR_INVALID, "%s: window (%d) is negative", fn, window);
    if (!std::isfinite(scale)) return fail(MI_ATTN_ERR_INVALID, "%s: scale is not finite", fn);
    if (!supported_head_dim(head_dim))
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: head_dim %d is not one of 32, 64, 128", fn, head_dim);
    if (batch == 0 || max_seqlen == 0) return MI_ATTN_OK;
    if (!q || !k || !v || !out || !cu_seqlens) return fail(MI_ATTN_ERR_INVALID, "%s: null pointer argument", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(MI_ATTN_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
    if ((uintptr_t)cu_seqlens & 3u) return fail(MI_ATTN_ERR_INVALID, "%s: cu_seqlens must be 4-byte aligned", fn);
    if ((long)q_heads > 65535 || (long)batch > 65535)
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: q_heads and batch must be <= 65535", fn);

    mi_attn::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.cu_seqlens = cu_seqlens;
    a.batch = batch;
    a.q_heads = q_heads;
    a.kv_heads = kv_heads;
    a.q_len = max_seqlen;
    a.kv_len = max_seqlen;
    a.pos_offset = 0;
    a.window = window;
    a.causal = causal ? 1 : 0;
    a.scale = scale;
    hipStream_t s = (hipStream_t)stream;
    a.f16 = dtype == MI_ATTN_F16;
    hipError_t e = dtype != MI_ATTN_F32 ? mi_attn::launch_prefill_bf16(a, head_dim, s)
                                        : mi_attn::launch_prefill_f32(a, head_dim, s);
    if (e != hipSuccess) return fail(MI_ATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return MI_ATTN_OK;
}

size_t attn_decode_workspace_bytes(int batch, int q_heads, int kv_heads, int kv_len, int head_dim) {
    if (batch <= 0 || q_heads < 1 || kv_heads < 1 || q_heads % kv_heads || kv_len < 1 ||
        !supported_head_dim(head_dim))
        return 0;
    const mi_attn::plan::DecodePlan p = mi_attn::plan_decode(batch, q_heads, kv_heads, kv_len, head_dim);
    if (p.splits == 1) return 0;   // one workgroup per key range writes the output itself
    return (size_t)batch * q_heads * p.splits * (head_dim + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// attn_decode and attn_decode_noalloc.  noalloc: the workspace is the library's scratch
// array on the current device instead of the caller's.
int decode_stacked(const char* fn, const void* q, const void* k_cache, const void* v_cache, void* out, int batch,
                   int q_heads, int kv_heads, int kv_len, int capacity, int head_dim, int pos_offset,
                   const int32_t* kv_lens, int window, float scale, int dtype, void* workspace,
                   size_t workspace_bytes, bool noalloc, void* stream) {
    g_error[0] = '\0';
    if (dtype != MI_ATTN_BF16 && dtype != MI_ATTN_F32 && dtype != MI_ATTN_F16)
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
    if (batch < 0) return fail(MI_ATTN_ERR_INVALID, "%s: negative batch (%d)", fn, batch);
    if (q_heads < 1 || kv_heads < 1)
        return fail(MI_ATTN_ERR_INVALID, "%s: q_heads (%d) and kv_heads (%d) must be >= 1", fn, q_heads,
                    kv_heads);
    if (q_heads % kv_heads != 0)
        return fail(MI_ATTN_ERR_INVALID, "%s: q_heads (%d) is not a multiple of kv_heads (%d)", fn, q_heads,
                    kv_heads);
    if (kv_len < 1 || kv_len > capacity)
        return fail(MI_ATTN_ERR_INVALID, "%s: need 1 <= kv_len (%d) <= capacity (%d)", fn, kv_len, capacity);
    if (!kv_lens && (pos_offset < 0 || pos_offset >= kv_len))
        return fail(MI_ATTN_ERR_INVALID, "%s: pos_offset (%d) must lie in [0, kv_len %d)", fn, pos_offset,
                    kv_len);
    if (window < 0) return fail(MI_ATTN_ERR_INVALID, "%s: window (%d) is negative", fn, window);
    if (!std::isfinite(scale)) return fail(MI_ATTN_ERR_INVALID, "%s: scale is not finite", fn);
    if (!supported_head_dim(head_dim))
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: head_dim %d is not one of 32, 64, 128", fn, head_dim);
    if (batch == 0) return MI_ATTN_OK;
    if (!q || !k_cache || !v_cache || !out) return fail(MI_ATTN_ERR_INVALID, "%s: null tensor pointer", fn);
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(MI_ATTN_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
    if (kv_lens && ((uintptr_t)kv_lens & 3u))
        return fail(MI_ATTN_ERR_INVALID, "%s: kv_lens must be 4-byte aligned", fn);
    if ((long)batch > 65535 || (long)q_heads > 65535)
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: q_heads and batch must be <= 65535", fn);
    const size_t need = attn_decode_workspace_bytes(batch, q_heads, kv_heads, kv_len, head_dim);
    if (noalloc) {
        if (need > kScratchBytes)
            return fail(MI_ATTN_ERR_UNSUPPORTED,
                        "%s: these sizes need %zu bytes of split-decode scratch, more than the %zu bytes the "
                        "library's no-allocation scratch holds (use attn_decode with a workspace)",
                        fn, need, kScratchBytes);
        const int st = scratch_for_current_device(fn, &workspace);
        if (st != MI_ATTN_OK) return st;
        workspace_bytes = kScratchBytes;
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(MI_ATTN_ERR_INVALID, "%s: workspace of %zu bytes given, %zu needed", fn, workspace_bytes,
                    need);
    if (!aligned16(workspace)) return fail(MI_ATTN_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);

    const mi_attn::plan::DecodePlan p = mi_attn::plan_decode(batch, q_heads, kv_heads, kv_len, head_dim);
    mi_attn::DecodeArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.ws = (float*)workspace;
    a.kv_lens = kv_lens;
    a.batch = batch;
    a.q_heads = q_heads;
    a.kv_heads = kv_heads;
    a.kv_len = kv_len;
    a.capacity = capacity;
    a.pos_offset = pos_offset;
    a.window = window;
    a.scale = scale;
    a.splits = p.splits;
    a.split_len = p.split_len;
    a.head_groups = p.head_groups;
    a.q_rs = q_heads * head_dim;
    a.new_rs = kv_heads * head_dim;
    hipError_t e = mi_attn::launch_decode(a, head_dim, p.heads_per_group, dtype,
                                          (hipStream_t)stream);
    if (e != hipSuccess) return fail(MI_ATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return MI_ATTN_OK;
}

}  // namespace

extern "C" {


int attn_decode(const void* q, const void* k_cache, const void* v_cache, void* out, int batch,
                int q_heads, int kv_heads, int kv_len, int capacity, int head_dim, int pos_offset,
                const int32_t* kv_lens, int window, float scale, int dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
    return decode_stacked("attn_decode", q, k_cache, v_cache, out, batch, q_heads, kv_heads, kv_len, capacity,
                          head_dim, pos_offset, kv_lens, window, scale, dtype, workspace, workspace_bytes, false,
                          stream);
}

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, int batch,
                        int q_heads, int kv_heads, int kv_len, int capacity, int head_dim, int pos_offset,
                        const int32_t* kv_lens, int window, float scale, int dtype, void* stream) {
    return decode_stacked("attn_decode_noalloc", q, k_cache, v_cache, out, batch, q_heads, kv_heads, kv_len,
                          capacity, head_dim, pos_offset, kv_lens, window, scale, dtype, nullptr, 0, true, stream);
}

}  // extern "C"

namespace {

// Shared checks and launch of the per-item-cache decode calls.
// fused_rs > 0: q, k_new and v_new are the parts of one fused row per item of fused_rs
// elements (attn_decode_append_qkv); 0: the separate [batch, heads, head_dim] tensors.
int decode_per_item(const char* fn, const void* q, const void* const* k_caches, const void* const* v_caches,
                    const void* k_new, const void* v_new, void* out, int batch, int q_heads, int kv_heads,
                    int capacity, int head_dim, const int32_t* lens, int window, float scale, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream, int fused_rs = 0) {
    g_error[0] = '\0';
    if (dtype != MI_ATTN_BF16 && dtype != MI_ATTN_F32 && dtype != MI_ATTN_F16)
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
    if (batch < 0) return fail(MI_ATTN_ERR_INVALID, "%s: negative batch (%d)", fn, batch);
    if (q_heads < 1 || kv_heads < 1)
        return fail(MI_ATTN_ERR_INVALID, "%s: q_heads (%d) and kv_heads (%d) must be >= 1", fn, q_heads,
                    kv_heads);
    if (q_heads % kv_heads != 0)
        return fail(MI_ATTN_ERR_INVALID, "%s: q_heads (%d) is not a multiple of kv_heads (%d)", fn, q_heads,
                    kv_heads);
    if (capacity < 1) return fail(MI_ATTN_ERR_INVALID, "%s: capacity (%d) must be >= 1", fn, capacity);
    if (window < 0) return fail(MI_ATTN_ERR_INVALID, "%s: window (%d) is negative", fn, window);
    if (!std::isfinite(scale)) return fail(MI_ATTN_ERR_INVALID, "%s: scale is not finite", fn);
    if (!supported_head_dim(head_dim))
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: head_dim %d is not one of 32, 64, 128", fn, head_dim);
    if (batch == 0) return MI_ATTN_OK;
    if (!q || !k_caches || !v_caches || !out || !lens)
        return fail(MI_ATTN_ERR_INVALID, "%s: null pointer argument", fn);
    if (k_new && (!v_new || !aligned16(k_new) || !aligned16(v_new)))
        return fail(MI_ATTN_ERR_INVALID, "%s: new K/V rows must both be given, 16-byte aligned", fn);
    if (!aligned16(q) || !aligned16(out))
        return fail(MI_ATTN_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
    if (((uintptr_t)k_caches & 7u) || ((uintptr_t)v_caches & 7u) || ((uintptr_t)lens & 3u))
        return fail(MI_ATTN_ERR_INVALID, "%s: pointer arrays must be 8-byte and lengths 4-byte aligned", fn);
    if ((long)batch > 65535 || (long)q_heads > 65535)
        return fail(MI_ATTN_ERR_UNSUPPORTED, "%s: q_heads and batch must be <= 65535", fn);
    const size_t need = attn_decode_workspace_bytes(batch, q_heads, kv_heads, capacity, head_dim);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(MI_ATTN_ERR_INVALID, "%s: workspace of %zu bytes given, %zu needed", fn, workspace_bytes,
                    need);
    if (!aligned16(workspace)) return fail(MI_ATTN_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);

    const mi_attn::plan::DecodePlan p = mi_attn::plan_decode(batch, q_heads, kv_heads, capacity, head_dim);
    mi_attn::DecodeArgs a{};
    a.q = q;
    a.k_ptrs = k_caches;
    a.v_ptrs = v_caches;
    a.k_new = k_new;
    a.v_new = v_new;
    a.out = out;
    a.ws = (float*)workspace;
    a.kv_lens = lens;
    a.batch = batch;
    a.q_heads = q_heads;
    a.kv_heads = kv_heads;
    a.kv_len = capacity;
    a.capacity = capacity;
    a.window = window;
    a.scale = scale;
    a.splits = p.splits;
    a.split_len = p.split_len;
    a.head_groups = p.head_groups;
    a.q_rs = fused_rs > 0 ? fused_rs : q_heads * head_dim;
    a.new_rs = fused_rs > 0 ? fused_rs : kv_heads * head_dim;
    hipError_t e = mi_attn::launch_decode(a, head_dim, p.heads_per_group, dtype,
                                          (hipStream_t)stream);
    if (e != hipSuccess) return fail(MI_ATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return MI_ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_per_cache(const void* q, const void* const* k_caches, const void* const* v_caches, void* out,
                          int batch, int q_heads, int kv_heads, int capacity, int head_dim,
                          const int32_t* kv_lens, int window, float scale, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return decode_per_item("attn_decode_per_cache", q, k_caches, v_caches, nullptr, nullptr, out, batch, q_heads,
                           kv_heads, capacity, head_dim, kv_lens, window, scale, dtype, workspace,
                           workspace_bytes, stream);
}

int attn_decode_append(const void* q, const void* k_new, const void* v_new, void* const* k_caches,
                       void* const* v_caches, void* out, int batch, int q_heads, int kv_heads, int capacity,
                       int head_dim, const int32_t* cache_lens, int window, float scale, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
    if (batch > 0 && (!k_new || !v_new)) {
        g_error[0] = '\0';
        return fail(MI_ATTN_ERR_INVALID, "attn_decode_append: null new K/V rows");
    }
    return decode_per_item("attn_decode_append", q, (const void* const*)k_caches, (const void* const*)v_caches,
                           k_new, v_new, out, batch, q_heads, kv_heads, capacity, head_dim, cache_lens, window,
                           scale, dtype, workspace, workspace_bytes, stream);
}

int attn_decode_append_qkv(const void* qkv, void* const* k_caches, void* const* v_caches, void* out, int batch,
                           int q_heads, int kv_heads, int capacity, int head_dim, const int32_t* cache_lens,
                           int window, float scale, int dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
    g_error[0] = '\0';
    if (batch > 0 && !qkv) return fail(MI_ATTN_ERR_INVALID, "attn_decode_append_qkv: null fused row");
    if (q_heads < 1 || kv_heads < 1 || head_dim < 1 ||
        (long)(q_heads + 2L * kv_heads) * head_dim > 0x7fffffffL)
        return fail(MI_ATTN_ERR_INVALID, "attn_decode_append_qkv: bad head counts (%d, %d) or head_dim %d",
                    q_heads, kv_heads, head_dim);
    const size_t esize = dtype == MI_ATTN_F32 ? 4 : 2;
    const char* row = (const char*)qkv;
    const void* k_new = qkv ? row + (size_t)q_heads * head_dim * esize : nullptr;
    const void* v_new = qkv ? row + (size_t)(q_heads + kv_heads) * head_dim * esize : nullptr;
    return decode_per_item("attn_decode_append_qkv", qkv, (const void* const*)k_caches,
                           (const void* const*)v_caches, k_new, v_new, out, batch, q_heads, kv_heads, capacity,
                           head_dim, cache_lens, window, scale, dtype, workspace, workspace_bytes, stream,
                           (q_heads + 2 * kv_heads) * head_dim);
}

}  // extern "C"
