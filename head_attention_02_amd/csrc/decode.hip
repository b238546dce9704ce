// decode.hip -- single-token attention over a head-major KV cache (split-KV).
//
// The operation is `flash_attention_batched_per_cache` of the ferrum-kernels `Backend`
// page: one query token per (item, query head) against that item's cache
// [kv_heads, capacity, head_dim], with per-item lengths read on the device and an
// optional causal window (the last w positions).  It is bound by HBM bandwidth: every
// cache byte in range is read exactly once.
//
// Pass 1 (decode_split_kernel): the key range of each (item, kv head) is cut into
// `splits` pieces, one workgroup each.  Every K/V row (head_dim bf16 = 256 bytes at
// head_dim 128) is read by D/8 lanes with one 16-byte load each, so one wave load covers
// 64 / (D/8) consecutive rows (1 KiB) -- fully coalesced.  The workgroup keeps the
// queries of all GT query heads of the group in registers, so each K/V byte is read once
// for the whole group (no per-query-head copy of the cache).  Dot products are reduced
// across the lanes of a row with DPP, the softmax runs online in fp32, and the
// workgroup's partial state (running max m, running sum l, unnormalised output o) is
// written to the workspace.
// Pass 2 (decode_combine_kernel): per (item, query head) the partial states of the
// splits are merged exactly: m* = max m_s, out = sum_s 2^(m_s - m*) o_s / sum_s 2^(m_s - m*) l_s.
// With a single split (enough (item, kv head) units to fill the GPU) the first pass
// normalises and stores the output itself, and there is no workspace and no second pass.
#include <type_traits>

#include "mi_attn_device.hpp"
#include "mi_attn_kernels.hpp"

namespace mi_attn {
namespace {

constexpr int kWaves = plan::DecodeGeo<128>::WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;   // log2 units the stale running max may lag behind

// Eight consecutive elements as fp32.  STREAM marks a load of cache rows, which are read
// exactly once: it is issued non-temporal, so the rows stream through the caches without
// displacing anything (a plain-load read of 2 GiB measured about 6.3 TB/s on MI355X, the
// same read with non-temporal loads about 7.0 TB/s).
// Element formats (the values of mi_attn_dtype).
constexpr int kF32 = 0, kBF16 = 1, kF16 = 2;

template <int FMT, bool STREAM = false>
__device__ __forceinline__ void load8(const void* base, size_t elem, float* x) {
    if constexpr (FMT != kF32) {
        const u32x4* src = (const u32x4*)((const uint16_t*)base + elem);
        const u32x4 w = STREAM ? __builtin_nontemporal_load(src) : *src;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = FMT == kBF16 ? bf16_lo(w[i]) : f16_lo(w[i]);
            x[2 * i + 1] = FMT == kBF16 ? bf16_hi(w[i]) : f16_hi(w[i]);
        }
    } else {
        const f32x4* src = (const f32x4*)((const float*)base + elem);
        const f32x4 a = STREAM ? __builtin_nontemporal_load(src) : src[0];
        const f32x4 b = STREAM ? __builtin_nontemporal_load(src + 1) : src[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = a[i];
            x[4 + i] = b[i];
        }
    }
}

// The 16 (bf16, fp16) or 32 (fp32) bytes of eight consecutive elements, copied unchanged.
template <int FMT>
__device__ __forceinline__ void copy8(const void* src, size_t src_elem, void* dst, size_t dst_elem) {
    constexpr int esz = FMT == kF32 ? 4 : 2;
    const u32x4* s = (const u32x4*)((const char*)src + src_elem * esz);
    u32x4* d = (u32x4*)((char*)dst + dst_elem * esz);
    d[0] = s[0];
    if constexpr (FMT == kF32) d[1] = s[1];
}

// Cache addressing modes of the split kernel.
enum CacheMode {
    kStacked = 0,   // caches [batch, kv_heads, capacity, D] in one allocation
    kPerItem = 1,   // one [kv_heads, capacity, D] allocation per item, via a pointer array
    kAppend = 2,    // per item, and the new token's K/V row is appended before attending
};

// One result in the output format (round to nearest even for the 16-bit formats).
template <int FMT>
__device__ __forceinline__ void store1(void* out, size_t at, float v) {
    if constexpr (FMT == kBF16)
        ((__bf16*)out)[at] = (__bf16)v;
    else if constexpr (FMT == kF16)
        ((_Float16*)out)[at] = (_Float16)v;
    else
        ((float*)out)[at] = v;
}

// Two-element dot product of packed 16-bit pairs, accumulated in fp32:
// c + a.lo * b.lo + a.hi * b.hi (v_dot2_f32_bf16 / v_dot2_f32_f16).
template <int FMT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (FMT == kBF16) {
        typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
    } else {
        typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
    }
}

// Sixteen raw bytes (eight 16-bit elements) of a cache row, non-temporal.
__device__ __forceinline__ u32x4 load8_raw(const void* base, size_t elem) {
    return __builtin_nontemporal_load((const u32x4*)((const uint16_t*)base + elem));
}

// Merges the online-softmax states (m, l, o) of the lanes lane ^ x for x = first,
// 2*first, ..., 32 (the row streams of one wave that hold the same elements): every lane
// ends with the merge of its group.
template <int GT, int EPL>
__device__ __forceinline__ void merge_lanes(float (&m)[GT], float (&l)[GT], float (&o)[GT][EPL], int first) {
    for (int x = first; x < 64; x *= 2) {
#pragma unroll
        for (int t = 0; t < GT; ++t) {
            const float mo = __shfl_xor(m[t], x), lo = __shfl_xor(l[t], x);
            const float mm = fmaxf(m[t], mo);
            const float m_use = mm == kNegInf ? 0.0f : mm;
            const float a1 = fast_exp2(m[t] - m_use), a2 = fast_exp2(mo - m_use);
            l[t] = l[t] * a1 + lo * a2;
#pragma unroll
            for (int i = 0; i < EPL; ++i) o[t][i] = o[t][i] * a1 + __shfl_xor(o[t][i], x) * a2;
            m[t] = mm;
        }
    }
}

template <int D, int GT, int FMT, int MODE>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
    // 16-bit caches are read as packed pairs, EPL (8 or 16) elements per lane and row:
    // word w (8 elements, 16 bytes) of lane c holds elements w*D/NW + 8c + [0, 8), so that
    // each load instruction reads whole 128-byte runs of its rows
    constexpr bool PACKED = FMT != kF32;
    constexpr int EPL = PACKED && D >= 64 ? 16 : 8;
    constexpr int NW = EPL / 8;                                      // 16-byte words per lane and row
    using DG = plan::DecodeGeo<D, EPL>;
    constexpr int LPR = DG::LPR;          // lanes per key row
    constexpr int RPW = DG::RPW;          // rows per wave load
    constexpr int BATCH = DG::BATCH;
    constexpr int kSteps = DG::STEPS;     // wave loads per batch (rows per lane group between softmax updates)

    __shared__ float s_m[kWaves][GT];
    __shared__ float s_l[kWaves][GT];
    __shared__ float s_o[kWaves][GT][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane / LPR, c = lane % LPR;
    const int b = blockIdx.z;
    const int kvh = blockIdx.y / a.head_groups;
    const int hg = blockIdx.y % a.head_groups;
    const int split = blockIdx.x;
    const int group = a.q_heads / a.kv_heads;
    const int h0 = kvh * group + hg * GT;

    // the query's position and the keys [s0, s1) this split attends (plan::decode_query,
    // plan::decode_split_keys)
    const plan::DecodeQuery dq = plan::decode_query(MODE == kAppend, a.kv_lens != nullptr,
                                                    a.kv_lens ? a.kv_lens[b] : 0, a.kv_len, a.capacity,
                                                    a.pos_offset);
    const int pos = dq.pos;
    const plan::KeyRange kr_split = plan::decode_split_keys(dq, a.window, split, a.split_len);
    const int s0 = kr_split.s0;
    const int s1 = kr_split.s1;

    // queries of the GT heads: fp32, pre-multiplied by scale * log2(e); 16-bit formats
    // keep them packed as given (the scale is applied to each dot product)
    const float c2 = a.scale * kLog2e;
    float qf[GT][8];
    u32x4 qw[GT][NW];
#pragma unroll
    for (int t = 0; t < GT; ++t) {
        const size_t q_at = (size_t)b * a.q_rs + (size_t)(h0 + t) * D + 8 * c;
        if constexpr (PACKED) {
#pragma unroll
            for (int w = 0; w < NW; ++w) qw[t][w] = *(const u32x4*)((const uint16_t*)a.q + q_at + w * (D / NW));
        } else {
            load8<FMT>(a.q, q_at, qf[t]);
#pragma unroll
            for (int i = 0; i < 8; ++i) qf[t][i] *= c2;
        }
    }

    float m[GT], l[GT], o[GT][EPL];
#pragma unroll
    for (int t = 0; t < GT; ++t) {
        m[t] = kNegInf;
        l[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) o[t][i] = 0.0f;
    }

    const void* kc = a.k;
    const void* vc = a.v;
    size_t head_base = ((size_t)b * a.kv_heads + kvh) * (size_t)a.capacity * D;
    if constexpr (MODE != kStacked) {
        kc = a.k_ptrs[b];
        vc = a.v_ptrs[b];
        head_base = (size_t)kvh * a.capacity * D;
    }
    // append: the row at the query position comes from the new token (registers of the
    // lanes that read it), not from the cache; the split that holds the position also
    // stores the new rows into the cache (first head group only).  No other workgroup
    // reads that slot, so the store does not race with the reads.
    const size_t new_row = (size_t)b * a.new_rs + (size_t)kvh * D + 8 * c;
    if constexpr (MODE == kAppend) {
        if (hg == 0 && pos >= s0 && pos < s1 && tid < LPR) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                copy8<FMT>(a.k_new, new_row + w * (D / NW), (void*)kc, head_base + (size_t)pos * D + 8 * c + w * (D / NW));
                copy8<FMT>(a.v_new, new_row + w * (D / NW), (void*)vc, head_base + (size_t)pos * D + 8 * c + w * (D / NW));
            }
        }
    }
    // One batch of kSteps wave loads per lane group.  TAIL: the last batch of the key range;
    // it may reach past the end, so its rows are clamped to a valid one and masked, and it
    // holds the query position, the only row an append takes from the new token (key
    // s1 - 1 when this split holds the position).  The other batches skip all three.  The
    // running max is moved lazily, only when a batch's max exceeds it by more than 2^8
    // (p <= 256 otherwise; o and l share the stale max, so the merges below and the
    // combine pass are unchanged).
    auto batch = [&](int base, auto tail_c) {
        constexpr bool TAIL = decltype(tail_c)::value;
        int key[kSteps];
        float s[kSteps][GT];
        // K rows -> scores (log2 units, scale applied)
        if constexpr (PACKED) {
            u32x4 kw[kSteps][NW];
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
                key[u] = base + (u * kWaves + wave) * RPW + r;
                const int kr = plan::decode_key_row(key[u], s0, s1, TAIL);   // out-of-range rows read a valid row
                const bool nw = MODE == kAppend && TAIL && kr == pos;
                const void* src = nw ? a.k_new : kc;
                const size_t at = nw ? new_row : head_base + (size_t)kr * D + 8 * c;
#pragma unroll
                for (int w = 0; w < NW; ++w) kw[u][w] = load8_raw(src, at + w * (D / NW));
            }
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
#pragma unroll
                for (int t = 0; t < GT; ++t) {
                    float d = 0.0f;
#pragma unroll
                    for (int w = 0; w < NW; ++w)
#pragma unroll
                        for (int i = 0; i < 4; ++i) d = dot2<FMT>(kw[u][w][i], qw[t][w][i], d);
                    d = row_sum<LPR>(d) * c2;
                    s[u][t] = !TAIL || key[u] < s1 ? d : kNegInf;
                }
            }
        } else {
            float kx[kSteps][8];
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
                key[u] = base + (u * kWaves + wave) * RPW + r;
                const int kr = plan::decode_key_row(key[u], s0, s1, TAIL);
                const bool nw = MODE == kAppend && TAIL && kr == pos;
                load8<FMT, true>(nw ? a.k_new : kc, nw ? new_row : head_base + (size_t)kr * D + 8 * c, kx[u]);
            }
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
#pragma unroll
                for (int t = 0; t < GT; ++t) {
                    float d = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) d = fmaf(qf[t][i], kx[u][i], d);
                    d = row_sum<LPR>(d);
                    s[u][t] = !TAIL || key[u] < s1 ? d : kNegInf;
                }
            }
        }
        // V rows (loaded before the softmax so that they are in flight during it)
        float vx[PACKED ? 1 : kSteps][8];
        u32x4 vw[PACKED ? kSteps : 1][NW];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int kr = plan::decode_key_row(key[u], s0, s1, TAIL);
            const bool nw = MODE == kAppend && TAIL && kr == pos;
            const void* src = nw ? a.v_new : vc;
            const size_t at = nw ? new_row : head_base + (size_t)kr * D + 8 * c;
            if constexpr (PACKED) {
#pragma unroll
                for (int w = 0; w < NW; ++w) vw[u][w] = load8_raw(src, at + w * (D / NW));
            } else {
                load8<FMT, true>(src, at, vx[u]);
            }
        }
        float m_new[GT];
        bool need_any = false;
#pragma unroll
        for (int t = 0; t < GT; ++t) {
            float mx = kNegInf;
#pragma unroll
            for (int u = 0; u < kSteps; ++u) mx = fmaxf(mx, s[u][t]);
            m_new[t] = fmaxf(m[t], mx);
            need_any |= m_new[t] > m[t] + kRescaleSlack;
        }
        if (__builtin_amdgcn_ballot_w64(need_any)) {
#pragma unroll
            for (int t = 0; t < GT; ++t) {
                const bool need = m_new[t] > m[t] + kRescaleSlack;
                const float alpha = need ? fast_exp2(m[t] - m_new[t]) : 1.0f;
                m[t] = need ? m_new[t] : m[t];
                l[t] *= alpha;
#pragma unroll
                for (int i = 0; i < EPL; ++i) o[t][i] *= alpha;
            }
        }
        if constexpr (PACKED) {
            // rows u and u+1 of this lane go together: each dot2 takes one element of both
            // rows (v_perm_b32 pairs them) against the two probabilities, rounded to the
            // cache format as the P.V products of the prefill kernels take them
            float p[kSteps][GT];
#pragma unroll
            for (int t = 0; t < GT; ++t) {
                const float m_use = m[t] == kNegInf ? 0.0f : m[t];
                float ps = 0.0f;
#pragma unroll
                for (int u = 0; u < kSteps; ++u) {
                    p[u][t] = fast_exp2(s[u][t] - m_use);
                    ps += p[u][t];
                }
                l[t] += ps;
            }
#pragma unroll
            for (int u = 0; u < kSteps; u += 2) {
                uint32_t lo[NW][4], hi[NW][4];
#pragma unroll
                for (int w = 0; w < NW; ++w)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        lo[w][i] = __builtin_amdgcn_perm(vw[u + 1][w][i], vw[u][w][i], 0x05040100u);   // element 2i of rows u, u+1
                        hi[w][i] = __builtin_amdgcn_perm(vw[u + 1][w][i], vw[u][w][i], 0x07060302u);   // element 2i+1
                    }
#pragma unroll
                for (int t = 0; t < GT; ++t) {
                    const uint32_t pp = FMT == kBF16 ? pack_bf16x2(p[u][t], p[u + 1][t]) : pack_f16x2(p[u][t], p[u + 1][t]);
#pragma unroll
                    for (int w = 0; w < NW; ++w)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            o[t][8 * w + 2 * i] = dot2<FMT>(lo[w][i], pp, o[t][8 * w + 2 * i]);
                            o[t][8 * w + 2 * i + 1] = dot2<FMT>(hi[w][i], pp, o[t][8 * w + 2 * i + 1]);
                        }
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < GT; ++t) {
                const float m_use = m[t] == kNegInf ? 0.0f : m[t];
                float ps = 0.0f;
#pragma unroll
                for (int u = 0; u < kSteps; ++u) {
                    const float p = fast_exp2(s[u][t] - m_use);
                    ps += p;
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[t][i] = fmaf(p, vx[u][i], o[t][i]);
                }
                l[t] += ps;
            }
        }
    };
    int base = s0;
    for (; base + BATCH < s1; base += BATCH) batch(base, std::integral_constant<bool, false>{});
    if (base < s1) batch(base, std::integral_constant<bool, true>{});

    // merge the row streams: first those of each wave (lanes with the same elements), then
    // the waves' through LDS
    merge_lanes<GT, EPL>(m, l, o, LPR);
    if (r == 0) {
#pragma unroll
        for (int t = 0; t < GT; ++t) {
            if (c == 0) {
                s_m[wave][t] = m[t];
                s_l[wave][t] = l[t];
            }
#pragma unroll
            for (int i = 0; i < EPL; ++i) s_o[wave][t][(i / 8) * (D / NW) + 8 * c + i % 8] = o[t][i];
        }
    }
    __syncthreads();
    for (int x = tid; x < GT * D; x += kThreads) {
        const int t = x / D, d = x % D;
        float mm = kNegInf;
#pragma unroll
        for (int st = 0; st < kWaves; ++st) mm = fmaxf(mm, s_m[st][t]);
        const float m_use = mm == kNegInf ? 0.0f : mm;
        float acc = 0.0f, ll = 0.0f;
#pragma unroll
        for (int st = 0; st < kWaves; ++st) {
            const float w = fast_exp2(s_m[st][t] - m_use);
            acc = fmaf(w, s_o[st][t][d], acc);
            ll = fmaf(w, s_l[st][t], ll);
        }
        if (a.splits == 1) {
            // the whole key range is this workgroup's: normalise and store (what the
            // combine pass would compute from this one partial state, bit for bit)
            const size_t at = ((size_t)b * a.q_heads + h0 + t) * D + d;
            const float res = ll > 0.0f ? acc / ll : 0.0f;
            store1<FMT>(a.out, at, res);
        } else {
            float* ws = a.ws + (((size_t)b * a.q_heads + h0 + t) * a.splits + split) * (D + 2);
            ws[d] = acc;
            if (d == 0) {
                ws[D] = mm;
                ws[D + 1] = ll;
            }
        }
    }
}

template <int D, int FMT>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
    const int d = threadIdx.x;
    const size_t bh = blockIdx.x;   // b * q_heads + h
    const float* ws = a.ws + bh * a.splits * (D + 2);
    float mm = kNegInf;
    for (int s = 0; s < a.splits; ++s) mm = fmaxf(mm, ws[s * (D + 2) + D]);
    const float m_use = mm == kNegInf ? 0.0f : mm;
    float acc = 0.0f, ll = 0.0f;
    for (int s = 0; s < a.splits; ++s) {
        const float w = fast_exp2(ws[s * (D + 2) + D] - m_use);
        acc = fmaf(w, ws[s * (D + 2) + d], acc);
        ll = fmaf(w, ws[s * (D + 2) + D + 1], ll);
    }
    const float res = ll > 0.0f ? acc / ll : 0.0f;
    store1<FMT>(a.out, bh * D + d, res);
}

template <int D, int FMT, int MODE>
void launch_split(const DecodeArgs& a, int gt, dim3 grid, hipStream_t stream) {
    const dim3 block(kThreads);
    switch (gt) {
        case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1, FMT, MODE>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2, FMT, MODE>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4, FMT, MODE>), grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL((decode_split_kernel<D, 8, FMT, MODE>), grid, block, 0, stream, a); break;
    }
}

template <int D, int FMT>
hipError_t launch_d(const DecodeArgs& a, int gt, hipStream_t stream) {
    if (gt != 1 && gt != 2 && gt != 4 && gt != 8) return hipErrorInvalidValue;
    const dim3 grid(a.splits, a.kv_heads * a.head_groups, a.batch);
    if (a.k_new)
        launch_split<D, FMT, kAppend>(a, gt, grid, stream);
    else if (a.k_ptrs)
        launch_split<D, FMT, kPerItem>(a, gt, grid, stream);
    else
        launch_split<D, FMT, kStacked>(a, gt, grid, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL((decode_combine_kernel<D, FMT>), dim3(a.batch * a.q_heads), dim3(D), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// Two workgroups fit on a CU (the split kernel's register use allows two waves per
// SIMD), so 512 workgroups fill MI355X's 256 CUs exactly once.  Splitting further only
// shortens the streams and adds partial states: on the batch-64 kv-8192 decode, 512
// workgroups (no split) ran in 318 us, 1024 in 324 us, 2048 in 333 us.
plan::DecodePlan plan_decode(int batch, int q_heads, int kv_heads, int kv_len, int head_dim) {
    (void)head_dim;
    return plan::decode_plan(batch, q_heads, kv_heads, kv_len, 512);
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int heads_per_group, int dtype,
                         hipStream_t stream) {
    const int gt = heads_per_group;
    auto by_format = [&](auto d_c) -> hipError_t {
        constexpr int D = decltype(d_c)::value;
        switch (dtype) {
            case kF32: return launch_d<D, kF32>(a, gt, stream);
            case kBF16: return launch_d<D, kBF16>(a, gt, stream);
            case kF16: return launch_d<D, kF16>(a, gt, stream);
            default: return hipErrorInvalidValue;
        }
    };
    switch (head_dim) {
        case 32: return by_format(std::integral_constant<int, 32>{});
        case 64: return by_format(std::integral_constant<int, 64>{});
        case 128: return by_format(std::integral_constant<int, 128>{});
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mi_attn
