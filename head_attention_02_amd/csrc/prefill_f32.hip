// prefill_f32.hip -- attention prefill for fp32 inputs (the accuracy path).
//
// Same single-pass, online-softmax algorithm as the bf16 kernel, in plain fp32 on the
// vector ALUs: each query row is held by eight lanes, each with an eighth of the row's q
// and output accumulator in registers; a score is the sum of the eight partial dot
// products (cross-lane adds within the group of eight).  Key/value tiles are staged in
// LDS (two buffers; the next tile's loads are in flight while the current one is
// computed) and read by the rows' lanes at the same addresses (a broadcast).  Only the
// keys of the row's key set contribute; tiles outside the union of the rows' key ranges
// are never loaded.  Exponentials are exp2 of scores carried in log2 units (the scale
// times log2(e) applied to each dot product).
#include "mi_attn_device.hpp"
#include "mi_attn_kernels.hpp"

namespace mi_attn {
namespace {

constexpr int kRows = 64;   // query rows per workgroup
constexpr int kLpr = 8;     // lanes per query row
constexpr int kKeys = 32;   // keys per LDS tile

template <int D>
__global__ __launch_bounds__(kRows * kLpr) void prefill_f32_kernel(PrefillArgs a) {
    constexpr int DQ = D / kLpr;   // dims per lane
    __shared__ __attribute__((aligned(16))) float k_lds[2][kKeys * D];
    __shared__ __attribute__((aligned(16))) float v_lds[2][kKeys * D];

    const int tid = threadIdx.x;
    const int part = tid % kLpr;
    const int b = blockIdx.z, h = blockIdx.y;
    const int qt = a.causal ? (a.n_qtiles - 1 - (int)blockIdx.x) : (int)blockIdx.x;
    const int kvh = h / (a.q_heads / a.kv_heads);

    const plan::Rows ir = item_rows(a, b, h, kvh, D);
    const int valid = ir.kv_valid;
    const int q_len = ir.q_len;

    const int q0 = qt * kRows;
    if (q0 >= q_len) return;   // no query row of this item in the tile (unpadded layout)
    const int last_row = min(q0 + kRows, q_len) - 1;
    const bool causal = a.causal != 0;
    // key tiles of the union of the rows' key sets
    const plan::Tiles tiles = plan::key_tiles(
        plan::span_union(a.pos_offset + q0, a.pos_offset + last_row, valid, causal, a.window), kKeys);

    const int row = q0 + tid / kLpr;
    plan::Keys mine = plan::row_keys(a.pos_offset + row, valid, causal, a.window);
    if (row >= q_len) mine.hi = -1;
    const int lo_r = mine.lo, hi_r = mine.hi;

    const float* qrow = (const float*)a.q + ir.q_base + (size_t)min(row, q_len - 1) * ir.q_rs + part * DQ;
    float q[DQ], o[DQ];
#pragma unroll
    for (int d = 0; d < DQ; ++d) {
        q[d] = row < q_len ? qrow[d] : 0.0f;
        o[d] = 0.0f;
    }
    const float* kg = (const float*)a.k + ir.kv_base;
    const float* vg = (const float*)a.v + ir.kv_base;

    // this thread's part of a tile's K and V rows (zero past the valid keys)
    constexpr int kPer = (kKeys * D / 4 + kRows * kLpr - 1) / (kRows * kLpr);
    f32x4 kr[kPer], vr[kPer];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int x = tid + i * kRows * kLpr;
            const int r = x / (D / 4), c4 = x % (D / 4);
            const int j = t * kKeys + r;
            kr[i] = f32x4{0, 0, 0, 0};
            vr[i] = f32x4{0, 0, 0, 0};
            if (x < kKeys * D / 4 && j < valid) {
                kr[i] = *(const f32x4*)(kg + (size_t)j * ir.kv_rs + 4 * c4);
                vr[i] = *(const f32x4*)(vg + (size_t)j * ir.kv_rs + 4 * c4);
            }
        }
    };
    const float c2 = a.scale * kLog2e;   // scores in log2 units
    float m_run = kNegInf, l_run = 0.0f;
    if (tiles.begin < tiles.end) load_tile(tiles.begin);
    for (int t = tiles.begin; t < tiles.end; ++t) {
        const int kbase = t * kKeys;
        float* kb = k_lds[t & 1];
        float* vb = v_lds[t & 1];
        __syncthreads();   // nobody still reads this buffer (tile t-2)
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int x = tid + i * kRows * kLpr;
            if (x < kKeys * D / 4) {
                const int r = x / (D / 4), c4 = x % (D / 4);
                *(f32x4*)(kb + r * D + 4 * c4) = kr[i];
                *(f32x4*)(vb + r * D + 4 * c4) = vr[i];
            }
        }
        __syncthreads();
        if (t + 1 < tiles.end) load_tile(t + 1);   // in flight while tile t is computed

        float s[kKeys];
        float mx = kNegInf;
#pragma unroll
        for (int jj = 0; jj < kKeys; ++jj) {
            float dot = 0.0f;
#pragma unroll
            for (int d = 0; d < DQ; ++d) dot = fmaf(q[d], kb[jj * D + part * DQ + d], dot);
            dot = row_sum<kLpr>(dot);   // the row's eight parts
            const int j = kbase + jj;
            s[jj] = (j >= lo_r && j <= hi_r) ? dot * c2 : kNegInf;
            mx = fmaxf(mx, s[jj]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == kNegInf ? 0.0f : m_new;
        const float alpha = exp2f(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < DQ; ++d) o[d] *= alpha;
#pragma unroll
        for (int jj = 0; jj < kKeys; ++jj) {
            const float p = exp2f(s[jj] - m_use);
            l_run += p;
#pragma unroll
            for (int d = 0; d < DQ; ++d) o[d] = fmaf(p, vb[jj * D + part * DQ + d], o[d]);
        }
    }

    if (row >= q_len) return;
    const float inv = (hi_r >= 0 && l_run > 0.0f) ? 1.0f / l_run : 0.0f;
    float* orow = (float*)a.out + ir.q_base + (size_t)row * ir.q_rs + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d += 4) *(f32x4*)(orow + d) = f32x4{o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv};
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, int head_dim, hipStream_t stream) {
    PrefillArgs args = a;
    args.n_qtiles = (a.q_len + kRows - 1) / kRows;
    dim3 grid(args.n_qtiles, a.q_heads, a.batch), block(kRows * kLpr);
    switch (head_dim) {
        case 32: hipLaunchKernelGGL(prefill_f32_kernel<32>, grid, block, 0, stream, args); break;
        case 64: hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, 0, stream, args); break;
        case 128: hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, block, 0, stream, args); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mi_attn
