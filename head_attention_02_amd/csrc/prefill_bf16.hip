// prefill_bf16.hip -- fused attention prefill for bf16 inputs on gfx950 matrix cores.
//
// Computes softmax(scale * Q K^T + mask) V per (item, query head) in one pass over the
// keys, without materialising the score matrix: the scores of one key tile live in
// registers, the row softmax is kept online in fp32 (running max and running sum,
// partial results rescaled when the max grows), and both products run on 32x32x16
// bf16 MFMA with fp32 accumulation.  The pages' backends compute the same thing as two
// batched GEMMs around a materialised, masked softmax (ripvec-core `Driver` page,
// `gemm_batched` + `fused_scale_mask_softmax`; realizar `cached/attention.rs`,
// `single_dispatch_multihead_attention`); the banded variant only visits keys inside
// the band (ripvec-core `Driver`, `banded_qk`), which here is done by skipping whole
// key tiles.
//
// Work decomposition: one workgroup = 4 waves = 128 query rows of one (item, head);
// wave w owns rows [32w, 32w+32).  The grid is one-dimensional with the q-tile index
// slowest (longest causal tiles first).  Key tiles of 64 rows of K and V are copied from
// HBM straight into LDS (global_load_lds_dwordx4, 16 bytes per lane, no registers),
// double buffered so that the copy of tile t+1 overlaps the math on tile t, with one
// barrier per tile.  LDS rows are padded (K: D/8+1, V: D/8+4 sixteen-byte slots) so
// that both the 128-bit K reads and the transposing V reads are free of bank conflicts.
//
// Per wave and key tile:
//   S^T (64 keys x 32 rows) = K_tile (A operand, from LDS) x Q^T (B operand, registers).
//     With S^T instead of S, lane l holds scores of query row l%32 only, so the
//     online softmax state (max, sum) of a row is private to lanes l and l^32.
//   O^T (D x 32 rows) += V_tile^T (A operand) x P^T (B operand).
//     P^T comes straight out of the S^T accumulator registers (packed to bf16);
//     V^T is read from the row-major V tile with the transposing LDS read
//     ds_read_b64_tr_b16, so V needs no transpose on its way into LDS.
//   The key order inside each 16-key MFMA step is permuted identically on both
//   operands (P from the accumulator layout, V by the LDS addresses), which leaves the
//   contraction unchanged.
//
// Softmax bookkeeping per tile, for scale > 0: the max is taken over raw scores and the
// scale is folded into one FMA per score, p = exp2(s*c - m*c) with c = scale*log2(e).
// The running max is only moved (and O, l rescaled) when the tile's max exceeds it by
// more than 2^8; otherwise the stale max is kept, p <= 256, and the final O / l is
// unchanged because numerator and denominator share it.
#include "mi_attn_device.hpp"
#include "mi_attn_kernels.hpp"

namespace mi_attn {
namespace {

constexpr int kBM = 128;    // query rows per workgroup
constexpr int kBN = 64;     // keys per tile
constexpr int kThreads = 256;
constexpr float kRescaleSlack = 8.0f;  // log2 units the stale max may lag behind

// LDS row strides in 16-byte slots.  One ds_read_b128 phase (16 lanes) reads 16
// consecutive K rows at one chunk: a K row stride of CPR+1 slots puts them in 16
// distinct slots modulo 256 bytes (gfx950 has 64 four-byte LDS banks).  One
// ds_read_b64_tr_b16 phase (32 lanes) reads 4 consecutive V rows (aligned to 4) at 64
// adjacent bytes: a V row stride of CPR+4 slots keeps those 256 bytes distinct modulo 256.
template <int D> constexpr int k_stride() { return D / 8 + 1; }
template <int D> constexpr int v_stride() { return D / 8 + 4; }

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Row max over both halves of the wave (lanes l and l^32 hold the same query row).
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 16-byte-per-lane copy from global memory straight into LDS: lane l's 16 bytes land
// at lds_base + 16 * l (lds_base must be wave-uniform).  Written as inline assembly so
// that the compiler does not track it as an outstanding LDS write -- it would otherwise
// wait for every copy in flight (vmcnt(0)), including the next tile's, before each LDS
// read -- and the kernel's own vmcnt wait and barrier order the copies against the
// reads.  Copies the compiler does not see can only make its own vmcnt waits stricter.
__device__ __forceinline__ void lds_dma16(const void* src, const void* lds_base) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_base;
    asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0));
}

// Copy key tile `kt` of K or V into LDS rows of STRIDE slots (16 bytes each).  Lanes that
// land on a pad slot fetch the row's first chunk again (harmless).  Rows past the valid
// length are clamped to valid-1: they hold finite copies of a valid row and are masked
// out of the softmax.
template <int D, int STRIDE>
__device__ __forceinline__ void tile_to_lds(u32x4* dst, const uint16_t* src, int kt, int valid, int wave, int lane) {
    constexpr int CPR = D / 8;
    constexpr int NI = kBN * STRIDE / 64;   // wave-wide copy instructions per tile
#pragma unroll
    for (int i0 = 0; i0 < NI; i0 += kThreads / 64) {
        const int i = i0 + wave;            // wave-uniform
        if (i < NI) {
            const int p = i * 64 + lane;
            const int row = p / STRIDE;
            int c = p - row * STRIDE;
            c = c < CPR ? c : 0;
            const int j = min(kt * kBN + row, valid - 1);
            lds_dma16(src + (size_t)j * D + c * 8, dst + i * 64);
        }
    }
}

template <int D, bool POS_SCALE>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(PrefillArgs a) {
    constexpr int KC = D / 16;                // MFMA k-steps of Q.K^T
    constexpr int DB = D / 32;                // 32-wide blocks of the output head dim
    constexpr int KS = k_stride<D>();
    constexpr int VS = v_stride<D>();

    __shared__ __attribute__((aligned(16))) u32x4 k_lds[2][kBN * KS];
    __shared__ __attribute__((aligned(16))) u32x4 v_lds[2][kBN * VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;                  // half of the wave
    // One-dimensional grid, q-tile slowest: for causal attention the tiles near the end of
    // the sequence carry the most keys, so the whole grid runs longest-first and the short
    // tiles fill in at the end instead of leaving a tail of long ones.
    const int bh = (int)(blockIdx.x % (unsigned)(a.batch * a.q_heads));
    const int qt_rank = (int)(blockIdx.x / (unsigned)(a.batch * a.q_heads));
    const int b = bh / a.q_heads;
    const int h = bh % a.q_heads;
    const int qt = a.causal ? (a.n_qtiles - 1 - qt_rank) : qt_rank;
    const int kvh = h / (a.q_heads / a.kv_heads);

    int valid = a.kv_len;
    if (a.seq_lens) valid = min(max(a.seq_lens[b], 0), a.kv_len);

    const int q0 = qt * kBM;
    const int last_row = min(q0 + kBM, a.q_len) - 1;
    const int half_w = a.window / 2;

    // ---- key range of the whole workgroup -------------------------------------------
    const int p_lo = a.pos_offset + q0;
    const int p_hi = a.pos_offset + last_row;
    int k_begin = 0;
    int k_end = valid;
    if (a.causal) k_end = min(k_end, p_hi + 1);
    if (a.window > 0) {
        if (a.causal) {
            k_begin = max(k_begin, p_lo - a.window + 1);
        } else {
            k_begin = max(k_begin, p_lo - half_w);
            k_end = min(k_end, p_hi + half_w + 1);
        }
    }
    if (p_lo >= valid) k_end = k_begin;       // every row of the tile is padding
    const int kt_begin = k_begin / kBN;
    const int kt_end = k_end > k_begin ? (k_end + kBN - 1) / kBN : kt_begin;

    // ---- this lane's query row and its key interval [lo_r, hi_r] ------------------------
    const int my_row = q0 + wave * 32 + (lane & 31);
    const int my_pos = a.pos_offset + my_row;
    int lo_r = 0, hi_r = valid - 1;
    if (a.causal) hi_r = min(hi_r, my_pos);
    if (a.window > 0) {
        if (a.causal) {
            lo_r = max(0, my_pos - a.window + 1);
        } else {
            lo_r = max(0, my_pos - half_w);
            hi_r = min(hi_r, my_pos + half_w);
        }
    }
    if (my_pos >= valid || my_row >= a.q_len) hi_r = -1;

    // the same for the wave as a whole (uniform): union and intersection of row intervals
    const int w_row0 = q0 + wave * 32;
    const int w_row1 = min(w_row0 + 31, a.q_len - 1);
    const bool wave_live = w_row0 < a.q_len && a.pos_offset + w_row0 < valid;
    const int wp_lo = a.pos_offset + w_row0, wp_hi = a.pos_offset + w_row1;
    int w_union_lo = 0, w_union_hi = valid - 1, w_inter_lo = 0, w_inter_hi = valid - 1;
    if (a.causal) {
        w_union_hi = min(w_union_hi, wp_hi);
        w_inter_hi = min(w_inter_hi, wp_lo);
    }
    if (a.window > 0) {
        if (a.causal) {
            w_union_lo = max(0, wp_lo - a.window + 1);
            w_inter_lo = max(0, wp_hi - a.window + 1);
        } else {
            w_union_lo = max(0, wp_lo - half_w);
            w_inter_lo = max(0, wp_hi - half_w);
            w_union_hi = min(w_union_hi, wp_hi + half_w);
            w_inter_hi = min(w_inter_hi, wp_lo + half_w);
        }
    }
    const bool wave_all_rows_valid = wp_hi < valid;

    // ---- Q^T operand: lane l holds row l%32, dims 16*kc + 8*g + [0, 8) ---------------
    const size_t q_head = ((size_t)b * a.q_heads + h) * (size_t)a.q_len;
    bf16x8 qf[KC];
    {
        const uint16_t* qrow = (const uint16_t*)a.q + (q_head + (size_t)min(my_row, a.q_len - 1)) * D;
        const bool in = my_row < a.q_len;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            u32x4 w = in ? *(const u32x4*)(qrow + 16 * kc + 8 * g) : u32x4{0, 0, 0, 0};
            qf[kc] = __builtin_bit_cast(bf16x8, w);
        }
    }
    // Q must have arrived before any copy is in flight: otherwise the compiler's own wait
    // for Q inside the loop would be a vmcnt(0) that also waits for the next tile's copy
    __builtin_amdgcn_s_waitcnt(0x0F70);

    const size_t kv_head = ((size_t)b * a.kv_heads + kvh) * (size_t)a.kv_len;
    const uint16_t* kg = (const uint16_t*)a.k + kv_head * D;
    const uint16_t* vg = (const uint16_t*)a.v + kv_head * D;

    // ---- running state ----------------------------------------------------------------
    f32x16 o[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] = f32x16{};
    float m_run = kNegInf;    // running (possibly stale) max of this lane's row, log2 units
    float l_run = 0.0f;       // running sum over this lane's half of the keys
    const float c2 = a.scale * kLog2e;

    if (kt_begin < kt_end) {
        tile_to_lds<D, KS>(k_lds[0], kg, kt_begin, valid, wave, lane);
        tile_to_lds<D, VS>(v_lds[0], vg, kt_begin, valid, wave, lane);
    }
    typedef __attribute__((address_space(3))) char lds_char;
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    const int k_lane = ((lane & 31) * KS + g) * 16;   // K bytes of (row l%32, chunk g)
    // bytes of the transposing V read of source lane `lane` (see the P.V step below)
    const int v_lane = ((4 * g + ((lane & 15) >> 2)) * VS) * 16 + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

    for (int kt = kt_begin; kt < kt_end; ++kt) {
        const int buf = (kt - kt_begin) & 1;
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's copies of tile kt landed
        __syncthreads();                        // ... everyone's; and tile kt-1 is no longer read
        if (kt + 1 < kt_end) {
            tile_to_lds<D, KS>(k_lds[buf ^ 1], kg, kt + 1, valid, wave, lane);
            tile_to_lds<D, VS>(v_lds[buf ^ 1], vg, kt + 1, valid, wave, lane);
        }

        const int kbase = kt * kBN;
        if (!wave_live || kbase > w_union_hi || kbase + kBN - 1 < w_union_lo) continue;
        const bool full = wave_all_rows_valid && kbase >= w_inter_lo && kbase + kBN - 1 <= w_inter_hi;
        lds_char* const k_t = (lds_char*)(void*)k_lds[buf];

        // S^T = K_tile . Q^T : two 32-key blocks
        f32x16 s[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            s[kb2] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const bf16x8 kf = __builtin_bit_cast(bf16x8, *(lds_u32x4*)(k_t + k_lane + (kb2 * 32 * KS + 2 * kc) * 16));
                s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kc], s[kb2], 0, 0, 0);
            }
        }

        // mask: element e of block kb2 is key kbase + 32*kb2 + 8*(e/4) + 4*g + e%4
        if (!full) {
            const int lo = lo_r - kbase - 4 * g, hi = hi_r - kbase - 4 * g;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int jj = 32 * kb2 + 8 * (e / 4) + (e % 4);
                    if (!POS_SCALE) s[kb2][e] *= c2;
                    s[kb2][e] = (jj >= lo && jj <= hi) ? s[kb2][e] : kNegInf;
                }
        } else if (!POS_SCALE) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) s[kb2] *= c2;
        }

        // tile row max (raw scores when scale > 0, scaled scores otherwise)
        float mx = kNegInf;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int e = 0; e < 16; e += 2) mx = max3(mx, s[kb2][e], s[kb2][e + 1]);
        mx = halves_max(mx);
        const float m_tile = POS_SCALE ? mx * c2 : mx;

        // lazy rescale: move the running max only when the tile's max runs ahead of it
        const bool need = m_tile > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float alpha = need ? fast_exp2(m_run - m_tile) : 1.0f;
            m_run = need ? m_tile : m_run;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < DB; ++i) o[i] *= alpha;
        }
        const float m_use = m_run == kNegInf ? 0.0f : m_run;

        // probabilities -> packed bf16 B operands; P chunk c4 (16 keys) = block c4/2,
        // elements 8*(c4%2) + [0, 8).
        bf16x8 pf[4];
        float lsum0 = 0.0f, lsum1 = 0.0f;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            u32x4 w;
#pragma unroll
            for (int jj = 0; jj < 8; jj += 2) {
                float p0, p1;
                if (POS_SCALE) {
                    p0 = fast_exp2(fmaf(s[c4 / 2][8 * (c4 % 2) + jj], c2, -m_use));
                    p1 = fast_exp2(fmaf(s[c4 / 2][8 * (c4 % 2) + jj + 1], c2, -m_use));
                } else {
                    p0 = fast_exp2(s[c4 / 2][8 * (c4 % 2) + jj] - m_use);
                    p1 = fast_exp2(s[c4 / 2][8 * (c4 % 2) + jj + 1] - m_use);
                }
                w[jj / 2] = pack_bf16x2(p0, p1);
                lsum0 += p0; lsum1 += p1;
            }
            pf[c4] = __builtin_bit_cast(bf16x8, w);
        }
        l_run += lsum0 + lsum1;

        // O^T += V^T . P^T; V^T via transposing reads. Within 16-lane group G = lane/16,
        // source lane s points at key 16*c4 + 4*g + s/4 (+8), dims 32*db + 16*(G%2) + 4*(s%4).
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        lds_char* const v_t = (lds_char*)(void*)v_lds[buf] + v_lane;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int imm = (16 * c4 * VS) * 16 + 64 * db;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v_t + imm));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v_t + imm + 8 * VS * 16));
                typedef __attribute__((ext_vector_type(8))) short s16x8;
                const s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[c4], o[db],
                                                               0, 0, 0);
            }
        }
    }

    // ---- epilogue: normalise, zero padded / empty rows, store bf16 --------------------
    const float l_tot = halves_sum(l_run);
    if (my_row >= a.q_len) return;
    const float inv = (hi_r >= 0 && l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
    uint16_t* orow = (uint16_t*)a.out + (q_head + (size_t)my_row) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const int d = 32 * db + 8 * e4 + 4 * g;
            u32x2 w;
            w[0] = pack_bf16x2(o[db][4 * e4] * inv, o[db][4 * e4 + 1] * inv);
            w[1] = pack_bf16x2(o[db][4 * e4 + 2] * inv, o[db][4 * e4 + 3] * inv);
            *(u32x2*)(orow + d) = w;
        }
    }
}

template <int D>
hipError_t launch_d(const PrefillArgs& args, dim3 grid, hipStream_t stream) {
    if (args.scale > 0.0f)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, true>), grid, dim3(kThreads), 0, stream, args);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, false>), grid, dim3(kThreads), 0, stream, args);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, hipStream_t stream) {
    PrefillArgs args = a;
    args.n_qtiles = (a.q_len + kBM - 1) / kBM;
    dim3 grid((unsigned)args.n_qtiles * a.q_heads * a.batch);
    switch (head_dim) {
        case 32: return launch_d<32>(args, grid, stream);
        case 64: return launch_d<64>(args, grid, stream);
        case 128: return launch_d<128>(args, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mi_attn
