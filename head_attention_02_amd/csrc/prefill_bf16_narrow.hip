// prefill_bf16_narrow.hip -- fused bf16 attention prefill for head dims 32 and 64.
//
// Same computation, operand layouts and softmax bookkeeping as the head-dim-128 kernel
// in prefill_bf16.hip: softmax(scale * Q K^T + mask) V per (item, query head) in one pass
// over the keys, online softmax in fp32, both products on 32x32x16 bf16 MFMA with fp32
// accumulation (S^T = K Q^T so that a lane holds one query row; P^T straight from the
// accumulator; V^T through the transposing LDS read), masked key tiles skipped whole.
//
// What differs is the schedule.  At these head dims the vector work of a tile (mask,
// max, exp, pack: fixed per key) is as large as its matrix work (which scales with the
// head dim), so the two-group ping-pong of the wide kernel leaves the matrix core idle
// half the time.  Here every wave runs both streams itself, in one explicitly ordered
// instruction sequence, and two workgroups share a CU.
//
// Work decomposition: one workgroup = 4 waves = 128 query rows of one (item, head);
// wave w owns rows [32w, 32w+32).  The grid is one-dimensional with the q-tile index
// slowest (longest tiles first) and XCD-aware.  Key tiles of 64 rows of K and V
// are copied from HBM straight into LDS (global_load_lds_dwordx4, 16 bytes per lane, no
// registers) with per-lane offsets computed once; one barrier per tile.
//
// Software pipeline: the loop body for tile t issues the Q.K^T MFMAs of tile t+1 next
// to the exp/pack work of tile t (matrix core and vector ALU run side by side), then
// the P.V MFMAs of tile t next to the row max of tile t+1.  K is therefore kept one
// tile ahead of V: the copies issued in the body of tile t are K(t+2) and V(t+1), each
// into the buffer its predecessor vacated.
//
// Softmax bookkeeping per tile, for scale > 0: the max is taken over raw scores and the
// scale is folded into one FMA per score, p = exp2(s*c - m*c) with c = scale*log2(e).
// The running max is only moved (and O, l rescaled) when the tile's max exceeds it by
// more than 2^8; otherwise the stale max is kept, p <= 256, and the final O / l is
// unchanged because numerator and denominator share it.
//
// LDS layout (bank conflicts): gfx950 LDS has 64 four-byte banks.  One ds_read_b128
// phase (16 lanes) reads 16 consecutive K rows at one 16-byte chunk, so K rows are
// padded to D/8+1 chunks.  One ds_read_b64_tr_b16 phase (32 lanes) reads 4 consecutive V
// rows at one 64-byte column group, so V rows are XOR-swizzled at 64-byte granularity:
// chunk c of row r sits at chunk c ^ vswz(r), which puts the four rows in four
// different quarters of the 256 bytes the banks cover.
#include <type_traits>

#include "prefill_common.hpp"

namespace mi_attn {
namespace {

constexpr int kBN = 64;     // keys per tile (plan::NarrowGeo::BN)
constexpr float kRescaleSlack = 8.0f;  // log2 units the stale max may lag behind

template <int D, int W>
using Geo = plan::NarrowGeo<D, W>;

template <int D, int RB, int W, bool POS_SCALE, bool F16>
struct Prefill {
    using G = Geo<D, W>;
    using H = Fmt16<F16>;

    // ---- per-lane constants ---------------------------------------------------------
    int lane, wave, g;
    int kvalid;                 // valid key rows of this item
    int kv_rs;                  // elements from one K/V row to the next
    const char* kg;             // K rows of this (item, kv head)
    const char* vg;
    uint32_t k_lds0, v_lds0;    // LDS byte addresses of buffer 0
    uint32_t koff[G::NKW];      // byte offsets of this lane's K copy chunks inside a tile
    uint32_t voff;              // ... V (first copy; copy ii reads v_step * ii bytes further)
    size_t v_step;              // byte distance between the rows of consecutive V copies
    int k_read;                 // LDS byte offset of this lane's K operand (row l%32, chunk g)
    int v_read[G::DB];          // LDS byte offsets of this lane's transposing V reads
    int lo_r[RB], hi_r[RB];     // this lane's key interval, per row block
    bool blk_all_rows_valid[RB];
    int b_inter_lo[RB], b_inter_hi[RB];  // keys every row of a row block sees
    int union_lo, union_hi;     // keys some row of the wave sees (a superset; empty if hi < lo)
    float c2;                   // scale * log2(e)

    // ---- running state ----------------------------------------------------------------
    bf16x8 qf[RB][G::KC];
    f32x16 o[RB][G::DB];
    float m_run[RB], l_run[RB];

    // Tile copies (addresses from plan::narrow_k_chunk / narrow_v_chunk).  The tail case
    // (rows past the valid length repeat the last valid row, clamped from the tile base) is
    // decided once per tile; whole tiles use the precomputed per-lane offsets.
    __device__ __forceinline__ void copy_k(int kt, int par) {
        const char* base = kg + (size_t)kt * kBN * kv_rs * 2;
        const uint32_t lds = k_lds0 + par * G::K_BYTES + wave * 1024;
        if (kt * kBN + kBN <= kvalid) {
#pragma unroll
            for (int ii = 0; ii < G::NKW; ++ii)
                if (G::NK % W == 0 || ii + 1 < G::NKW || wave + W * ii < G::NK)
                    lds_dma16(base, koff[ii], lds + W * ii * 1024);
        } else {
            keep_branch();
#pragma unroll
            for (int ii = 0; ii < G::NKW; ++ii) {
                const int i = wave + W * ii;
                if (i < G::NK) {
                    plan::Chunk c = plan::narrow_k_chunk(i, lane, G::CPR);
                    c.row = plan::tail_row(c.row, kvalid, kt * kBN);
                    lds_dma16(base, plan::chunk_offset(c, kv_rs), lds + W * ii * 1024);
                }
            }
        }
    }

    __device__ __forceinline__ void copy_v(int kt, int par) {
        const char* base = vg + (size_t)kt * kBN * kv_rs * 2;
        const uint32_t lds = v_lds0 + par * G::V_BYTES + wave * 1024;
        if (kt * kBN + kBN <= kvalid) {
            // copy ii covers the rows W*64/CPR further down than copy ii-1 (same lane
            // offsets: the swizzle repeats with that period)
#pragma unroll
            for (int ii = 0; ii < G::NVW; ++ii) lds_dma16(base + ii * v_step, voff, lds + W * ii * 1024);
        } else {
            keep_branch();
#pragma unroll
            for (int ii = 0; ii < G::NVW; ++ii) {
                plan::Chunk c = plan::narrow_v_chunk(wave + W * ii, lane, D);
                c.row = plan::tail_row(c.row, kvalid, kt * kBN);
                lds_dma16(base, plan::chunk_offset(c, kv_rs), lds + W * ii * 1024);
            }
        }
    }

    // K operand f of a tile (f = 32-key block * KC + k-step): row l%32 of the block,
    // dims 16*kc + 8*g + [0, 8).
    __device__ __forceinline__ bf16x8 k_frag(const lds_char* kbuf, int f) const {
        const int kb2 = f / G::KC, kc = f % G::KC;
        return __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(kbuf + k_read + (kb2 * 32 * G::KS + 2 * kc) * 16));
    }

    // V^T operand j of a tile (j = 16-key chunk * DB + 32-dim block) via two transposing
    // reads.  Within 16-lane group G = lane/16, source lane s points at key
    // 16*c4 + 4*g + s/4 (+8), dims 32*db + 16*(G%2) + 4*(s%4).
    __device__ __forceinline__ bf16x8 v_frag(const lds_char* vbuf, int j) const {
        const int c4 = j / G::DB, db = j % G::DB;
        const lds_char* p = vbuf + v_read[db] + 16 * c4 * 2 * D;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * 2 * D));
        typedef __attribute__((ext_vector_type(8))) short s16x8;
        const s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, vv);
    }

    // Probabilities of one 16-key chunk u (row block u/4, chunk c4 = u%4 = block c4/2,
    // elements 8*(c4%2) + [0, 8)) -> packed bf16 P^T operand, plus their fp32 row sums.
    __device__ __forceinline__ void probs_chunk(const f32x16 (&s)[RB][2], bf16x8 (&pf)[RB][4], float (&ls)[RB][2],
                                                const float (&m_use)[RB], int u) const {
        const int rb = u / 4, c4 = u % 4;
        u32x4 w;
#pragma unroll
        for (int jj = 0; jj < 8; jj += 2) {
            const float s0 = s[rb][c4 / 2][8 * (c4 % 2) + jj], s1 = s[rb][c4 / 2][8 * (c4 % 2) + jj + 1];
            const float p0 = POS_SCALE ? fast_exp2(fmaf(s0, c2, -m_use[rb])) : fast_exp2(s0 - m_use[rb]);
            const float p1 = POS_SCALE ? fast_exp2(fmaf(s1, c2, -m_use[rb])) : fast_exp2(s1 - m_use[rb]);
            w[jj / 2] = H::pack2(p0, p1);
            ls[rb][0] += p0;
            ls[rb][1] += p1;
        }
        // anchor the operand here: left alone, the compiler sinks this side-effect-free
        // work past the masking branch, next to the P.V products, away from the
        // Q.K^T MFMAs it is meant to run beside
        asm volatile("" : "+v"(w));
        pf[rb][c4] = __builtin_bit_cast(bf16x8, w);
    }

    // S^T = K_tile . Q^T for every row block (the first tile, before the loop).
    __device__ __forceinline__ void qk(f32x16 (&s)[RB][2], const lds_char* kbuf) const {
#pragma unroll
        for (int f = 0; f < 2 * G::KC; ++f) {
            const int kb2 = f / G::KC, kc = f % G::KC;
            const bf16x8 kf = k_frag(kbuf, f);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                s[rb][kb2] = H::mfma32x32x16(kf, qf[rb][kc], kc == 0 ? f32x16{} : s[rb][kb2]);
        }
    }

    // First half of a pipelined step, as one explicitly ordered stream: the Q.K^T MFMAs
    // of the next tile (each K operand read from LDS four steps ahead of its use and
    // shared by all row blocks) with a slice of this tile's softmax after each of them.
    // sched_barrier(0) keeps the compiler from regrouping the MFMAs.
    // Whether key tile kt holds a key that some row of this wave sees.  A tile that holds
    // none (outside the band, past the causal diagonal) takes no MFMA and no softmax work
    // in this wave; the other waves of the workgroup may still need it.
    __device__ __forceinline__ bool wave_sees(int kt) const {
        return kt * kBN <= union_hi && kt * kBN + kBN - 1 >= union_lo;
    }

    // The two halves of a step when only one of them has work in this wave.
    __device__ __forceinline__ void probs_only(const f32x16 (&cur)[RB][2], bf16x8 (&pf)[RB][4]) {
        float m_use[RB], ls[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            m_use[rb] = m_run[rb] == kNegInf ? 0.0f : m_run[rb];
            ls[rb][0] = ls[rb][1] = 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 4 * RB; ++u) probs_chunk(cur, pf, ls, m_use, u);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) l_run[rb] += ls[rb][0] + ls[rb][1];
    }

    template <bool HAS_NEXT>
    __device__ __forceinline__ void qk_next_probs(f32x16 (&nxt)[RB][2], const f32x16 (&cur)[RB][2],
                                                  bf16x8 (&pf)[RB][4], const lds_char* kbuf) {
        constexpr int NF = 2 * G::KC;   // K operands per tile
        constexpr int NU = 4 * RB;      // softmax chunks
        constexpr int PF = 4;           // K operands in flight
        float m_use[RB], ls[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            m_use[rb] = m_run[rb] == kNegInf ? 0.0f : m_run[rb];
            ls[rb][0] = ls[rb][1] = 0.0f;
        }
        if constexpr (HAS_NEXT) {
            bf16x8 kf[PF];
#pragma unroll
            for (int f = 0; f < PF; ++f) kf[f] = k_frag(kbuf, f);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int kb2 = f / G::KC, kc = f % G::KC;
                const bf16x8 k_now = kf[f % PF];
                if (f + PF < NF) kf[f % PF] = k_frag(kbuf, f + PF);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    nxt[rb][kb2] = H::mfma32x32x16(k_now, qf[rb][kc], kc == 0 ? f32x16{} : nxt[rb][kb2]);
#pragma unroll
                for (int u = f * NU / NF; u < (f + 1) * NU / NF; ++u) probs_chunk(cur, pf, ls, m_use, u);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int u = 0; u < NU; ++u) probs_chunk(cur, pf, ls, m_use, u);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            l_run[rb] += ls[rb][0] + ls[rb][1];
            asm volatile("" : "+v"(l_run[rb]));
        }
    }

    // Masks the scores of tile kt for rows that do not see every key of it (and scales
    // them when the scale is not positive); element e of block kb2 is key
    // kt*64 + 32*kb2 + 8*(e/4) + 4*g + e%4.
    __device__ __forceinline__ void mask_scale(f32x16 (&s)[RB][2], int kt) const {
        const int kbase = kt * kBN;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const bool full = blk_all_rows_valid[rb] && kbase >= b_inter_lo[rb] && kbase + kBN - 1 <= b_inter_hi[rb];
            if (!full) {
                keep_branch();
                // key jj is kept iff lo <= jj <= hi, tested as one unsigned compare
                // (jj - lo) <= (hi - lo): no scalar mask arithmetic between the compares
                const int lo = lo_r[rb] - kbase - 4 * g, hi = hi_r[rb] - kbase - 4 * g;
                const int lo2 = hi >= lo ? lo : (1 << 30);        // empty interval: nothing kept
                const unsigned span = hi >= lo ? (unsigned)(hi - lo) : 0u;
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int jj = 32 * kb2 + 8 * (e / 4) + (e % 4);
                        if (!POS_SCALE) s[rb][kb2][e] *= c2;
                        s[rb][kb2][e] = ((unsigned)(jj - lo2) <= span) ? s[rb][kb2][e] : kNegInf;
                    }
            } else if (!POS_SCALE) {
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2) s[rb][kb2] *= c2;
            }
        }
    }

    // Running-max update from the per-lane partial maxima of a tile (log2 units after the
    // scale), with the lazy rescale of O and l.
    __device__ __forceinline__ void finish_max(float (&mx)[RB]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float m = halves_max(mx[rb]);
            const float m_tile = POS_SCALE ? m * c2 : m;
            const bool need = m_tile > m_run[rb] + kRescaleSlack;
            if (__builtin_amdgcn_ballot_w64(need)) {
                keep_branch();
                const float alpha = need ? fast_exp2(m_run[rb] - m_tile) : 1.0f;
                m_run[rb] = need ? m_tile : m_run[rb];
                l_run[rb] *= alpha;
#pragma unroll
                for (int i = 0; i < G::DB; ++i) o[rb][i] *= alpha;
            }
        }
    }

    // Row max of a whole (masked) score tile, then the running-max update.
    __device__ __forceinline__ void update_max(const f32x16 (&s)[RB][2]) {
        float mx[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            mx[rb] = kNegInf;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int e = 0; e < 16; e += 2) mx[rb] = max3(mx[rb], s[rb][kb2][e], s[rb][kb2][e + 1]);
        }
        finish_max(mx);
    }

    // Second half of a pipelined step: this tile's P.V MFMAs (each V^T operand read two
    // steps ahead and shared by all row blocks) with a slice of the next tile's row max
    // after each of them; then the running-max update for the next tile.
    template <bool HAS_NEXT>
    __device__ __forceinline__ void pv_max_next(const bf16x8 (&pf)[RB][4], const lds_char* vbuf,
                                                const f32x16 (&nxt)[RB][2]) {
        constexpr int NJ = 4 * G::DB;   // V^T operands per tile
        constexpr int NP = 16 * RB;     // max3 steps of the next tile
        constexpr int PF = 2;           // V^T operands in flight
        float mx[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) mx[rb] = kNegInf;
        bf16x8 vf[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) vf[j] = v_frag(vbuf, j);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c4 = j / G::DB, db = j % G::DB;
            const bf16x8 v_now = vf[j % PF];
            if (j + PF < NJ) vf[j % PF] = v_frag(vbuf, j + PF);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                o[rb][db] = H::mfma32x32x16(v_now, pf[rb][c4], o[rb][db]);
            if constexpr (HAS_NEXT) {
#pragma unroll
                for (int q = j * NP / NJ; q < (j + 1) * NP / NJ; ++q) {
                    const int rb = q / 16, k = q % 16;
                    mx[rb] = max3(mx[rb], nxt[rb][k / 8][2 * (k % 8)], nxt[rb][k / 8][2 * (k % 8) + 1]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (HAS_NEXT) finish_max(mx);
    }
};

// Launch shape: RB row blocks of 32 query rows per wave, W waves per workgroup (sharing
// each K/V tile in LDS), MINB workgroups per CU.
template <int D>
struct Cfg {
    static_assert(D == 32 || D == 64, "head dim 128 runs the ping-pong kernel");
    static constexpr int RB = 1;
    static constexpr int W = 4;
    static constexpr int THREADS = 64 * W;
    static constexpr int BM = 32 * RB * W;          // query rows per workgroup
    static constexpr int MINB = 2;
};

// GATE: waves skip the work of key tiles none of their rows sees.  Only causal and banded
// launches have such tiles; the full bidirectional launch keeps the ungated stream, whose
// schedule the extra branches would only disturb (measured 39.9 vs 41.3 us on the padded
// BERT batch, both timed in the kernel's form for a non-positive scale).
template <int D, bool POS_SCALE, bool GATE, bool F16>
__global__ __launch_bounds__(Cfg<D>::THREADS, Cfg<D>::MINB) void prefill_bf16_narrow_kernel(PrefillArgs a) {
    constexpr int RB = Cfg<D>::RB;
    constexpr int W = Cfg<D>::W;
    constexpr int BM = Cfg<D>::BM;
    using G = Geo<D, W>;
    __shared__ __attribute__((aligned(16))) u32x4 k_lds[2][kBN * G::KS];
    __shared__ __attribute__((aligned(16))) u32x4 v_lds[2][kBN * G::CPR];

    Prefill<D, RB, W, POS_SCALE, F16> st;
    using H = Fmt16<F16>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave >= 0 && wave < W);
    const int g = lane >> 5;                  // half of the wave
    st.lane = lane;
    st.wave = wave;
    st.g = g;
    // block -> (q-tile, item, head): longest tiles first, XCD-aware (plan::map_block)
    const plan::BlockCoord bc = plan::map_block(blockIdx.x, a.n_qtiles, a.batch, a.q_heads, a.kv_heads,
                                                last_tiles_first(a), kXcds);
    const int qt = bc.qt, b = bc.b, h = bc.h;
    const int grp = a.q_heads / a.kv_heads;
    const int kvh = h / grp;

    const plan::Rows ir = item_rows(a, b, h, kvh, D);
    const int valid = ir.kv_valid;
    const int q_len = ir.q_len;
    st.kvalid = valid;
    st.kv_rs = ir.kv_rs;

    const int q0 = qt * BM;
    if (q0 >= q_len) return;   // no query row of this item in the tile (unpadded layout)
    const int last_row = min(q0 + BM, q_len) - 1;

    // ---- key tiles of the whole workgroup: the union of its rows' key sets -------------
    const plan::Tiles tiles = plan::key_tiles(
        plan::span_union(a.pos_offset + q0, a.pos_offset + last_row, valid, a.causal != 0, a.window), kBN);
    const int kt_begin = tiles.begin;
    const int kt_end = tiles.end;

    // ---- per row block: this lane's query row and key interval, the block's common keys
    int my_row[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r0 = q0 + (wave * RB + rb) * 32;
        my_row[rb] = r0 + (lane & 31);
        const RowBlockKeys k = row_block_keys(a, r0, 32, my_row[rb], q_len, valid);
        st.lo_r[rb] = k.lane.lo;
        st.hi_r[rb] = k.lane.hi;
        st.b_inter_lo[rb] = k.inter.lo;
        st.b_inter_hi[rb] = k.inter.hi;
        st.blk_all_rows_valid[rb] = k.all_rows_valid;
    }
    {   // the union of the key intervals of the wave's rows (all its row blocks)
        const int r0 = q0 + wave * RB * 32;
        const RowBlockKeys k = row_block_keys(a, r0, RB * 32, r0, q_len, valid);
        st.union_lo = k.uni.lo;
        st.union_hi = k.uni.hi;
    }

    // ---- Q^T operands: lane l holds row l%32 of each block, dims 16*kc + 8*g + [0, 8)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const uint16_t* qrow = (const uint16_t*)a.q + ir.q_base + (size_t)min(my_row[rb], q_len - 1) * ir.q_rs;
        const bool in = my_row[rb] < q_len;
#pragma unroll
        for (int kc = 0; kc < G::KC; ++kc) {
            u32x4 w = in ? *(const u32x4*)(qrow + 16 * kc + 8 * g) : u32x4{0, 0, 0, 0};
            st.qf[rb][kc] = __builtin_bit_cast(bf16x8, w);
        }
    }
    // Q is waited for in the prologue below, together with the first tile copies (one
    // memory latency instead of several).  That explicit wait also keeps the compiler from
    // placing its own wait for Q inside the loop, where it would also wait for the next
    // tile's copy.

    st.kg = (const char*)((const uint16_t*)a.k + ir.kv_base);
    st.vg = (const char*)((const uint16_t*)a.v + ir.kv_base);
    st.k_lds0 = lds_addr(k_lds[0]);
    st.v_lds0 = lds_addr(v_lds[0]);
#pragma unroll
    for (int ii = 0; ii < G::NKW; ++ii) st.koff[ii] = plan::chunk_offset(plan::narrow_k_chunk(wave + W * ii, lane, G::CPR), ir.kv_rs);
    st.voff = plan::chunk_offset(plan::narrow_v_chunk(wave, lane, D), ir.kv_rs);
    st.v_step = plan::narrow_v_copy_step(W, D, ir.kv_rs);
    st.k_read = ((lane & 31) * G::KS + g) * 16;
    {
        const int r = 4 * g + ((lane & 15) >> 2);
#pragma unroll
        for (int db = 0; db < G::DB; ++db) {
            const int cb = 64 * db + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);   // column byte
            st.v_read[db] = r * 2 * D + 16 * ((cb >> 4) ^ plan::narrow_vswz(r, D)) + (cb & 15);
        }
    }
    st.c2 = a.scale * kLog2e;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int i = 0; i < G::DB; ++i) st.o[rb][i] = f32x16{};
        st.m_run[rb] = kNegInf;   // running (possibly stale) max of this lane's row, log2 units
        st.l_run[rb] = 0.0f;      // running sum over this lane's half of the keys
    }

    const lds_char* kb[2] = {(const lds_char*)(const void*)k_lds[0], (const lds_char*)(const void*)k_lds[1]};
    const lds_char* vb[2] = {(const lds_char*)(const void*)v_lds[0], (const lds_char*)(const void*)v_lds[1]};

    // One pipelined step for tile kt = kt_begin + j (buffer parity PAR = j & 1): cur holds
    // the masked scores of tile kt with the running max already updated for it.
    auto step = [&](auto has_next_c, auto par_c, f32x16 (&cur)[RB][2], f32x16 (&nxt)[RB][2], int j) {
        constexpr bool HAS_NEXT = decltype(has_next_c)::value;
        constexpr int PAR = decltype(par_c)::value;
        const int kt = kt_begin + j;
        wait_vm0();          // this thread's copies of K(kt+1) and V(kt) have landed
        __syncthreads();     // ... everyone's; and nobody still reads K(kt) or V(kt-1)
        if (kt + 2 < kt_end) st.copy_k(kt + 2, PAR);
        if (HAS_NEXT) st.copy_v(kt + 1, PAR ^ 1);
        bf16x8 pf[RB][4];
        // Wave-uniform: whether this wave has rows that see tile kt (its softmax and P.V)
        // and tile kt+1 (its Q.K^T, mask and max).
        const bool see_cur = !GATE || st.wave_sees(kt);
        const bool see_nxt = HAS_NEXT && (!GATE || st.wave_sees(kt + 1));
        if (!GATE || (see_cur && see_nxt)) {
            st.template qk_next_probs<HAS_NEXT>(nxt, cur, pf, kb[PAR ^ 1]);
            if (HAS_NEXT) st.mask_scale(nxt, kt + 1);
            st.template pv_max_next<HAS_NEXT>(pf, vb[PAR], nxt);
        } else if (see_cur && see_nxt) {
            st.template qk_next_probs<true>(nxt, cur, pf, kb[PAR ^ 1]);
            st.mask_scale(nxt, kt + 1);
            st.template pv_max_next<true>(pf, vb[PAR], nxt);
        } else if (see_cur) {
            keep_branch();
            st.probs_only(cur, pf);
            st.template pv_max_next<false>(pf, vb[PAR], nxt);
        } else if (see_nxt) {
            keep_branch();
            st.qk(nxt, kb[PAR ^ 1]);
            st.mask_scale(nxt, kt + 1);
            st.update_max(nxt);
        }
    };

    const int n = kt_end - kt_begin;
    if (n > 0) {
        f32x16 sa[RB][2], sb[RB][2];
        st.copy_k(kt_begin, 0);
        if (n > 1) st.copy_k(kt_begin + 1, 1);
        st.copy_v(kt_begin, 0);
        wait_vm0();          // Q, K(0), K(1) and V(0) have landed
        __syncthreads();
        if (!GATE || st.wave_sees(kt_begin)) {
            st.qk(sa, kb[0]);
            st.mask_scale(sa, kt_begin);
            st.update_max(sa);
        }
        typedef std::integral_constant<bool, true> T_;
        typedef std::integral_constant<bool, false> F_;
        typedef std::integral_constant<int, 0> P0;
        typedef std::integral_constant<int, 1> P1;
        int j = 0;
        for (; j + 2 < n; j += 2) {
            step(T_{}, P0{}, sa, sb, j);
            step(T_{}, P1{}, sb, sa, j + 1);
        }
        if (j + 1 < n) {
            step(T_{}, P0{}, sa, sb, j);
            step(F_{}, P1{}, sb, sa, j + 1);
        } else {
            step(F_{}, P0{}, sa, sb, j);
        }
    }

    // ---- epilogue: normalise, zero padded / empty rows, store bf16 --------------------
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float l_tot = halves_sum(st.l_run[rb]);
        if (my_row[rb] < q_len) {
            const float inv = (st.hi_r[rb] >= 0 && l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
            uint16_t* orow = (uint16_t*)a.out + ir.q_base + (size_t)my_row[rb] * ir.q_rs;
#pragma unroll
            for (int db = 0; db < G::DB; ++db) {
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int d = 32 * db + 8 * e4 + 4 * g;
                    u32x2 w;
                    w[0] = H::pack2(st.o[rb][db][4 * e4] * inv, st.o[rb][db][4 * e4 + 1] * inv);
                    w[1] = H::pack2(st.o[rb][db][4 * e4 + 2] * inv, st.o[rb][db][4 * e4 + 3] * inv);
                    *(u32x2*)(orow + d) = w;
                }
            }
        }
    }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
    PrefillArgs args = a;
    args.n_qtiles = (a.q_len + Cfg<D>::BM - 1) / Cfg<D>::BM;
    const dim3 grid((unsigned)args.n_qtiles * a.q_heads * a.batch);
    const dim3 block(Cfg<D>::THREADS);
    const bool gate = a.causal || a.window > 0;
    if (args.f16) {
        if (args.scale > 0.0f) {
            if (gate)
                hipLaunchKernelGGL((prefill_bf16_narrow_kernel<D, true, true, true>), grid, block, 0, stream, args);
            else
                hipLaunchKernelGGL((prefill_bf16_narrow_kernel<D, true, false, true>), grid, block, 0, stream, args);
        } else {
            hipLaunchKernelGGL((prefill_bf16_narrow_kernel<D, false, true, true>), grid, block, 0, stream, args);
        }
    } else {
        if (args.scale > 0.0f) {
            if (gate)
                hipLaunchKernelGGL((prefill_bf16_narrow_kernel<D, true, true, false>), grid, block, 0, stream, args);
            else
                hipLaunchKernelGGL((prefill_bf16_narrow_kernel<D, true, false, false>), grid, block, 0, stream, args);
        } else {
            hipLaunchKernelGGL((prefill_bf16_narrow_kernel<D, false, true, false>), grid, block, 0, stream, args);
        }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16_narrow(const PrefillArgs& a, int head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 32: return launch_d<32>(a, stream);
        case 64: return launch_d<64>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mi_attn
