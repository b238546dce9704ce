// prefill_bf16.hip -- fused attention prefill for 16-bit inputs (bf16, and fp16 through
// the same code with the fp16 MFMA) on gfx950 matrix cores (head dim 128; head dims 32
// and 64 run prefill_bf16_narrow.hip).
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
// Work decomposition: one workgroup = 8 waves = 256 query rows of one (item, head);
// wave w owns rows [32w, 32w+32).  The grid is one-dimensional with the q-tile index
// slowest (longest tiles first) and XCD-aware.  Key tiles of 64 rows of K and V
// are copied from HBM straight into LDS (global_load_lds_dwordx4, 16 bytes per lane, no
// registers, per-lane offsets computed once), double buffered.
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
// Ping-pong: the work of a tile splits into a matrix phase M(t) -- the Q.K^T MFMAs of
// tile t+1 and the P.V MFMAs of tile t -- and a vector phase V(t) -- mask, row max and
// exp/pack of tile t+1.  Waves 0-3 and waves 4-7 (one of each on every SIMD) run the
// same sequence one phase apart, with a workgroup barrier after every phase, so each
// SIMD always has one wave on the matrix core and one on the vector ALU.
//
// Softmax bookkeeping per tile, for scale > 0, with c = scale*log2(e): bf16 Q is
// multiplied by c once, as it is loaded (and rounded to bf16 again), and each tile's Q.K^T
// accumulators start from minus the running max m, so the MFMAs leave s*c - m, the
// exponent of p = exp2(s*c - m) itself, and the vector phase spends no instruction per
// score on the scale.  fp16 Q does the same when c <= 1 (then |c*q| <= |q| stays within
// fp16's range); with a larger scale it keeps the unscaled form, p = exp2(fma(s, c, -m)),
// since c*q could overflow fp16 where the fp32 product does not.
// The running max is only moved (and O, l rescaled) when the tile's max exceeds it by
// more than 2^8; otherwise the stale max is kept, p <= 256, and the final O / l is
// unchanged because numerator and denominator share it.
//
// LDS layout: operand-linear 1 KiB blocks, no padding and no swizzle.  Copy f of a K tile
// places at byte 16*l of block f exactly the 16 bytes lane l's MFMA A operand needs, and
// copy j of a V tile places what lane l's two transposing reads need at 8*l of two
// 512-byte blocks (plan::wide_k_chunk, plan::wide_v_chunk).  Every operand read is then
// one contiguous 1 KiB (or 512-byte) access with no bank conflict.
#include <type_traits>

#include "prefill_common.hpp"

namespace mi_attn {
namespace {

constexpr int kBN = plan::WideGeo<128>::BN;            // keys per tile
constexpr int kWaves = plan::WideGeo<128>::WAVES;       // two groups of four, one wave of each per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = plan::WideGeo<128>::BM;             // query rows per workgroup
constexpr int kCopyWaves = plan::WideGeo<128>::COPY_WAVES;   // the trailing group issues every tile copy
constexpr float kRescaleSlack = 8.0f;  // log2 units the stale max may lag behind

template <int D>
using Geo = plan::WideGeo<D>;

// FOLD16: fp16 with c = scale*log2(e) <= 1, where c*q cannot overflow fp16 either.
template <int D, bool POS_SCALE, bool F16, bool FOLD16>
struct Prefill {
    using G = Geo<D>;
    using H = Fmt16<F16>;
    // Q carries the scale and the accumulators the running max: bf16 with a positive
    // scale, fp16 when the scale also keeps c*q within fp16's range
    static constexpr bool FOLD = POS_SCALE && (!F16 || FOLD16);

    // ---- per-lane constants ---------------------------------------------------------
    int lane, wave, g;
    int cw;                     // index among the copying waves (group 1)
    int kvalid;                 // valid key rows of this item
    int kv_rs;                  // elements from one K/V row to the next
    const char* kg;             // K rows of this (item, kv head)
    const char* vg;
    uint32_t k_lds0, v_lds0;    // LDS byte addresses of buffer 0
    uint32_t k_off;             // byte offset of this lane's K copy chunk from a copy's base
    uint32_t v_off;             // ... V
    uint32_t k_cb[G::NKW];      // byte offset of this wave's K copy ii from the tile base (uniform)
    uint32_t v_cb[G::NVW];      // ... V
    int lo_r, hi_r;             // this lane's key interval
    int inter_lo, inter_hi;     // keys every row of the wave that sees a key sees
    int union_lo, union_hi;     // keys some row of the wave sees (a superset; empty if hi < lo)
    float c2;                   // scale * log2(e)

    // ---- running state ----------------------------------------------------------------
    bf16x8 qf[G::KC];
    f32x16 o[G::DB];
    f32x16 s[2];                // scores of the tile the next vector phase works on
    bf16x8 pf[4];               // probabilities of the tile the next matrix phase uses
    float m_run, l_run;
    f32x16 acc0;                // FOLD: what Q.K^T accumulators start from, -m_run (0 before any key)

    // K tile layout in LDS: 1 KiB block f = kb2*KC + kc holds, at 16*p, the chunk 2kc + p/32
    // (dims 16kc + 8(p/32) + [0, 8)) of key 32*kb2 + p%32 -- exactly the MFMA A operand of
    // lane p, so every K operand read is the lane-linear base + 16*lane.  Copy f fills block
    // f (plan::wide_k_chunk): a per-lane offset plus a per-copy base for whole tiles; tail
    // tiles clamp their rows to the last valid key, addressed from the tile base.
    __device__ __forceinline__ void copy_k(int kt, int par) const {
        const char* base = kg + (size_t)kt * kBN * kv_rs * 2;
        const uint32_t lds = k_lds0 + par * G::K_BYTES + cw * 1024;
        if (kt * kBN + kBN <= kvalid) {   // the whole tile is valid: per-copy bases precomputed
#pragma unroll
            for (int ii = 0; ii < G::NKW; ++ii) lds_dma16(base + k_cb[ii], k_off, lds + kCopyWaves * ii * 1024);
        } else {
            keep_branch();
#pragma unroll
            for (int ii = 0; ii < G::NKW; ++ii) {
                plan::Chunk c = plan::wide_k_chunk(cw + kCopyWaves * ii, lane, G::KC);
                c.row = plan::tail_row(c.row, kvalid, kt * kBN);
                lds_dma16(base, plan::chunk_offset(c, kv_rs), lds + kCopyWaves * ii * 1024);
            }
        }
    }

    // V tile layout in LDS: 512-byte block 2j + hi (j = c4*DB + db) holds, at 8*l, what
    // lane l reads in the transposing read of V^T operand j, half hi: key
    // 16c4 + 8hi + 4(l/32) + (l%16)/4, dims 32db + 16((l/16)%2) + 4(l%4) + [0, 4).  So both
    // transposing reads are the lane-linear base + 8*lane (+512).  Copy j fills blocks 2j,
    // 2j+1 (plan::wide_v_chunk), addressed like the K copies.
    __device__ __forceinline__ void copy_v(int kt, int par) const {
        const char* base = vg + (size_t)kt * kBN * kv_rs * 2;
        const uint32_t lds = v_lds0 + par * G::V_BYTES + cw * 1024;
        if (kt * kBN + kBN <= kvalid) {
#pragma unroll
            for (int ii = 0; ii < G::NVW; ++ii) lds_dma16(base + v_cb[ii], v_off, lds + kCopyWaves * ii * 1024);
        } else {
            keep_branch();
#pragma unroll
            for (int ii = 0; ii < G::NVW; ++ii) {
                plan::Chunk c = plan::wide_v_chunk(cw + kCopyWaves * ii, lane, G::DB);
                c.row = plan::tail_row(c.row, kvalid, kt * kBN);
                lds_dma16(base, plan::chunk_offset(c, kv_rs), lds + kCopyWaves * ii * 1024);
            }
        }
    }

    // K operand f of a tile (32-key block f/KC, k-step f%KC): key l%32 of the block,
    // dims 16*kc + 8*g + [0, 8).
    __device__ __forceinline__ bf16x8 k_frag(const lds_char* kbuf, int f) const {
        return __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(kbuf + f * 1024 + lane * 16));
    }

    // V^T operand j of a tile (j = 16-key chunk * DB + 32-dim block) via two transposing
    // reads.  Within 16-lane group G = lane/16, source lane s supplies key
    // 16*c4 + 4*g + s/4 (+8 for the second read), dims 32*db + 16*(G%2) + 4*(s%4).
    __device__ __forceinline__ bf16x8 v_frag(const lds_char* vbuf, int j) const {
        const lds_char* p = vbuf + j * 1024 + lane * 8;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 512));
        typedef __attribute__((ext_vector_type(8))) short s16x8;
        const s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, vv);
    }

    // Matrix phase: S^T of the next tile (when there is one) from the K buffer, then
    // O^T += V^T P^T of the current tile (when there is one) from the V buffer.  Operands
    // are read from LDS a few MFMAs ahead of their use.
    // Whether key tile kt holds a key that some row of this wave sees.  Tiles that hold
    // none (the far side of the causal diagonal, outside the band) take no MFMA and no
    // softmax work in this wave; the other waves of the workgroup still need them.
    __device__ __forceinline__ bool wave_sees(int kt) const {
        return kt * kBN <= union_hi && kt * kBN + kBN - 1 >= union_lo;
    }

    __device__ __forceinline__ void matrix_phase(bool do_qk, const lds_char* kbuf, bool do_pv, const lds_char* vbuf) {
        constexpr int NF = 2 * G::KC;   // K operands per tile
        constexpr int NJ = 4 * G::DB;   // V^T operands per tile

        if (do_qk) {
            constexpr int PF = 4;
            bf16x8 kf[PF];
            // step f works on block kb2 = f%2, k-step kc = f/2: consecutive MFMAs alternate
            // between the two accumulation chains
            auto blk = [](int f) { return (f % 2) * G::KC + f / 2; };
            const f32x16 c0 = FOLD ? acc0 : f32x16{};
#pragma unroll
            for (int f = 0; f < PF; ++f) kf[f] = k_frag(kbuf, blk(f));
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int kb2 = f % 2, kc = f / 2;
                const bf16x8 k_now = kf[f % PF];
                if (f + PF < NF) kf[f % PF] = k_frag(kbuf, blk(f + PF));
                s[kb2] = H::mfma32x32x16(k_now, qf[kc], kc == 0 ? c0 : s[kb2]);
                __builtin_amdgcn_sched_barrier(0);   // keep the reads PF steps ahead, no further
            }
        }
        if (do_pv) {
            constexpr int PF = 3;
            bf16x8 vf[PF];
#pragma unroll
            for (int j = 0; j < PF; ++j) vf[j] = v_frag(vbuf, j);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int c4 = j / G::DB, db = j % G::DB;
                const bf16x8 v_now = vf[j % PF];
                if (j + PF < NJ) vf[j % PF] = v_frag(vbuf, j + PF);
                o[db] = H::mfma32x32x16(v_now, pf[c4], o[db]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // Vector phase for tile kt (its scores are in s): mask the rows that do not see every
    // key of it (scaling them when the scale is not positive), row max and lazy rescale,
    // then probabilities -> packed bf16 P^T operands and the row sum.  Element e of block
    // kb2 is key kt*64 + 32*kb2 + 8*(e/4) + 4*g + e%4; P chunk c4 (16 keys) = block c4/2,
    // elements 8*(c4%2) + [0, 8).
    // FULL: the caller knows that every row of the workgroup sees every key of tile kt
    // (then no wave can skip it and no element needs a test), and the phase runs without
    // those checks and their branches.
    template <bool FULL = false>
    __device__ __forceinline__ void vector_phase(int kt) {
        // Issue priority: the other wave on this SIMD is in its matrix phase.  The vector
        // phase is a dense stream of independent VALU instructions, and MFMAs issue through
        // the same port; by age the vector wave would win it whenever it is the older one
        // and starve the matrix core.  So this phase runs at priority 0 and hands the wave
        // back priority 2 at its end -- before the barrier, so that the priority is already
        // in place when the following matrix phase starts.
        __builtin_amdgcn_s_setprio(0);
        if (!FULL && !wave_sees(kt)) {   // no score of this tile was computed, and none is used
            __builtin_amdgcn_s_setprio(2);
            return;
        }
        const int kbase = kt * kBN;
        const bool full = FULL || (kbase >= inter_lo && kbase + kBN - 1 <= inter_hi);
        if (!full) {
            keep_branch();
            // key jj is kept iff lo <= jj <= hi, tested as one unsigned compare
            // (jj - lo) <= (hi - lo): no scalar mask arithmetic between the compares
            const int lo = lo_r - kbase - 4 * g, hi = hi_r - kbase - 4 * g;
            const int lo2 = hi >= lo ? lo : (1 << 30);        // empty interval: nothing kept
            const unsigned span = hi >= lo ? (unsigned)(hi - lo) : 0u;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int jj = 32 * kb2 + 8 * (e / 4) + (e % 4);
                    if (!POS_SCALE) s[kb2][e] *= c2;
                    s[kb2][e] = ((unsigned)(jj - lo2) <= span) ? s[kb2][e] : kNegInf;
                }
        } else if (!POS_SCALE) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) s[kb2] *= c2;
        }

        float mx = kNegInf;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int e = 0; e < 16; e += 2) mx = max3(mx, s[kb2][e], s[kb2][e + 1]);
        mx = halves_max(mx);
        // FOLD: the scores are already s*c - m_ref, with m_ref what the accumulators
        // started from (m_run has not moved since this tile's Q.K^T)
        const float m_ref = m_run == kNegInf ? 0.0f : m_run;
        const float m_tile = FOLD ? m_ref + mx : POS_SCALE ? mx * c2 : mx;
        const bool need = m_tile > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(need)) {
            keep_branch();
            const float alpha = need ? fast_exp2(m_run - m_tile) : 1.0f;
            if constexpr (FOLD) {   // re-reference this tile's exponents to the new max
                const float d = need ? m_tile - m_ref : 0.0f;
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2) s[kb2] -= d;
            }
            m_run = need ? m_tile : m_run;
            if constexpr (FOLD) acc0 = f32x16{} - (m_run == kNegInf ? 0.0f : m_run);
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < G::DB; ++i) o[i] *= alpha;
        }

        const float m_use = m_run == kNegInf ? 0.0f : m_run;
        float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            u32x4 w;
#pragma unroll
            for (int jj = 0; jj < 8; jj += 2) {
                const float s0 = s[c4 / 2][8 * (c4 % 2) + jj], s1 = s[c4 / 2][8 * (c4 % 2) + jj + 1];
                const float p0 = FOLD ? fast_exp2(s0) : POS_SCALE ? fast_exp2(fmaf(s0, c2, -m_use)) : fast_exp2(s0 - m_use);
                const float p1 = FOLD ? fast_exp2(s1) : POS_SCALE ? fast_exp2(fmaf(s1, c2, -m_use)) : fast_exp2(s1 - m_use);
                w[jj / 2] = H::pack2(p0, p1);
                ls0 += p0;
                ls1 += p1;
            }
            pf[c4] = __builtin_bit_cast(bf16x8, w);
        }
        l_run += ls0 + ls1;
        __builtin_amdgcn_s_setprio(2);
    }
};

template <int D, bool POS_SCALE, bool F16, bool FOLD16>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(PrefillArgs a) {
    using G = Geo<D>;
    __shared__ __attribute__((aligned(16))) u32x4 k_lds[2][kBN * G::CPR];
    __shared__ __attribute__((aligned(16))) u32x4 v_lds[2][kBN * G::CPR];

    Prefill<D, POS_SCALE, F16, FOLD16> st;
    using H = Fmt16<F16>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;                  // half of the wave
    const int grp = wave / 4;                 // ping-pong group: 0 leads, 1 trails a phase
    st.lane = lane;
    st.wave = wave;
    st.g = g;
    st.cw = wave - 4;
    // block -> (q-tile, item, head): longest tiles first, XCD-aware (plan::map_block)
    const plan::BlockCoord bc = plan::map_block(blockIdx.x, a.n_qtiles, a.batch, a.q_heads, a.kv_heads,
                                                last_tiles_first(a), kXcds);
    const int qt = bc.qt, b = bc.b, h = bc.h;
    const int kvh = h / (a.q_heads / a.kv_heads);

    const plan::Rows ir = item_rows(a, b, h, kvh, D);
    const int valid = ir.kv_valid;
    const int q_len = ir.q_len;
    st.kvalid = valid;
    st.kv_rs = ir.kv_rs;

    const int q0 = qt * kBM;
    if (q0 >= q_len) return;   // no query row of this item in the tile (unpadded layout)
    const int last_row = min(q0 + kBM, q_len) - 1;

    // ---- key tiles of the whole workgroup, and those every row sees in full -------------
    const bool causal = a.causal != 0;
    const int p_lo = a.pos_offset + q0;
    const int p_hi = a.pos_offset + last_row;
    const plan::Tiles tiles = plan::key_tiles(plan::span_union(p_lo, p_hi, valid, causal, a.window), kBN);
    const int kt_begin = tiles.begin;
    const int kt_end = tiles.end;
    plan::Keys full = plan::span_inter(p_lo, p_hi, valid, causal, a.window);
    if (p_hi >= valid || q0 + kBM > q_len) full.hi = -1;   // some row is padding or past the end
    // the loop runs V(t) on tile kt_begin + t + 1, t in [0, n-1): tiles of t in [ta, tb) are full
    const int nv = max(kt_end - kt_begin - 1, 0);   // vector phases in the loop
    int ta = 0, tb = 0;
    if (full.hi >= full.lo) {
        const int f0 = (full.lo + kBN - 1) / kBN, f1 = (full.hi + 1) / kBN;   // full tiles [f0, f1)
        ta = min(max(f0 - kt_begin - 1, 0), nv);
        tb = min(max(f1 - kt_begin - 1, ta), nv);
    }
    typedef std::integral_constant<bool, true> T_;
    typedef std::integral_constant<bool, false> F_;

    // ---- this lane's query row and key interval, the wave's common keys ----------------
    const int r0 = q0 + wave * 32;
    const int my_row = r0 + (lane & 31);
    {
        const RowBlockKeys k = row_block_keys(a, r0, 32, my_row, q_len, valid);
        st.lo_r = k.lane.lo;
        st.hi_r = k.lane.hi;
        st.inter_lo = k.inter.lo;
        st.inter_hi = k.inter.hi;
        st.union_lo = k.uni.lo;
        st.union_hi = k.uni.hi;
    }

    // ---- Q^T operand: lane l holds row l%32, dims 16*kc + 8*g + [0, 8) ---------------
    {
        const uint16_t* qrow = (const uint16_t*)a.q + ir.q_base + (size_t)min(my_row, q_len - 1) * ir.q_rs;
        const bool in = my_row < q_len;
#pragma unroll
        for (int kc = 0; kc < G::KC; ++kc) {
            u32x4 w = in ? *(const u32x4*)(qrow + 16 * kc + 8 * g) : u32x4{0, 0, 0, 0};
            if constexpr (Prefill<D, POS_SCALE, F16, FOLD16>::FOLD) {   // c*q, rounded to 16 bits (nearest, ties to even)
                const float c = a.scale * kLog2e;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = H::pack2(H::lo(w[i]) * c, H::hi(w[i]) * c);
            }
            st.qf[kc] = __builtin_bit_cast(bf16x8, w);
        }
    }
    // Q is waited for in the prologue below, together with the first tile copies (one
    // memory latency instead of two).  That explicit wait also keeps the compiler from
    // placing its own wait for Q inside the loop, where it would also wait for the tile
    // copies in flight.

    st.kg = (const char*)((const uint16_t*)a.k + ir.kv_base);
    st.vg = (const char*)((const uint16_t*)a.v + ir.kv_base);
    st.k_lds0 = lds_addr(k_lds[0]);
    st.v_lds0 = lds_addr(v_lds[0]);
    st.k_off = plan::wide_k_lane_off(lane, ir.kv_rs);
#pragma unroll
    for (int ii = 0; ii < G::NKW; ++ii) st.k_cb[ii] = plan::wide_k_copy_base(st.cw + kCopyWaves * ii, ir.kv_rs, G::KC);
    st.v_off = plan::wide_v_lane_off(lane, ir.kv_rs);
#pragma unroll
    for (int ii = 0; ii < G::NVW; ++ii) st.v_cb[ii] = plan::wide_v_copy_base(st.cw + kCopyWaves * ii, ir.kv_rs, G::DB);
    st.c2 = a.scale * kLog2e;
#pragma unroll
    for (int i = 0; i < G::DB; ++i) st.o[i] = f32x16{};
    st.m_run = kNegInf;    // running (possibly stale) max of this lane's row, log2 units
    st.acc0 = f32x16{};
    st.l_run = 0.0f;       // running sum over this lane's half of the keys

    // ---- the phase sequence ------------------------------------------------------------
    // With n tiles (relative index t = 0..n-1) a wave runs M(-1) V(-1) M(0) V(0) ... M(n-1):
    // M(t) = S of tile t+1 (if t+1 < n) and O += P V of tile t (if t >= 0), V(t) = vector
    // phase of tile t+1 (if t+1 < n).  Group 0 runs phase p in slot p, group 1 in slot
    // p+1; every slot ends with a workgroup barrier (2n+3 slots in all).
    // Tiles: K(t+1) and V(t) are read in slots 2t+2 and 2t+3.  For t >= 1 they are copied
    // in slot 2t (into the buffers of K(t-1) and V(t-2), last read in slot 2t-1) and
    // waited for at the end of slot 2t+1; K(0), V(0) and K(1) are copied before slot 0.
    const int n = kt_end - kt_begin;
    const lds_char* kb0 = (const lds_char*)(const void*)k_lds[0];
    const lds_char* vb0 = (const lds_char*)(const void*)v_lds[0];
    auto kbuf = [&](int t) { return kb0 + (t & 1) * G::K_BYTES; };
    auto vbuf = [&](int t) { return vb0 + (t & 1) * G::V_BYTES; };
    auto copies = [&](int t) {   // the copies of even slot 2t (t >= 1), issued by group 1
        if (t + 1 < n) st.copy_k(kt_begin + t + 1, (t + 1) & 1);
        if (t < n) st.copy_v(kt_begin + t, t & 1);
    };
    auto slot_end = [&](bool odd) {
        if (odd) wait_vm0();   // this wave's copies of the previous slot have landed
        __syncthreads();
    };
    if (n > 0) {
        __builtin_amdgcn_s_setprio(2);   // matrix phases run at priority 2, vector phases at 0
        if (grp == 1) {
            st.copy_k(kt_begin, 0);
            st.copy_v(kt_begin, 0);
            if (n > 1) st.copy_k(kt_begin + 1, 1);
        }
        wait_vm0();   // Q, and group 1's first tile copies, have landed
        __syncthreads();
        if (grp == 0) {
            st.matrix_phase(st.wave_sees(kt_begin), kbuf(0), false, vbuf(0));           // slot 0: M(-1)
            slot_end(false);
            st.vector_phase(kt_begin);                                 // slot 1: V(-1)
            slot_end(true);
            auto body0 = [&](int t, auto full_c) {
                st.matrix_phase(st.wave_sees(kt_begin + t + 1), kbuf(t + 1), st.wave_sees(kt_begin + t), vbuf(t));     // slot 2t+2: M(t)
                slot_end(false);
                st.template vector_phase<decltype(full_c)::value>(kt_begin + t + 1);   // slot 2t+3: V(t)
                slot_end(true);
            };
            int t = 0;
            for (; t < ta; ++t) body0(t, F_{});
            for (; t < tb; ++t) body0(t, T_{});
            for (; t + 1 < n; ++t) body0(t, F_{});
            st.matrix_phase(false, kbuf(0), st.wave_sees(kt_begin + n - 1), vbuf(n - 1));        // slot 2n: M(n-1)
            slot_end(false);
            slot_end(true);                                            // slot 2n+1
            slot_end(false);                                           // slot 2n+2
        } else {
            slot_end(false);                                           // slot 0
            st.matrix_phase(st.wave_sees(kt_begin), kbuf(0), false, vbuf(0));           // slot 1: M(-1)
            slot_end(true);
            copies(1);                                                 // slot 2: V(-1)
            st.vector_phase(kt_begin);
            slot_end(false);
            auto body1 = [&](int t, auto full_c) {
                st.matrix_phase(st.wave_sees(kt_begin + t + 1), kbuf(t + 1), st.wave_sees(kt_begin + t), vbuf(t));     // slot 2t+3: M(t)
                slot_end(true);
                copies(t + 2);                                         // slot 2t+4: V(t)
                st.template vector_phase<decltype(full_c)::value>(kt_begin + t + 1);
                slot_end(false);
            };
            int t = 0;
            for (; t < ta; ++t) body1(t, F_{});
            for (; t < tb; ++t) body1(t, T_{});
            for (; t + 1 < n; ++t) body1(t, F_{});
            st.matrix_phase(false, kbuf(0), st.wave_sees(kt_begin + n - 1), vbuf(n - 1));        // slot 2n+1: M(n-1)
            slot_end(true);
            slot_end(false);                                           // slot 2n+2
        }
    }

    // ---- epilogue: normalise, zero padded / empty rows, store in the input format -----
    const float l_tot = halves_sum(st.l_run);
    if (my_row >= q_len) return;
    // a row that sees no key is written as zeros by a select, whatever its (unmasked) sums
    const bool keep = st.hi_r >= 0 && l_tot > 0.0f;
    const float inv = keep ? 1.0f / l_tot : 0.0f;
    uint16_t* orow = (uint16_t*)a.out + ir.q_base + (size_t)my_row * ir.q_rs;
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const int d = 32 * db + 8 * e4 + 4 * g;
            u32x2 w;
            w[0] = H::pack2(keep ? st.o[db][4 * e4] * inv : 0.0f, keep ? st.o[db][4 * e4 + 1] * inv : 0.0f);
            w[1] = H::pack2(keep ? st.o[db][4 * e4 + 2] * inv : 0.0f, keep ? st.o[db][4 * e4 + 3] * inv : 0.0f);
            *(u32x2*)(orow + d) = w;
        }
    }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
    PrefillArgs args = a;
    args.n_qtiles = (a.q_len + kBM - 1) / kBM;
    const dim3 grid((unsigned)args.n_qtiles * a.q_heads * a.batch);
    const dim3 block(kThreads);
    if (args.f16) {
        // c as the kernel computes it (one float product): c <= 1 here means |c*q| <= |q| there
        const bool fold16 = args.scale * kLog2e <= 1.0f;
        if (args.scale > 0.0f && fold16)
            hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, true>), grid, block, 0, stream, args);
        else if (args.scale > 0.0f)
            hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, false>), grid, block, 0, stream, args);
        else
            hipLaunchKernelGGL((prefill_bf16_kernel<D, false, true, false>), grid, block, 0, stream, args);
    } else {
        if (args.scale > 0.0f)
            hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, false>), grid, block, 0, stream, args);
        else
            hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, false>), grid, block, 0, stream, args);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 32:
        case 64: return launch_prefill_bf16_narrow(a, head_dim, stream);
        case 128: return launch_d<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mi_attn
