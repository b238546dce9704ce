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
    int kv_rs;                  // elements from one K/V row to the next
    uint32_t k_lds0, v_lds0;    // LDS byte addresses of buffer 0
    uint32_t koff[G::NKW];      // byte offsets of this lane's K copy chunks inside a tile
    uint32_t voff;              // ... V (first copy; copy ii reads v_step * ii bytes further)
    size_t v_step;              // byte distance between the rows of consecutive V copies
    int k_read;                 // LDS byte offset of this lane's K operand (row l%32, chunk g)
    int v_read[G::DB];          // LDS byte offsets of this lane's transposing V reads
    // the q-tile whose scores the next Q.K^T produces (its mask)
    int lo_r[RB], hi_r[RB];     // this lane's key interval, per row block
    int b_inter_lo[RB], b_inter_hi[RB];  // keys every row of a row block that sees a key sees
    float c2;                   // scale * log2(e)

    // ---- running state ----------------------------------------------------------------
    bf16x8 qf[RB][G::KC];
    f32x16 o[RB][G::DB];
    float m_run[RB], l_run[RB];

    // Tile copies (addresses from plan::narrow_k_chunk / narrow_v_chunk).  The tail case
    // (rows past the valid length repeat the last valid row, clamped from the tile base) is
    // decided once per tile; whole tiles use the precomputed per-lane offsets.
    // kg / vg: K / V rows of the tile's (item, kv head); kvalid: its valid keys.
    __device__ __forceinline__ void copy_k(const char* kg, int kvalid, int kt, int par) {
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

    __device__ __forceinline__ void copy_v(const char* vg, int kvalid, int kt, int par) {
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

    // S^T = K_tile . Q^T for every row block (no softmax work to interleave).
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

    // Whether key tile kt holds a key of uni, the keys some row of this wave sees in a
    // q-tile.  A tile that holds none (outside the band, past the causal diagonal) takes no
    // MFMA and no softmax work in this wave; the other waves of the workgroup may still
    // need it.
    static __device__ __forceinline__ bool wave_sees(plan::Keys uni, int kt) {
        return kt * kBN <= uni.hi && kt * kBN + kBN - 1 >= uni.lo;
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

    // First half of a pipelined step, as one explicitly ordered stream: the Q.K^T MFMAs
    // of the next tile (each K operand read from LDS four steps ahead of its use and
    // shared by all row blocks) with a slice of this tile's softmax after each of them.
    // sched_barrier(0) keeps the compiler from regrouping the MFMAs.
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
            const bool full = kbase >= b_inter_lo[rb] && kbase + kBN - 1 <= b_inter_hi[rb];
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

    // Per-lane partial row max of a whole (masked) score tile (finish_max completes it).
    __device__ __forceinline__ void row_max(const f32x16 (&s)[RB][2], float (&mx)[RB]) const {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            mx[rb] = kNegInf;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int e = 0; e < 16; e += 2) mx[rb] = max3(mx[rb], s[rb][kb2][e], s[rb][kb2][e + 1]);
        }
    }

    // Second half of a pipelined step: this tile's P.V MFMAs (each V^T operand read two
    // steps ahead and shared by all row blocks) with a slice of the next tile's row max
    // after each of them (per lane, in mx; finish_max turns it into the running-max update).
    template <bool HAS_NEXT>
    __device__ __forceinline__ void pv_max_next(const bf16x8 (&pf)[RB][4], const lds_char* vbuf,
                                                const f32x16 (&nxt)[RB][2], float (&mx)[RB]) {
        constexpr int NJ = 4 * G::DB;   // V^T operands per tile
        constexpr int NP = 16 * RB;     // max3 steps of the next tile
        constexpr int PF = 2;           // V^T operands in flight
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

// One q-tile of a workgroup's list (in LDS): where its rows live and which key tiles it
// visits.  kind 0: key tiles [kt_begin, kt_end) to visit; 1: rows that see no key (written
// as zeros).
struct TileEnt {
    unsigned long long q_base, kv_base;   // element offsets of row 0 (plan::Rows)
    int q0, q_len, kvalid, kt_begin, kt_end, kind;
};

constexpr int kMaxList = 64;   // q-tiles one workgroup takes at most

// A position in a workgroup's stream of key tiles: list entry e, key tile kt of it (the
// entry's end kt_end, K/V rows kv_base and valid keys cached in scalar registers).
struct Cursor {
    int e, kt, kt_end, kvalid;
    unsigned long long kv_base;
    bool valid, first;   // first: kt is the entry's first key tile
};

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ unsigned long long uni64(unsigned long long x) {
    return (unsigned long long)(unsigned)uni((int)(unsigned)x) |
           ((unsigned long long)(unsigned)uni((int)(unsigned)(x >> 32)) << 32);
}

// Exclusive prefix sum of x over the 64 lanes of the wave; total: the sum over all.
// Exclusive prefix sum over the 64 lanes (and the total in `total`), by row shifts within
// each 16-lane row, then the broadcasts of a row's last lane into the rows above it.
__device__ __forceinline__ int wave_excl_scan(int x, int& total) {
    int v = x;
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);    // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);    // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);    // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);    // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
    total = __builtin_amdgcn_readlane(v, 63);
    return v - x;
}

__device__ __forceinline__ Cursor cursor_at(const TileEnt* ents, int e, int n) {
    Cursor c{};
    c.e = e;
    c.valid = e < n;
    if (c.valid) {
        c.kt = uni(ents[e].kt_begin);
        c.kt_end = uni(ents[e].kt_end);
        c.kvalid = uni(ents[e].kvalid);
        c.kv_base = uni64(ents[e].kv_base);
        c.first = true;
    }
    return c;
}

__device__ __forceinline__ Cursor advance(Cursor c, const TileEnt* ents, int n) {
    if (!c.valid) return c;
    if (c.kt + 1 < c.kt_end) {
        ++c.kt;
        c.first = false;
        return c;
    }
    return cursor_at(ents, c.e + 1, n);
}

// GATE: waves skip the work of key tiles none of their rows sees.  Only causal and banded
// launches have such tiles; the full bidirectional launch keeps the ungated stream, whose
// schedule the extra branches would only disturb (measured 39.9 vs 41.3 us on the padded
// BERT batch, both timed in the kernel's form for a non-positive scale).
//
// Persistent: each workgroup walks the list of q-tiles plan::persist_pos deals it and runs
// their key tiles as one pipelined stream (the key tiles of the next q-tile follow those
// of the current one without a pause: its Q rows are loaded one step ahead of its first
// Q.K^T, its first K/V tiles are copied as any other), so that only the first q-tile of a
// workgroup waits for its start-up loads.
template <int D, bool POS_SCALE, bool GATE, bool F16>
__global__ __launch_bounds__(Cfg<D>::THREADS, Cfg<D>::MINB) void prefill_bf16_narrow_kernel(PrefillArgs a) {
    constexpr int RB = Cfg<D>::RB;
    constexpr int W = Cfg<D>::W;
    constexpr int BM = Cfg<D>::BM;
    static_assert(RB == 1, "one row block per wave");
    using G = Geo<D, W>;
    __shared__ __attribute__((aligned(16))) u32x4 k_lds[2][kBN * G::KS];
    __shared__ __attribute__((aligned(16))) u32x4 v_lds[2][kBN * G::CPR];
    __shared__ __attribute__((aligned(16))) u32x4 q_lds[W * G::KC * 64];   // next q-tile's Q^T operands
    __shared__ TileEnt ents[kMaxList];
    __shared__ int s_counts[3];   // entries with key tiles, entries of zero rows, key tiles in all

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
    const bool causal = a.causal != 0;
    // row strides of q / out and of k / v (plan::item_rows: token-major and unpadded
    // layouts interleave the heads of a token)
    const int q_rs = (a.cu_seqlens != nullptr || a.token_major) ? a.q_heads * D : D;
    st.kv_rs = (a.cu_seqlens != nullptr || a.token_major) ? a.kv_heads * D : D;

    // ---- this workgroup's q-tiles: lane k of wave 0 looks up the k-th ------------------
    // (plan::persist_pos; with per-item lengths for at most kRankedItems items, in the
    // ranked order of plan::ranked_tile)
    __shared__ __attribute__((aligned(16))) uint32_t s_key[plan::kRankedItems];
    __shared__ int s_order[plan::kRankedItems], s_ne[plan::kRankedItems], s_nrow[plan::kRankedItems];
    __shared__ int s_tiles[plan::kRankedItems], s_i0[plan::kRankedItems], s_i1[plan::kRankedItems];
    __shared__ int s_start_ne[plan::kRankedItems], s_start_z[plan::kRankedItems];
    const bool has_len = a.seq_lens != nullptr || a.cu_seqlens != nullptr;
    const bool ranked = plan::ranked_order(has_len, a.batch, a.n_qtiles, a.q_heads);
    if (wave == 0) {
        const long pk = plan::persist_pos((int)blockIdx.x, lane, (int)gridDim.x, kXcds);
        bool have = false;
        int b = 0, h = 0, qt = 0;
        plan::Rows ir{};
        if (ranked) {
            // lane b: item b's rows, keys and schedule numbers; its rank by cost
            const int B = a.batch;
            int i0 = 0, i1 = 0, rows = 0, valid = 0;
            if (lane < B) {
                if (a.cu_seqlens) {
                    i0 = a.cu_seqlens[lane];
                    i1 = a.cu_seqlens[lane + 1];
                    rows = min(max(i1 - i0, 0), a.q_len);
                    valid = rows;
                } else {
                    i0 = a.seq_lens[lane];
                    rows = a.q_len;
                    valid = min(max(i0, 0), a.kv_len);
                }
            }
            const plan::ItemSched is = lane < B ? plan::item_sched(rows, valid, a.pos_offset, causal, a.window, BM, kBN)
                                                : plan::ItemSched{0, 0, -1};
            // rank: the items whose key is above this one's (keys of all 64 lanes, read back
            // as 16 broadcast reads)
            typedef __attribute__((address_space(3))) const int lds_int;
            typedef __attribute__((address_space(3))) const u32x4 lds_key4;
            const uint32_t key = lane < B ? plan::rank_key(is.cost, lane) : 0u;
            s_key[lane] = key;
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the writes have landed
            __builtin_amdgcn_wave_barrier();
            int rank = 0;
#pragma unroll
            for (int x4 = 0; x4 < plan::kRankedItems / 4; ++x4) {
                const u32x4 k4 = ((lds_key4*)(const void*)s_key)[x4];
                rank += (k4[0] > key ? 1 : 0) + (k4[1] > key ? 1 : 0) + (k4[2] > key ? 1 : 0) + (k4[3] > key ? 1 : 0);
            }
            if (lane < B) {
                s_order[rank] = lane;
                s_tiles[rank] = is.ne * a.q_heads;   // non-empty q-tiles of rank `rank`
                s_ne[lane] = is.ne;
                s_nrow[lane] = is.nrow;
                s_i0[lane] = i0;
                s_i1[lane] = i1;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
            int n_ne = 0, n_z = 0;
            const int x_ne = wave_excl_scan(lane < B ? s_tiles[lane] : 0, n_ne);
            const int x_z = wave_excl_scan(lane < B ? (is.nrow - is.ne) * a.q_heads : 0, n_z);
            if (lane < B) {
                s_start_ne[lane] = x_ne;
                s_start_z[lane] = x_z;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
            const plan::RankedRef rr =
                plan::ranked_tile(pk < (long)n_ne + n_z ? (int)pk : -1, B, n_ne, n_z, (lds_int*)s_order,
                                  (lds_int*)s_start_ne, (lds_int*)s_start_z, (lds_int*)s_ne, (lds_int*)s_nrow);
            if (rr.kind != 2) {
                have = true;
                // (clamped: an item, head and q-tile of the launch whatever the LDS holds)
                b = min(max(rr.b, 0), B - 1);
                h = min(max(rr.h, 0), a.q_heads - 1);
                qt = min(max(rr.qt, 0), a.n_qtiles - 1);
                const plan::Layout lay = a.cu_seqlens ? plan::kUnpadded : a.token_major ? plan::kTokenMajor : plan::kHeadMajor;
                ir = plan::item_rows(lay, b, h, h / (a.q_heads / a.kv_heads), D, a.q_heads, a.kv_heads, a.q_len,
                                     a.kv_len, s_i0[b], s_i1[b], a.seq_lens != nullptr, s_i0[b]);
            }
        } else if (pk < (long)a.batch * a.q_heads * a.n_qtiles) {
            const plan::TileRef t = plan::persist_tile(pk, a.q_heads, a.n_qtiles);
            have = true;
            b = t.b;
            h = t.h;
            qt = t.qt;
            ir = item_rows(a, b, h, h / (a.q_heads / a.kv_heads), D);
        }
        TileEnt e{};
        int kind = 2;   // no q-tile (past the list, or no rows in it)
        if (have) {
            const int q0 = qt * BM;
            if (q0 < ir.q_len) {
                const int last = min(q0 + BM, ir.q_len) - 1;
                const plan::Tiles kt = plan::key_tiles(
                    plan::span_union(a.pos_offset + q0, a.pos_offset + last, ir.kv_valid, causal, a.window), kBN);
                e.q_base = ir.q_base;
                e.kv_base = ir.kv_base;
                e.q0 = q0;
                e.q_len = ir.q_len;
                e.kvalid = ir.kv_valid;
                e.kt_begin = kt.begin;
                e.kt_end = kt.end;
                kind = kt.end > kt.begin ? 0 : 1;
                e.kind = kind;
            }
        }
        const unsigned long long m0 = __builtin_amdgcn_ballot_w64(kind == 0);
        const unsigned long long m1 = __builtin_amdgcn_ballot_w64(kind == 1);
        const unsigned long long below = (1ull << lane) - 1ull;
        const int n0 = __builtin_popcountll(m0);
        if (kind == 0) ents[__builtin_popcountll(m0 & below)] = e;
        if (kind == 1) ents[n0 + __builtin_popcountll(m1 & below)] = e;
        int steps = 0;   // key tiles of the whole list
        wave_excl_scan(kind == 0 ? e.kt_end - e.kt_begin : 0, steps);
        if (lane == 0) {
            s_counts[0] = n0;
            s_counts[1] = __builtin_popcountll(m1);
            s_counts[2] = steps;
        }
    }
    __syncthreads();
    const int n_ent = uni(s_counts[0]);
    const int n_zero = uni(s_counts[1]);
    const int n_steps = uni(s_counts[2]);

    // q-tiles whose rows see no key (padded rows, queries past the keys): zeros, written
    // after the workgroup's last key tile (or at once when it has none), so that they do not
    // delay its first tile copies
    auto zero_tiles = [&]() {
        for (int z = 0; z < n_zero; ++z) {
            const TileEnt& t = ents[n_ent + z];
            const int rows = min(BM, uni(t.q_len) - uni(t.q0));
            uint16_t* o0 = (uint16_t*)a.out + uni64(t.q_base) + (size_t)uni(t.q0) * q_rs;
            for (int i = tid; i < rows * (D / 8); i += W * 64)
                *(u32x4*)(o0 + (size_t)(i / (D / 8)) * q_rs + 8 * (i % (D / 8))) = u32x4{0, 0, 0, 0};
        }
    };
    if (n_ent == 0) {
        zero_tiles();
        return;
    }

    // ---- per-lane constants ---------------------------------------------------------------
    st.k_lds0 = lds_addr(k_lds[0]);
    st.v_lds0 = lds_addr(v_lds[0]);
#pragma unroll
    for (int ii = 0; ii < G::NKW; ++ii)
        st.koff[ii] = plan::chunk_offset(plan::narrow_k_chunk(wave + W * ii, lane, G::CPR), st.kv_rs);
    st.voff = plan::chunk_offset(plan::narrow_v_chunk(wave, lane, D), st.kv_rs);
    st.v_step = plan::narrow_v_copy_step(W, D, st.kv_rs);
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
    const char* kg0 = (const char*)a.k;
    const char* vg0 = (const char*)a.v;
    auto kg_of = [&](const Cursor& c) { return kg0 + 2 * c.kv_base; };
    auto vg_of = [&](const Cursor& c) { return vg0 + 2 * c.kv_base; };

    // Q^T operands of entry e's rows for this wave: lane l holds row l%32, dims
    // 16*kc + 8*g + [0, 8).  Rows past the end read the last row (their keys are masked
    // and their output is not stored).  load_q reads them into registers (the first
    // q-tile); copy_q copies them into this wave's part of q_lds (1 KiB per k-step, lane l's
    // 16 bytes at 16*l), and read_q moves them into registers once the copy has landed.
    auto load_q = [&](bf16x8 (&qf)[G::KC], int e) {
        const int q0 = uni(ents[e].q0), q_len = uni(ents[e].q_len);
        const uint16_t* qrow = (const uint16_t*)a.q + uni64(ents[e].q_base) +
                               (size_t)min(q0 + wave * 32 + (lane & 31), q_len - 1) * q_rs;
#pragma unroll
        for (int kc = 0; kc < G::KC; ++kc)
            qf[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * kc + 8 * g));
    };
    const uint32_t q_lds0 = lds_addr(q_lds) + wave * G::KC * 1024;
    auto copy_q = [&](int e) {
        const int q0 = uni(ents[e].q0), q_len = uni(ents[e].q_len);
        const int rb = min(q0 + wave * 32, q_len - 1);   // the wave's first row, clamped
        const char* src = (const char*)((const uint16_t*)a.q + uni64(ents[e].q_base) + (size_t)rb * q_rs);
        const uint32_t voff = plan::q_copy_offset(min(q0 + wave * 32 + (lane & 31), q_len - 1) - rb, g, q_rs);
#pragma unroll
        for (int kc = 0; kc < G::KC; ++kc) lds_dma16(src, voff + 32 * kc, q_lds0 + kc * 1024);
    };
    auto read_q = [&](bf16x8 (&qf)[G::KC]) {
        const lds_char* p = (const lds_char*)(const void*)q_lds + (wave * G::KC * 1024 + lane * 16);
#pragma unroll
        for (int kc = 0; kc < G::KC; ++kc) qf[kc] = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(p + kc * 1024));
    };
    // The rows of entry e as the next Q.K^T's mask and gate see them.
    auto set_rows = [&](int e) {
        const int q0 = uni(ents[e].q0), q_len = uni(ents[e].q_len), kvalid = uni(ents[e].kvalid);
        const int r0 = q0 + wave * 32;
        const RowBlockKeys k = row_block_keys(a, r0, 32, r0 + (lane & 31), q_len, kvalid);
        st.lo_r[0] = k.lane.lo;
        st.hi_r[0] = k.lane.hi;
        st.b_inter_lo[0] = k.inter.lo;
        st.b_inter_hi[0] = k.inter.hi;
        return plan::Keys{uni(k.uni.lo), uni(k.uni.hi)};
    };
    // Output of entry e: O / l, zero for rows that see no key, stored with RNE; then the
    // softmax state starts afresh.  Returns whether every row of the wave was stored (then
    // the stores are exactly kStores instructions).
    constexpr int kStores = G::DB * 4;
    auto finish_tile = [&](int e) {
        const int q0 = uni(ents[e].q0), q_len = uni(ents[e].q_len), kvalid = uni(ents[e].kvalid);
        const int row = q0 + wave * 32 + (lane & 31);
        const float l_tot = halves_sum(st.l_run[0]);
        const bool sees = plan::row_keys(a.pos_offset + row, kvalid, causal, a.window).hi >= 0;
        // a row that sees no key is written as zeros by a select, whatever its (unmasked) sums
        const bool keep = sees && l_tot > 0.0f;
        const float inv = keep ? 1.0f / l_tot : 0.0f;
        uint16_t* orow = (uint16_t*)a.out + uni64(ents[e].q_base) + (size_t)min(row, q_len - 1) * q_rs;
        const bool full = q0 + wave * 32 + 32 <= q_len;
        if (full || row < q_len) {
#pragma unroll
            for (int db = 0; db < G::DB; ++db) {
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int d = 32 * db + 8 * e4 + 4 * g;
                    u32x2 w;
                    w[0] = H::pack2(keep ? st.o[0][db][4 * e4] * inv : 0.0f, keep ? st.o[0][db][4 * e4 + 1] * inv : 0.0f);
                    w[1] = H::pack2(keep ? st.o[0][db][4 * e4 + 2] * inv : 0.0f, keep ? st.o[0][db][4 * e4 + 3] * inv : 0.0f);
                    *(u32x2*)(orow + d) = w;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < G::DB; ++i) st.o[0][i] = f32x16{};
        st.m_run[0] = kNegInf;
        st.l_run[0] = 0.0f;
        return full;
    };

    const lds_char* kb[2] = {(const lds_char*)(const void*)k_lds[0], (const lds_char*)(const void*)k_lds[1]};
    const lds_char* vb[2] = {(const lds_char*)(const void*)v_lds[0], (const lds_char*)(const void*)v_lds[1]};

    // ---- the stream: step s computes the softmax and P.V of key tile s and the Q.K^T of
    // key tile s+1; it copies K(s+2) and V(s+1) (cursors cur, nv, nk) --------------------
    Cursor cur{}, nv = cursor_at(ents, 0, n_ent), nk = advance(nv, ents, n_ent);
    load_q(st.qf[0], 0);
    if (nk.valid && nk.first) copy_q(nk.e);
    plan::Keys uni_nxt = set_rows(0), uni_cur{0, -1};
#pragma unroll
    for (int i = 0; i < G::DB; ++i) st.o[0][i] = f32x16{};
    st.m_run[0] = kNegInf;   // running (possibly stale) max of this lane's row, log2 units
    st.l_run[0] = 0.0f;      // running sum over this lane's half of the keys
    bool stores_pending = false;

    f32x16 sa[RB][2], sb[RB][2];
    st.copy_k(kg_of(nv), nv.kvalid, nv.kt, 0);
    if (nk.valid) st.copy_k(kg_of(nk), nk.kvalid, nk.kt, 1);
    st.copy_v(vg_of(nv), nv.kvalid, nv.kt, 0);
    wait_vm0();          // Q, the first K tiles and V tile have landed
    __syncthreads();
    if (!GATE || st.wave_sees(uni_nxt, nv.kt)) {
        float mx[RB];
        st.qk(sa, kb[0]);
        st.mask_scale(sa, nv.kt);
        st.row_max(sa, mx);
        st.finish_max(mx);
    }

    auto step = [&](auto has_next_c, auto par_c, f32x16 (&cs)[RB][2], f32x16 (&ns)[RB][2]) {
        constexpr bool HAS_NEXT = decltype(has_next_c)::value;
        constexpr int PAR = decltype(par_c)::value;
        // this thread's copies of K(s+1) and V(s) (and Q rows) have landed -- the output
        // stores of the previous step, issued after them, may stay in flight (vector memory
        // operations of a wave complete in issue order) ...
        if (stores_pending)
            wait_vm<kStores>();
        else
            wait_vm0();
        __syncthreads();     // ... everyone's; and nobody still reads K(s) or V(s-1)
        cur = nv;
        nv = nk;
        nk = advance(nk, ents, n_ent);
        uni_cur = uni_nxt;
        // the next key tile starts a q-tile: its Q rows (copied a step ago) and its masks;
        // the Q copy of the q-tile after it may then reuse q_lds
        if (HAS_NEXT && nv.first) {
            keep_branch();
            read_q(st.qf[0]);
            uni_nxt = set_rows(nv.e);
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the reads have left q_lds
        }
        if (nk.valid) st.copy_k(kg_of(nk), nk.kvalid, nk.kt, PAR);
        if (HAS_NEXT) st.copy_v(vg_of(nv), nv.kvalid, nv.kt, PAR ^ 1);
        if (nk.valid && nk.first) {
            keep_branch();
            copy_q(nk.e);
        }
        bf16x8 pf[RB][4];
        float mx[RB];
        // Wave-uniform: whether this wave has rows that see key tile s (its softmax and
        // P.V) and key tile s+1 (its Q.K^T, mask and max).
        const bool see_cur = !GATE || st.wave_sees(uni_cur, cur.kt);
        const bool see_nxt = HAS_NEXT && (!GATE || st.wave_sees(uni_nxt, nv.kt));
        if (!GATE || (see_cur && see_nxt)) {
            st.template qk_next_probs<HAS_NEXT>(ns, cs, pf, kb[PAR ^ 1]);
            if (HAS_NEXT) st.mask_scale(ns, nv.kt);
            st.template pv_max_next<HAS_NEXT>(pf, vb[PAR], ns, mx);
        } else if (see_cur && see_nxt) {
            st.template qk_next_probs<true>(ns, cs, pf, kb[PAR ^ 1]);
            st.mask_scale(ns, nv.kt);
            st.template pv_max_next<true>(pf, vb[PAR], ns, mx);
        } else if (see_cur) {
            keep_branch();
            st.probs_only(cs, pf);
            st.template pv_max_next<false>(pf, vb[PAR], ns, mx);
        } else if (see_nxt) {
            keep_branch();
            st.qk(ns, kb[PAR ^ 1]);
            st.mask_scale(ns, nv.kt);
            st.row_max(ns, mx);
        }
        // key tile s was the last of its q-tile: its output
        stores_pending = false;
        if (!HAS_NEXT || nv.first) {
            keep_branch();
            stores_pending = uni(finish_tile(cur.e)) != 0;
        }
        if (see_nxt) st.finish_max(mx);
    };

    typedef std::integral_constant<bool, true> T_;
    typedef std::integral_constant<bool, false> F_;
    typedef std::integral_constant<int, 0> P0;
    typedef std::integral_constant<int, 1> P1;
    int j = 0;
    for (; j + 2 < n_steps; j += 2) {
        step(T_{}, P0{}, sa, sb);
        step(T_{}, P1{}, sb, sa);
    }
    if (j + 1 < n_steps) {
        step(T_{}, P0{}, sa, sb);
        step(F_{}, P1{}, sb, sa);
    } else {
        step(F_{}, P0{}, sa, sb);
    }
    zero_tiles();
}

// Workgroups the device holds at once (Cfg::MINB per CU), per device.
int narrow_slots() {
    static int slots[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (slots[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return 0;
        slots[dev] = cus * Cfg<64>::MINB;
    }
    return slots[dev];
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
    PrefillArgs args = a;
    args.n_qtiles = (a.q_len + Cfg<D>::BM - 1) / Cfg<D>::BM;
    const long tiles = (long)args.n_qtiles * a.q_heads * a.batch;
    const int slots = narrow_slots();
    if (slots <= 0) return hipErrorInvalidDevice;
    const dim3 grid((unsigned)plan::persist_grid(tiles, slots, kXcds, kMaxList));
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
