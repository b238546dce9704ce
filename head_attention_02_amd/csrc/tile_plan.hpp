// tile_plan.hpp -- the integer planning of the attention kernels: which keys a query row
// sees, which key tiles a workgroup visits, how blocks map to (q-tile, item, head), where
// an item's rows live, and where every 16-byte tile copy reads from.
//
// Plain constexpr C++17 with no HIP header: the kernels call these functions on the
// device (clang treats constexpr functions as host-and-device), and a host-side check
// (g++) enumerates every copy address of a launch with the very same functions, so the
// address arithmetic the kernels run is the arithmetic that check proves in bounds.
//
// Key sets follow the readings of the pages (ripvec-core `Driver` page,
// `fused_scale_mask_softmax_windowed`: bidirectional band |p - j| <= window/2;
// ferrum-kernels `Backend` page, `flash_attention` and `flash_attention_batched_per_cache`:
// query i at position pos_offset + i, causal keys j <= p, causal window p - j < window).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mi_attn {
namespace plan {

constexpr int imin(int a, int b) { return a < b ? a : b; }
constexpr int imax(int a, int b) { return a > b ? a : b; }

// Keys lo..hi, both inclusive; empty when hi < lo.
struct Keys {
    int lo, hi;
};

// The keys a query at absolute position p sees among the valid keys [0, valid).  A query
// at or past the valid length is a padded row and sees none.
constexpr Keys row_keys(int p, int valid, bool causal, int window) {
    int lo = 0, hi = valid - 1;
    if (causal) hi = imin(hi, p);
    if (window > 0) {
        if (causal) {
            lo = imax(0, p - window + 1);
        } else {
            lo = imax(0, p - window / 2);
            hi = imin(hi, p + window / 2);
        }
    }
    if (p >= valid) hi = -1;
    return {lo, hi};
}

// A superset of the keys some query at positions p_lo..p_hi sees (the key set moves
// monotonically with the position, so the ends come from the first and last row).  Empty
// when every position is padding.
constexpr Keys span_union(int p_lo, int p_hi, int valid, bool causal, int window) {
    int lo = 0, hi = valid - 1;
    if (causal) hi = imin(hi, p_hi);
    if (window > 0) {
        if (causal) {
            lo = imax(0, p_lo - window + 1);
        } else {
            lo = imax(0, p_lo - window / 2);
            hi = imin(hi, p_hi + window / 2);
        }
    }
    if (p_lo >= valid) hi = -1;
    return {lo, hi};
}

// The keys every query at positions p_lo..p_hi sees, provided all of them are valid rows
// (the caller checks that: a padded row sees nothing).
constexpr Keys span_inter(int p_lo, int p_hi, int valid, bool causal, int window) {
    int lo = 0, hi = valid - 1;
    if (causal) hi = imin(hi, p_lo);
    if (window > 0) {
        if (causal) {
            lo = imax(0, p_hi - window + 1);
        } else {
            lo = imax(0, p_hi - window / 2);
            hi = imin(hi, p_lo + window / 2);
        }
    }
    return {lo, hi};
}

// Key tiles [begin, end) of `bn` keys that hold the keys k.lo..k.hi.
struct Tiles {
    int begin, end;
};
constexpr Tiles key_tiles(Keys k, int bn) {
    const int begin = k.lo / bn;
    return {begin, k.hi >= k.lo ? (k.hi + 1 + bn - 1) / bn : begin};
}

// ---- grid: block index -> (q-tile, item, query head) ---------------------------------
//
// One-dimensional grid, q-tile rank slowest.  With `last_first` the q-tiles run last to
// first, which runs the grid longest-first so that the short tiles fill in at the end:
// with a causal mask the tiles near the end of the sequence carry the most keys, and with
// per-item lengths a late q-tile exists only for the longer items (whose every tile
// carries more keys).  Workgroups are dealt
// round-robin to the XCDs (block i to XCD i % xcds), each with its own L2; when the
// (item, kv head) units divide evenly, every XCD gets whole units -- all query heads of a
// kv head -- so that a unit's K/V tiles are fetched into one L2 and reused there.
struct BlockCoord {
    int qt, b, h;
};
constexpr BlockCoord map_block(unsigned block, int n_qtiles, int batch, int q_heads, int kv_heads, bool last_first,
                               int xcds) {
    const int qgrp = q_heads / kv_heads;
    const int units = batch * kv_heads;
    int qt_rank = 0, b = 0, h = 0;
    if (units % xcds == 0) {
        const int xcd = (int)(block % (unsigned)xcds), k = (int)(block / (unsigned)xcds);
        const int per_xcd = units / xcds;
        const int hig = k % qgrp;
        const int unit = ((k / qgrp) % per_xcd) * xcds + xcd;
        qt_rank = k / (qgrp * per_xcd);
        b = unit / kv_heads;
        h = (unit % kv_heads) * qgrp + hig;
    } else {
        const int bh = (int)(block % (unsigned)(batch * q_heads));
        qt_rank = (int)(block / (unsigned)(batch * q_heads));
        b = bh / q_heads;
        h = bh % q_heads;
    }
    return {last_first ? n_qtiles - 1 - qt_rank : qt_rank, b, h};
}

// ---- persistent grid of the head-dim-32/64 kernel ------------------------------------------
//
// That kernel runs `wgs` workgroups (a multiple of xcds) and each walks a list of q-tiles,
// streaming the key tiles of one q-tile after another so that the start-up latency of a
// q-tile (its Q rows, its first K/V tiles) hides behind the work of the previous one.
// The q-tiles (item b, query head h, q-tile qt) are numbered
// p = (b * q_heads + h) * n_qtiles + (n_qtiles - 1 - qt), last q-tile first within a head,
// and dealt in rounds of `wgs` numbers: round k covers [k * wgs, (k + 1) * wgs), every other
// round in reverse order (so that a workgroup dealt an early number in one round gets a
// late one in the next), and within a round the workgroups of XCD x (block i runs on XCD
// i % xcds) take one contiguous block of wgs / xcds numbers, so that neighbouring q-tiles
// of a head -- which read the same K/V tiles -- are fetched into one L2.
constexpr int persist_slot(int wg, int wgs, int xcds) { return (wg % xcds) * (wgs / xcds) + wg / xcds; }

// The number of the k-th q-tile of workgroup wg (increasing in k; the list ends at the
// first number past the last q-tile).
constexpr long persist_pos(int wg, int k, int wgs, int xcds) {
    const int j = persist_slot(wg, wgs, xcds);
    return (long)k * wgs + ((k & 1) ? wgs - 1 - j : j);
}

struct TileRef {
    int b, h, qt;
};
constexpr TileRef persist_tile(long p, int q_heads, int n_qtiles) {
    const long bh = p / n_qtiles;
    return {(int)(bh / q_heads), (int)(bh % q_heads), n_qtiles - 1 - (int)(p % n_qtiles)};
}

// With per-item lengths (up to kRankedItems items) the numbers run over the q-tiles in
// a ranked order instead, so that the rounds deal the costliest q-tiles first (each
// workgroup's later, reversed rounds then bring it cheaper ones): first every q-tile that
// visits keys -- items by the key tiles of their costliest q-tile, most first (ties by item
// index), within an item query head by query head, last q-tile first -- then every
// q-tile whose rows see no key (zeros to write), items in index order.
constexpr int kRankedItems = 64;

struct ItemSched {
    int nrow;   // q-tiles holding rows of the item
    int ne;     // ... of which the first ne hold a row that sees a key
    int cost;   // key tiles of the item's costliest q-tile (its last non-empty one)
};
// rows: query rows of the item; valid: its keys; p: pos_offset.  A row r sees a key iff
// p + r < valid (plan::row_keys), so the non-empty q-tiles are a prefix.
constexpr ItemSched item_sched(int rows, int valid, int p, bool causal, int window, int bm, int bn) {
    ItemSched s{};
    s.nrow = (imax(rows, 0) + bm - 1) / bm;
    const int seen_rows = imin(imax(rows, 0), imax(valid - p, 0));
    s.ne = (seen_rows + bm - 1) / bm;
    if (s.ne > 0) {
        const int q0 = (s.ne - 1) * bm, last = imin(q0 + bm, rows) - 1;
        const Tiles t = key_tiles(span_union(p + q0, p + last, valid, causal, window), bn);
        s.cost = t.end - t.begin;
    }
    return s;
}

// Whether item a (cost_a) ranks before item b (cost_b).
constexpr bool ranks_before(int cost_a, int a, int cost_b, int b) { return cost_a > cost_b || (cost_a == cost_b && a < b); }

// The same order as one unsigned key per item (b < kRankedItems, 0 <= cost < 2^25): item a
// ranks before item b iff rank_key(cost_a, a) > rank_key(cost_b, b); 0 is below every
// item's key (the kernel gives it to lanes without an item).
constexpr uint32_t rank_key(int cost, int b) { return ((uint32_t)(cost + 1) << 6) | (uint32_t)(kRankedItems - 1 - b); }

// Whether a launch takes the ranked order: per-item lengths for at most kRankedItems
// items, and q-tile numbers that fit an int (the kernel numbers them in 32 bits).
constexpr bool ranked_order(bool has_len, int batch, int n_qtiles, int q_heads) {
    return has_len && batch <= kRankedItems && (long)batch * n_qtiles * q_heads < (1L << 31);
}

// The last index i in [0, n) with a[i] <= x (a non-decreasing, a[0] <= x).  P: a pointer
// or array-like type (the kernel passes LDS pointers).
template <class P>
constexpr int last_at_most(P a, int n, int x) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (a[mid] <= x)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Number p of the ranked order -> q-tile.  order[r]: the item of rank r; start_ne[r]: the
// number of its first non-empty q-tile (n_ne in all); start_z[b]: the number of item b's
// first zero q-tile, counted from n_ne (n_z in all).  kind 0: a q-tile with keys, 1: zeros,
// 2: past the end.
struct RankedRef {
    int b, h, qt, kind;
};
template <class IP>
constexpr RankedRef ranked_tile(int p, int items, int n_ne, int n_z, IP order, IP start_ne, IP start_z, IP ne,
                                IP nrow) {
    RankedRef t{0, 0, 0, 2};
    if (p >= 0 && p - n_ne < n_z) {
        const bool z = p >= n_ne;   // a zero q-tile
        const int x = z ? p - n_ne : p;
        const IP starts = z ? start_z : start_ne;
        const int r = last_at_most(starts, items, x);
        const int b = z ? r : order[r];
        const int n = z ? nrow[b] - ne[b] : ne[b];
        const int local = x - starts[r];
        const int h = local / n, i = local - h * n;
        t = {b, h, z ? ne[b] + i : ne[b] - 1 - i, z ? 1 : 0};
    }
    return t;
}

// Grid size: the `slots` workgroups that fit on the device at once (rounded down to a
// multiple of xcds), no more than `tiles` needs, and enough that no list is longer than
// max_list.
constexpr int persist_grid(long tiles, int slots, int xcds, int max_list) {
    long g = (long)slots / xcds * xcds;
    const long need = (tiles + xcds - 1) / xcds * xcds;
    if (g > need) g = need;
    const long min_g = ((tiles + max_list - 1) / max_list + xcds - 1) / xcds * xcds;
    if (g < min_g) g = min_g;
    if (g < xcds) g = xcds;
    return (int)g;
}

// ---- where an item's rows live ---------------------------------------------------------

// Layouts of the prefill tensors.
enum Layout { kHeadMajor = 0, kTokenMajor = 1, kUnpadded = 2 };

// One (item, query head)'s rows: element offsets and strides.
struct Rows {
    size_t q_base;    // row 0 of (item, query head) in q and out
    size_t kv_base;   // row 0 of (item, kv head) in k and v
    int q_rs, kv_rs;  // elements from one row to the next
    int q_len;        // query rows of the item
    int kv_valid;     // keys of the item (its valid length applied)
};

// `t0` and `t1`: the item's token range (unpadded layout: cu_seqlens[b], cu_seqlens[b+1]);
// `len_b`: the item's valid key count seq_lens[b] when `has_len` (clamped to [0, kv_len]).
constexpr Rows item_rows(Layout layout, int b, int h, int kvh, int D, int q_heads, int kv_heads, int q_len,
                         int kv_len, int t0, int t1, bool has_len, int len_b) {
    Rows r{};
    if (layout == kUnpadded) {
        const int n = imin(imax(t1 - t0, 0), q_len);
        r.q_rs = q_heads * D;
        r.kv_rs = kv_heads * D;
        r.q_base = (size_t)t0 * r.q_rs + (size_t)h * D;
        r.kv_base = (size_t)t0 * r.kv_rs + (size_t)kvh * D;
        r.q_len = n;
        r.kv_valid = n;
    } else if (layout == kTokenMajor) {
        r.q_rs = q_heads * D;
        r.kv_rs = kv_heads * D;
        r.q_base = (size_t)b * q_len * r.q_rs + (size_t)h * D;
        r.kv_base = (size_t)b * kv_len * r.kv_rs + (size_t)kvh * D;
        r.q_len = q_len;
        r.kv_valid = has_len ? imin(imax(len_b, 0), kv_len) : kv_len;
    } else {
        r.q_rs = D;
        r.kv_rs = D;
        r.q_base = ((size_t)b * q_heads + h) * (size_t)q_len * D;
        r.kv_base = ((size_t)b * kv_heads + kvh) * (size_t)kv_len * D;
        r.q_len = q_len;
        r.kv_valid = has_len ? imin(imax(len_b, 0), kv_len) : kv_len;
    }
    return r;
}

// ---- tile copies -------------------------------------------------------------------------
//
// A tile copy moves 64 lanes x 16 bytes from K or V rows into LDS.  Each function below
// names the tile row and element column one lane reads (`Chunk`); the byte offset from
// the tile's first row is (row * kv_rs + col) * 2.  Rows past the valid keys repeat the
// last valid one (their scores are masked), clamped relative to the TILE base:
// tail_row(row, kvalid, tile_key0) never goes below row 0 of the tile because a visited
// tile always starts at a valid key.
struct Chunk {
    int row, col;
};

constexpr uint32_t chunk_offset(Chunk c, int kv_rs) { return (uint32_t)((c.row * kv_rs + c.col) * 2); }
constexpr int tail_row(int row, int kvalid, int tile_key0) { return imin(row, kvalid - 1 - tile_key0); }

// Tile geometry of the head-dim-128 kernel: 8 waves of 32 query rows (256 rows per
// workgroup), 64-key tiles, the 4 waves of the trailing group issue every tile copy.
template <int D>
struct WideGeo {
    static constexpr int BN = 64;                        // keys per tile
    static constexpr int WAVES = 8;
    static constexpr int BM = 32 * WAVES;                // query rows per workgroup
    static constexpr int COPY_WAVES = 4;
    static constexpr int CPR = D / 8;                    // 16-byte chunks per row
    static constexpr int KC = D / 16;                    // MFMA k-steps of Q.K^T
    static constexpr int DB = D / 32;                    // 32-wide blocks of the output head dim
    static constexpr int NK = 2 * KC;                    // K copy instructions per tile (1 KiB each)
    static constexpr int NKW = (NK + COPY_WAVES - 1) / COPY_WAVES;
    static constexpr int NV = 4 * DB;                    // V copy instructions per tile (1 KiB each)
    static constexpr int NVW = (NV + COPY_WAVES - 1) / COPY_WAVES;
    static constexpr int K_BYTES = BN * D * 2;
    static constexpr int V_BYTES = BN * D * 2;
    static_assert(NV % COPY_WAVES == 0, "V copy rounds cover whole rows");
    static_assert(NK % COPY_WAVES == 0, "every copying wave issues the same number of K copies");
};

// Head-dim-128 kernel, K: copy f fills 1 KiB LDS block f = kb2*KC + kc, whose 16 bytes at
// 16*lane are lane's MFMA A operand: key 32*kb2 + lane%32, dims 16*kc + 8*(lane/32) + [0,8).
constexpr Chunk wide_k_chunk(int f, int lane, int kc_steps) {
    return {32 * (f / kc_steps) + (lane & 31), 16 * (f % kc_steps) + 8 * (lane >> 5)};
}
// ... the same split as a per-copy base (uniform) plus a per-lane offset (fixed for the
// kernel), so that a whole tile costs one add per copy
constexpr uint32_t wide_k_copy_base(int f, int kv_rs, int kc_steps) {
    return (uint32_t)((32 * (f / kc_steps) * kv_rs + 16 * (f % kc_steps)) * 2);
}
constexpr uint32_t wide_k_lane_off(int lane, int kv_rs) { return (uint32_t)(((lane & 31) * kv_rs + 8 * (lane >> 5)) * 2); }

// Head-dim-128 kernel, V: copy j = c4*DB + db fills the 512-byte blocks 2j and 2j+1 read by
// the transposing V^T loads of operand j; its lane p (half hi = p/32, q = p%32) takes key
// 16*c4 + 8*hi + 4*(q/16) + (q%8)/2 at dims 32*db + 16*((q/8)%2) + 8*(q%2).
constexpr Chunk wide_v_chunk(int j, int lane, int d_blocks) {
    const int q = lane & 31;
    return {16 * (j / d_blocks) + 8 * (lane >> 5) + 4 * (q >> 4) + ((q & 7) >> 1),
            32 * (j % d_blocks) + 16 * ((q >> 3) & 1) + 8 * (q & 1)};
}
constexpr uint32_t wide_v_copy_base(int j, int kv_rs, int d_blocks) {
    return (uint32_t)((16 * (j / d_blocks) * kv_rs + 32 * (j % d_blocks)) * 2);
}
constexpr uint32_t wide_v_lane_off(int lane, int kv_rs) {
    const int q = lane & 31;
    const int r = 8 * (lane >> 5) + 4 * (q >> 4) + ((q & 7) >> 1);
    return (uint32_t)((r * kv_rs + 16 * ((q >> 3) & 1) + 8 * (q & 1)) * 2);
}

// Tile geometry of the head-dim-32/64 kernel: W waves of 32 query rows, 64-key tiles, K
// rows padded to CPR+1 chunks in LDS, every wave issues its share of the tile copies.
template <int D, int W>
struct NarrowGeo {
    static constexpr int BN = 64;                // keys per tile
    static constexpr int BM = 32 * W;            // query rows per workgroup
    static constexpr int CPR = D / 8;            // 16-byte chunks per row
    static constexpr int KC = D / 16;            // MFMA k-steps of Q.K^T
    static constexpr int DB = D / 32;            // 32-wide blocks of the output head dim
    static constexpr int KS = CPR + 1;           // K row stride in chunks (padded)
    static constexpr int NK = BN * KS / 64;      // K copy instructions per tile
    static constexpr int NKW = (NK + W - 1) / W; // ... per wave (at most)
    static constexpr int NV = BN * CPR / 64;     // V copy instructions per tile
    static constexpr int NVW = NV / W;           // ... per wave
    static constexpr int K_BYTES = BN * KS * 16;
    static constexpr int V_BYTES = BN * CPR * 16;
    static_assert(NV % W == 0, "V copies split evenly over the waves");
};

// Head-dim-32/64 kernel, K: rows padded to cpr+1 chunks in LDS; copy i fills LDS chunks
// [64i, 64i+64) of the padded tile, so lane p writes padded chunk 64i + p = row * (cpr+1) + c
// (the pad chunk, c == cpr, repeats chunk 0).
constexpr Chunk narrow_k_chunk(int i, int lane, int cpr) {
    const int p = i * 64 + lane;
    const int row = p / (cpr + 1);
    const int c = p - row * (cpr + 1);
    return {row, 8 * (c < cpr ? c : 0)};
}

// Head-dim-32/64 kernel, V: rows XOR-swizzled at 64-byte granularity: chunk c of row r
// sits at chunk c ^ narrow_vswz(r), so that the four rows one transposing read phase
// touches fall into four different quarters of the banks.
constexpr int narrow_vswz(int r, int D) {
    return 4 * ((r / (4 / (D / 32))) & (D / 32 - 1));
}
constexpr Chunk narrow_v_chunk(int i, int lane, int D) {
    const int cpr = D / 8;
    const int p = i * 64 + lane;
    const int row = p / cpr;
    return {row, 8 * ((p % cpr) ^ narrow_vswz(row, D))};
}

// Whole-tile V copies of the head-dim-32/64 kernel: copy ii of wave w reads
// narrow_v_chunk(w + waves*ii, ...), which is wave w's copy 0 moved down by
// waves*64/cpr rows (a whole number of swizzle periods), i.e. this many bytes further.
constexpr size_t narrow_v_copy_step(int waves, int D, int kv_rs) { return (size_t)(waves * 64 / (D / 8)) * kv_rs * 2; }

// Q copy of the head-dim-32/64 kernel (a q-tile's rows copied ahead of its first Q.K^T):
// lane p reads query row r + p%32 (rows past the end clamped to the last; `row` is that
// row relative to the wave's first, clamped the same way) at elements 8*(p/32) + 16*kc,
// copy kc adding 32*kc bytes to this offset.
constexpr uint32_t q_copy_offset(int row, int half, int q_rs) { return (uint32_t)((row * q_rs + 8 * half) * 2); }

// ---- decode launch plan --------------------------------------------------------------------

// Decode split kernel shape: 4 waves; each K/V row (D elements) is read by D/EPL lanes
// with EPL/8 16-byte loads each, so a wave load covers 64/(D/EPL) rows; a batch is STEPS
// wave loads per row stream between two softmax updates.  EPL is 16 for 16-bit caches at
// head dims 64 and 128 (fewer lanes per row: fewer cross-lane sums per byte), else 8.
template <int D, int EPL = 8>
struct DecodeGeo {
    static constexpr int WAVES = 4;
    static constexpr int STEPS = EPL == 16 ? 4 : 8;
    static constexpr int LPR = D / EPL;            // lanes per key row
    static constexpr int RPW = 64 / LPR;           // rows per wave load
    static constexpr int STREAMS = RPW * WAVES;    // independent row streams in the workgroup
    static constexpr int BATCH = STREAMS * STEPS;  // keys per batch
};

struct DecodePlan {
    int splits, split_len, heads_per_group, head_groups;
};

// The key range of each (item, kv head) is cut into splits so that the grid reaches
// `target_wgs` workgroups; splits are whole multiples of 64 keys and at least 256 long.
constexpr DecodePlan decode_plan(int batch, int q_heads, int kv_heads, int kv_len, long target_wgs) {
    DecodePlan p{};
    const int group = q_heads / kv_heads;
    p.heads_per_group = group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
    p.head_groups = group / p.heads_per_group;
    const long units = (long)batch * kv_heads * p.head_groups;
    long splits = (target_wgs + units - 1) / units;
    const long max_splits = (kv_len + 255) / 256;
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    long split_len = (kv_len + splits - 1) / splits;
    split_len = (split_len + 63) / 64 * 64;
    splits = (kv_len + split_len - 1) / split_len;
    p.splits = (int)splits;
    p.split_len = (int)split_len;
    return p;
}

// The query of one decode item: the keys it may see are [0, len) and it sits at pos.
// append: len_b holds the length before the append; the new token goes to slot len_b and
// its query sits there (no room -- a length outside [0, capacity) -- leaves no key).
// With per-item lengths: the query sits at len_b - 1.  Otherwise at pos_offset.
struct DecodeQuery {
    int len, pos;
};
constexpr DecodeQuery decode_query(bool append, bool has_lens, int len_b, int kv_len, int capacity, int pos_offset) {
    if (append) {
        const int len = (len_b >= 0 && len_b < capacity) ? len_b + 1 : 0;
        return {len, len - 1};
    }
    if (has_lens) {
        const int len = imin(imax(len_b, 0), kv_len);
        return {len, len - 1};
    }
    return {kv_len, pos_offset};
}

// The keys [s0, s1) split `split` of that query attends: the causal prefix (or the last
// `window` positions) cut to the split's [split*split_len, (split+1)*split_len).
struct KeyRange {
    int s0, s1;
};
constexpr KeyRange decode_split_keys(DecodeQuery dq, int window, int split, int split_len) {
    const int lo = window > 0 ? imax(0, dq.pos - window + 1) : 0;
    const int hi = imin(dq.pos, dq.len - 1);
    return {imax(lo, split * split_len), imin(hi + 1, (split + 1) * split_len)};
}

// The cache row one decode lane reads: key = base + (u*waves + wave)*rows_per_load + r, and
// in the last batch of a split, keys at or past the split's end s1 read the split's first
// key s0 instead (their scores are masked).
constexpr int decode_key_row(int key, int s0, int s1, bool tail) { return !tail || key < s1 ? key : s0; }

}  // namespace plan
}  // namespace mi_attn
