// copy_addr_check.cpp -- host-side bounds check of every global address the attention
// kernels compute, using the kernels' own planning header (tile_plan.hpp), built with g++.
//
// Reads launch descriptions from stdin, one per line:
//   prefill LAYOUT B Hq Hkv Lq Lk D P CAUSAL W NLENS len_0 .. len_{NLENS-1}
//       LAYOUT 0 head-major, 1 token-major, 2 unpadded (lens are the item lengths, Lq = Lk =
//       the longest); D 32/64 run the narrow kernel's plan, 128 the wide kernel's.
//   decode MODE B Hq Hkv CAP KV_LEN D P W NLENS len_0 ..
//       MODE 0 stacked caches, 1 per-item caches, 2 per-item with append.
// For every block of the grid (the head-dim-32/64 kernel: every workgroup of its
// persistent grid and every q-tile of its list) it enumerates every tile visited, every copy
// instruction and every lane, computes the byte offset exactly as the kernel does (whole
// tiles: per-copy base + per-lane offset; tail tiles: rows clamped from the tile base),
// and checks that the 16 bytes lie inside the item's valid rows [0, kvalid) and columns
// [0, D), inside the tensor, and that the LDS destination lies inside the tile buffers.
// It also checks that the grid covers every (q-tile, item, head) exactly once, and the Q
// and output row addresses (and the head-dim-32/64 kernel's Q copies).  Decode: every cache row a lane reads lies in the
// split's key range inside [0, length) and inside the cache.
//
// --plant: compute tail-tile rows from each copy's first row (a block base) instead of
// the tile base -- the addressing that once produced a negative offset on a padded
// batch.  The check must report it.
//
// Prints "ok <checks>" or one "FAIL ..." line per violation (at most 20) and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "tile_plan.hpp"

using namespace mi_attn::plan;

namespace {

bool g_plant = false;
long g_checks = 0;
int g_fails = 0;

void fail(const std::string& what) {
    ++g_fails;
    if (g_fails <= 20) std::printf("FAIL %s\n", what.c_str());
}

struct Prefill {
    int layout, B, Hq, Hkv, Lq, Lk, D, P, causal, W;
    std::vector<int> lens;   // seq_lens (padded layouts) or item lengths (unpadded); empty: none
};

// One chunk read: tile kt, byte offset `off` from the tile's first row (uint32, as the
// kernel adds it to the tile base), of the rows of (item, kv head) `r`.
// The hardware adds the 32-bit per-lane offset zero-extended to the 64-bit (wave-uniform)
// base, so `off` is the uint32 offset widened, plus whatever uniform part sits in the base.
void check_chunk(const char* what, const Rows& r, int kt, int bn, uint64_t off, size_t kv_extent, int D,
                 const std::string& ctx) {
    ++g_checks;
    const uint64_t rel = (uint64_t)kt * bn * r.kv_rs + off / 2;   // elements from row 0 of (item, kv head)
    const uint64_t row = rel / (uint64_t)r.kv_rs, col = rel % (uint64_t)r.kv_rs;
    if (off % 16 != 0 || row >= (uint64_t)r.kv_valid || col + 8 > (uint64_t)D || r.kv_base + rel + 8 > kv_extent) {
        char buf[256];
        std::snprintf(buf, sizeof buf, "%s kt %d off %llu -> row %llu col %llu (valid %d, D %d)", what, kt,
                      (unsigned long long)off,
                      (unsigned long long)row, (unsigned long long)col, r.kv_valid, D);
        fail(ctx + " " + buf);
    }
}

// The tail-tile offset of a chunk: the kernel's form (clamped from the tile base, one
// 32-bit lane offset), or the planted form: the copy's first row in the uniform base and
// the clamped row addressed relative to it in the 32-bit lane offset, which wraps when the
// clamped row lies before the copy's first row.
uint64_t tail_offset(Chunk c, int first_row, int kvalid, int tile_key0, int kv_rs) {
    if (!g_plant) {
        c.row = tail_row(c.row, kvalid, tile_key0);
        return chunk_offset(c, kv_rs);
    }
    const int in_block = tail_row(c.row, kvalid, tile_key0) - first_row;
    return (uint64_t)first_row * kv_rs * 2 + (uint64_t)(uint32_t)((in_block * kv_rs + c.col) * 2);
}

void check_lds(const char* what, long byte, long limit, const std::string& ctx) {
    ++g_checks;
    if (byte < 0 || byte + 16 > limit) fail(ctx + " " + what + " LDS byte " + std::to_string(byte));
}

template <int D>
void prefill_wide(const Prefill& p, const Rows& r, int kt, size_t kv_extent, const std::string& ctx) {
    using G = WideGeo<D>;
    const bool whole = kt * G::BN + G::BN <= r.kv_valid;
    for (int cw = 0; cw < G::COPY_WAVES; ++cw)
        for (int ii = 0; ii < G::NKW; ++ii) {
            const int f = cw + G::COPY_WAVES * ii;
            for (int lane = 0; lane < 64; ++lane) {
                const Chunk c = wide_k_chunk(f, lane, G::KC);
                uint64_t off;
                if (whole) {
                    off = wide_k_copy_base(f, r.kv_rs, G::KC) + wide_k_lane_off(lane, r.kv_rs);
                    ++g_checks;
                    if (off != chunk_offset(c, r.kv_rs)) fail(ctx + " K whole-tile split disagrees with its chunk");
                } else {
                    off = tail_offset(c, 32 * (f / G::KC), r.kv_valid, kt * G::BN, r.kv_rs);
                }
                check_chunk("K", r, kt, G::BN, off, kv_extent, D, ctx);
                check_lds("K", (long)(kt & 1) * G::K_BYTES + f * 1024 + 16 * lane, 2L * G::K_BYTES, ctx);
            }
        }
    for (int cw = 0; cw < G::COPY_WAVES; ++cw)
        for (int ii = 0; ii < G::NVW; ++ii) {
            const int j = cw + G::COPY_WAVES * ii;
            for (int lane = 0; lane < 64; ++lane) {
                const Chunk c = wide_v_chunk(j, lane, G::DB);
                uint64_t off;
                if (whole) {
                    off = wide_v_copy_base(j, r.kv_rs, G::DB) + wide_v_lane_off(lane, r.kv_rs);
                    ++g_checks;
                    if (off != chunk_offset(c, r.kv_rs)) fail(ctx + " V whole-tile split disagrees with its chunk");
                } else {
                    off = tail_offset(c, 16 * (j / G::DB), r.kv_valid, kt * G::BN, r.kv_rs);
                }
                check_chunk("V", r, kt, G::BN, off, kv_extent, D, ctx);
                check_lds("V", (long)(kt & 1) * G::V_BYTES + j * 1024 + 16 * lane, 2L * G::V_BYTES, ctx);
            }
        }
}

template <int D>
void prefill_narrow(const Prefill& p, const Rows& r, int kt, size_t kv_extent, const std::string& ctx) {
    constexpr int W = 4;
    using G = NarrowGeo<D, W>;
    const bool whole = kt * G::BN + G::BN <= r.kv_valid;
    for (int wave = 0; wave < W; ++wave) {
        for (int ii = 0; ii < G::NKW; ++ii) {
            const int i = wave + W * ii;
            if (i >= G::NK) continue;   // the kernel issues no such copy
            for (int lane = 0; lane < 64; ++lane) {
                const Chunk c = narrow_k_chunk(i, lane, G::CPR);
                const uint64_t off = whole ? (uint64_t)chunk_offset(c, r.kv_rs)
                                           : tail_offset(c, (64 * i) / G::KS, r.kv_valid, kt * G::BN, r.kv_rs);
                check_chunk("K", r, kt, G::BN, off, kv_extent, D, ctx);
                check_lds("K", (long)(kt & 1) * G::K_BYTES + i * 1024 + 16 * lane, 2L * G::K_BYTES, ctx);
            }
        }
        for (int ii = 0; ii < G::NVW; ++ii) {
            const int i = wave + W * ii;
            for (int lane = 0; lane < 64; ++lane) {
                const Chunk c = narrow_v_chunk(i, lane, D);
                uint64_t off;
                if (whole) {
                    // the kernel: wave's copy-0 offset plus ii whole steps
                    const uint64_t o = chunk_offset(narrow_v_chunk(wave, lane, D), r.kv_rs) +
                                       (uint64_t)ii * narrow_v_copy_step(W, D, r.kv_rs);
                    off = o;
                    ++g_checks;
                    if (o != chunk_offset(c, r.kv_rs)) fail(ctx + " V whole-tile step disagrees with its chunk");
                } else {
                    off = tail_offset(c, (64 * i) / G::CPR, r.kv_valid, kt * G::BN, r.kv_rs);
                }
                check_chunk("V", r, kt, G::BN, off, kv_extent, D, ctx);
                check_lds("V", (long)(kt & 1) * G::V_BYTES + i * 1024 + 16 * lane, 2L * G::V_BYTES, ctx);
            }
        }
    }
}

// The Q copies of the head-dim-32/64 kernel's next q-tile: wave w, lane l, k-step kc reads
// 16 bytes at the wave's first row (clamped) plus plan::q_copy_offset, into its 1 KiB block
// of the Q buffer.
template <int D>
void q_copies(const Rows& r, int q0, size_t q_extent, const std::string& ctx) {
    constexpr int W = 4;
    using G = NarrowGeo<D, W>;
    for (int wave = 0; wave < W; ++wave) {
        const int rb = imin(q0 + wave * 32, r.q_len - 1);
        for (int lane = 0; lane < 64; ++lane) {
            const int row = imin(q0 + wave * 32 + (lane & 31), r.q_len - 1);
            for (int kc = 0; kc < G::KC; ++kc) {
                const uint64_t byte = (uint64_t)(r.q_base + (size_t)rb * r.q_rs) * 2 +
                                      q_copy_offset(row - rb, lane >> 5, r.q_rs) + 32 * kc;
                const uint64_t want = (uint64_t)(r.q_base + (size_t)row * r.q_rs + 8 * (lane >> 5) + 16 * kc) * 2;
                ++g_checks;
                if (byte != want || row < 0 || row >= r.q_len || 8 * (lane >> 5) + 16 * kc + 8 > D ||
                    byte + 16 > (uint64_t)q_extent * 2)
                    fail(ctx + " Q copy wave " + std::to_string(wave) + " lane " + std::to_string(lane) + " kc " +
                         std::to_string(kc) + " reads outside the q-tile's rows");
                check_lds("Q", (long)(wave * G::KC + kc) * 1024 + 16 * lane, (long)W * G::KC * 1024, ctx);
            }
        }
    }
}

template <int D>
void prefill(const Prefill& p, int slots) {
    constexpr bool wide = D == 128;
    constexpr int BN = 64;
    constexpr int kMaxList = 64;   // the narrow kernel's list capacity
    const int BM = wide ? WideGeo<D>::BM : NarrowGeo<D, 4>::BM;
    const Layout lay = (Layout)p.layout;
    std::vector<int> cu(p.B + 1, 0);
    if (lay == kUnpadded)
        for (int b = 0; b < p.B; ++b) cu[b + 1] = cu[b] + p.lens[b];
    const int tokens = cu[p.B];
    const size_t q_extent = lay == kUnpadded ? (size_t)tokens * p.Hq * D : (size_t)p.B * p.Hq * p.Lq * D;
    const size_t kv_extent = lay == kUnpadded ? (size_t)tokens * p.Hkv * D : (size_t)p.B * p.Hkv * p.Lk * D;
    const int n_qtiles = (p.Lq + BM - 1) / BM;
    const long tiles = (long)n_qtiles * p.Hq * p.B;
    std::vector<char> seen((size_t)tiles, 0);
    const int qgrp = p.Hq / p.Hkv;

    // one (q-tile, item, head): its rows, Q / output addresses, key tiles and their copies
    auto tile = [&](int qt, int b, int h, const std::string& ctx) {
        ++g_checks;
        if (qt < 0 || qt >= n_qtiles || b < 0 || b >= p.B || h < 0 || h >= p.Hq) {
            fail(ctx + " maps outside the grid");
            return;
        }
        char& s = seen[((size_t)qt * p.B + b) * p.Hq + h];
        if (s) fail(ctx + " maps onto a (q-tile, item, head) already taken");
        s = 1;
        const int kvh = h / qgrp;
        const bool has_len = lay != kUnpadded && !p.lens.empty();
        const Rows r = item_rows(lay, b, h, kvh, D, p.Hq, p.Hkv, p.Lq, p.Lk, cu[b], lay == kUnpadded ? cu[b + 1] : 0,
                                 has_len, has_len ? p.lens[b] : 0);
        const int q0 = qt * BM;
        if (q0 >= r.q_len) return;
        const int last_row = imin(q0 + BM, r.q_len) - 1;
        // Q rows the workgroup loads (clamped to the last row) and the rows it stores
        for (int row = q0; row < q0 + BM; ++row) {
            const size_t at = r.q_base + (size_t)imin(row, r.q_len - 1) * r.q_rs;
            ++g_checks;
            if (at + D > q_extent) fail(ctx + " Q row " + std::to_string(row) + " outside q");
            if (row < r.q_len && r.q_base + (size_t)row * r.q_rs + D > q_extent)
                fail(ctx + " output row " + std::to_string(row) + " outside out");
        }
        if (!wide) q_copies<D>(r, q0, q_extent, ctx);
        const Tiles t = key_tiles(span_union(p.P + q0, p.P + last_row, r.kv_valid, p.causal != 0, p.W), BN);
        for (int kt = t.begin; kt < t.end; ++kt) {
            ++g_checks;
            if (kt * BN >= r.kv_valid) fail(ctx + " visits tile " + std::to_string(kt) + " past the valid keys");
            if (wide)
                prefill_wide<D>(p, r, kt, kv_extent, ctx);
            else
                prefill_narrow<D>(p, r, kt, kv_extent, ctx);
        }
    };

    if (wide) {
        for (long blk = 0; blk < tiles; ++blk) {
            const BlockCoord bc = map_block((unsigned)blk, n_qtiles, p.B, p.Hq, p.Hkv,
                                            p.causal != 0 || !p.lens.empty() || lay == kUnpadded, 8);
            tile(bc.qt, bc.b, bc.h,
                 "prefill D" + std::to_string(D) + " block " + std::to_string(blk) + " (qt " + std::to_string(bc.qt) +
                     ", b " + std::to_string(bc.b) + ", h " + std::to_string(bc.h) + ")");
        }
    } else {
        // the persistent grid: every workgroup's list, at most kMaxList q-tiles long; with
        // per-item lengths for at most kRankedItems items the lists follow the ranked order
        const bool ranked = ranked_order(!p.lens.empty(), p.B, n_qtiles, p.Hq);
        std::vector<int> order(p.B), ne(p.B), nrow(p.B), cost(p.B);
        std::vector<int> start_ne(p.B), start_z(p.B);
        int n_ne = 0, n_z = 0;
        if (ranked) {
            for (int b = 0; b < p.B; ++b) {
                const int rows = lay == kUnpadded ? imin(imax(p.lens[b], 0), p.Lq) : p.Lq;
                const int valid = lay == kUnpadded ? rows : imin(imax(p.lens[b], 0), p.Lk);
                const ItemSched is = item_sched(rows, valid, p.P, p.causal != 0, p.W, BM, BN);
                ne[b] = is.ne;
                nrow[b] = is.nrow;
                cost[b] = is.cost;
            }
            // the kernel ranks by comparing one key per item: the same order as ranks_before
            std::vector<int> taken(p.B, 0);
            for (int b = 0; b < p.B; ++b) {
                int rank = 0;
                for (int x = 0; x < p.B; ++x) {
                    ++g_checks;
                    const bool before = rank_key(cost[x], x) > rank_key(cost[b], b);
                    if (before != ranks_before(cost[x], x, cost[b], b)) fail("rank_key disagrees with ranks_before");
                    rank += before ? 1 : 0;
                }
                ++g_checks;
                if (taken[rank]++) fail("two items of one rank");
                order[rank] = b;
            }
            for (int r = 0; r < p.B; ++r) {
                start_ne[r] = n_ne;
                n_ne += ne[order[r]] * p.Hq;
            }
            for (int b = 0; b < p.B; ++b) {
                start_z[b] = n_z;
                n_z += (nrow[b] - ne[b]) * p.Hq;
                // q-tiles without rows are in no list
                for (int qt = nrow[b]; qt < n_qtiles; ++qt)
                    for (int h = 0; h < p.Hq; ++h) seen[((size_t)qt * p.B + b) * p.Hq + h] = 1;
            }
        }
        const int wgs = persist_grid(tiles, slots, 8, kMaxList);
        ++g_checks;
        if (wgs % 8 != 0 || wgs <= 0) fail("prefill D" + std::to_string(D) + " grid of " + std::to_string(wgs));
        for (int wg = 0; wg < wgs; ++wg) {
            ++g_checks;
            if (persist_pos(wg, kMaxList, wgs, 8) < tiles)
                fail("prefill D" + std::to_string(D) + " workgroup " + std::to_string(wg) + " of " +
                     std::to_string(wgs) + " has more than " + std::to_string(kMaxList) + " q-tiles");
            for (int k = 0; k < kMaxList; ++k) {
                const long pos = persist_pos(wg, k, wgs, 8);
                TileRef tr{};
                if (ranked) {
                    const RankedRef rr = ranked_tile(pos < n_ne + n_z ? (int)pos : -1, p.B, n_ne, n_z, order.data(),
                                                     start_ne.data(), start_z.data(), ne.data(), nrow.data());
                    if (rr.kind == 2) break;
                    tr = {rr.b, rr.h, rr.qt};
                    // the kind the kernel derives from the q-tile's key tiles must agree
                    const int rows = lay == kUnpadded ? imin(imax(p.lens[rr.b], 0), p.Lq) : p.Lq;
                    const int valid = lay == kUnpadded ? rows : imin(imax(p.lens[rr.b], 0), p.Lk);
                    const int q0 = rr.qt * BM;
                    ++g_checks;
                    if (q0 >= rows) {
                        fail("ranked q-tile without rows");
                    } else {
                        const Tiles t = key_tiles(
                            span_union(p.P + q0, p.P + imin(q0 + BM, rows) - 1, valid, p.causal != 0, p.W), BN);
                        if ((t.end > t.begin) != (rr.kind == 0)) fail("ranked q-tile of the wrong kind");
                    }
                } else {
                    if (pos >= tiles) break;
                    tr = persist_tile(pos, p.Hq, n_qtiles);
                }
                tile(tr.qt, tr.b, tr.h,
                     "prefill D" + std::to_string(D) + " workgroup " + std::to_string(wg) + " of " +
                         std::to_string(wgs) + " entry " + std::to_string(k) + " (qt " + std::to_string(tr.qt) +
                         ", b " + std::to_string(tr.b) + ", h " + std::to_string(tr.h) + ")");
            }
        }
    }
    for (long i = 0; i < tiles; ++i)
        if (!seen[(size_t)i]) {
            fail("(q-tile, item, head) " + std::to_string(i) + " has no workgroup");
            break;
        }
}

// EPL: elements per lane and row (8 for fp32 caches and head dim 32, 16 for 16-bit caches
// at head dims 64 and 128); both shapes are checked where both can run.
template <int D, int EPL>
void decode(int mode, int B, int Hq, int Hkv, int cap, int kv_len, int P, int window, const std::vector<int>& lens) {
    using G = DecodeGeo<D, EPL>;
    const int len_arg = mode == 0 ? kv_len : cap;
    const DecodePlan pl = decode_plan(B, Hq, Hkv, len_arg, 512);
    const size_t head_extent = (size_t)cap * D;   // one (item, kv head) cache
    for (int b = 0; b < B; ++b)
        for (int y = 0; y < Hkv * pl.head_groups; ++y)
            for (int split = 0; split < pl.splits; ++split) {
                const DecodeQuery dq = decode_query(mode == 2, !lens.empty(), lens.empty() ? 0 : lens[b], len_arg,
                                                    cap, P);
                const KeyRange kr = decode_split_keys(dq, window, split, pl.split_len);
                const std::string ctx = "decode D" + std::to_string(D) + " b " + std::to_string(b) + " split " +
                                        std::to_string(split);
                ++g_checks;
                if (dq.len > cap) fail(ctx + " length past the capacity");
                auto batch = [&](int base, bool tail) {
                    for (int u = 0; u < G::STEPS; ++u)
                        for (int wave = 0; wave < G::WAVES; ++wave)
                            for (int r = 0; r < G::RPW; ++r) {
                                const int key = base + (u * G::WAVES + wave) * G::RPW + r;
                                const int row = decode_key_row(key, kr.s0, kr.s1, tail);
                                ++g_checks;
                                if (row < kr.s0 || row >= kr.s1 || row < 0 || row >= dq.len ||
                                    (size_t)row * D + D > head_extent)
                                    fail(ctx + " reads cache row " + std::to_string(row));
                            }
                };
                int base = kr.s0;
                for (; base + G::BATCH < kr.s1; base += G::BATCH) batch(base, false);
                if (base < kr.s1) batch(base, true);
            }
}

}  // namespace

int main(int argc, char** argv) {
    for (int i = 1; i < argc; ++i)
        if (!std::strcmp(argv[i], "--plant")) g_plant = true;
    std::string line;
    while (std::getline(std::cin, line)) {
        std::istringstream in(line);
        std::string kind;
        if (!(in >> kind)) continue;
        if (kind == "prefill") {
            Prefill p{};
            int n = 0;
            in >> p.layout >> p.B >> p.Hq >> p.Hkv >> p.Lq >> p.Lk >> p.D >> p.P >> p.causal >> p.W >> n;
            p.lens.resize(n);
            for (int& x : p.lens) in >> x;
            if (!in) {
                std::printf("FAIL unreadable line: %s\n", line.c_str());
                return 2;
            }
            // the narrow kernel's grid depends on the device's workgroup slots: MI355X's
            // 512, and small counts whose lists run long
            if (p.D == 32 || p.D == 64) {
                for (int slots : {512, 40, 8}) {
                    if (p.D == 32)
                        prefill<32>(p, slots);
                    else
                        prefill<64>(p, slots);
                }
            } else if (p.D == 128) {
                prefill<128>(p, 0);
            }
        } else if (kind == "decode") {
            int mode, B, Hq, Hkv, cap, kv_len, D, P, W, n;
            in >> mode >> B >> Hq >> Hkv >> cap >> kv_len >> D >> P >> W >> n;
            std::vector<int> lens(n);
            for (int& x : lens) in >> x;
            if (!in) {
                std::printf("FAIL unreadable line: %s\n", line.c_str());
                return 2;
            }
            if (D == 32)
                decode<32, 8>(mode, B, Hq, Hkv, cap, kv_len, P, W, lens);
            else if (D == 64) {
                decode<64, 8>(mode, B, Hq, Hkv, cap, kv_len, P, W, lens);
                decode<64, 16>(mode, B, Hq, Hkv, cap, kv_len, P, W, lens);
            } else {
                decode<128, 8>(mode, B, Hq, Hkv, cap, kv_len, P, W, lens);
                decode<128, 16>(mode, B, Hq, Hkv, cap, kv_len, P, W, lens);
            }
        }
    }
    // the ranked order's guards and key: q-tile numbers must fit 31 bits, at most
    // kRankedItems items, lengths given; the key orders as ranks_before up to the largest
    // cost a 31-bit key count allows
    {
        const bool guards[] = {ranked_order(true, 64, 1 << 20, 4096), ranked_order(true, 65, 1, 1),
                               ranked_order(false, 4, 4, 4), !ranked_order(true, 64, 1 << 12, 8191),
                               !ranked_order(true, 1, 1, 1)};
        for (bool bad : guards) {
            ++g_checks;
            if (bad) fail("ranked_order guard");
        }
        const int costs[] = {0, 1, 2, 63, 64, 65, (1 << 25) - 1, 1 << 25};
        for (int ca : costs)
            for (int cb : costs)
                for (int a = 0; a < kRankedItems; a += 21)
                    for (int b = 0; b < kRankedItems; b += 13) {
                        if (a == b) continue;
                        ++g_checks;
                        if ((rank_key(ca, a) > rank_key(cb, b)) != ranks_before(ca, a, cb, b)) fail("rank_key order");
                        if (rank_key(ca, a) == 0u) fail("rank_key zero");
                    }
    }
    if (g_fails) {
        std::printf("FAIL total %d violations in %ld checks\n", g_fails, g_checks);
        return 1;
    }
    std::printf("ok %ld\n", g_checks);
    return 0;
}
