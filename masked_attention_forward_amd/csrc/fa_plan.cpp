// fa_plan.cpp - host-side validation and planning (no HIP dependency).
//
// Validation follows the rules the pages state, in "sparseMode介绍":
//   sparseMode=0: negative nextTokens needs preTokens >= |nextTokens| and |nextTokens| < Skv;
//                 negative preTokens needs nextTokens >= |preTokens| and |preTokens| < Sq.
//   sparseMode=4: preTokens and nextTokens must intersect (read as pre + next >= 0).
//   sparseMode=7: band batch: preTokens >= last_Skv, last_Sq - last_Skv <= nextTokens <= 0;
//                 other batches Sq <= Skv; the optional pse (bias) input is not supported.
//   sparseMode=8: band batch: preTokens >= first_Skv, nextTokens >= first_Sq - first_Skv;
//                 no pse.
// and in "压缩mask" (constraints): alibi needs a head size of at most 128.
// Every check runs before any device work, as the return-code table of the
// "aclnnScatterPaKvCache" doc describes for its first phase.
#include "fa_plan.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <queue>

namespace {

int64_t clamp64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The MFMA kernels address a tile with 32-bit byte offsets: 256 rows of the widest row
// stride (N * D elements for BSND / TND) must stay below 2^31 bytes.
bool mfma_eligible(int32_t dtype, int64_t N, int64_t D) {
    return (dtype == FA_DTYPE_F16 || dtype == FA_DTYPE_BF16) && (D == 64 || D == 128) &&
           N * D * 2 * 256 < (int64_t(1) << 31);
}

// FA_KERNEL=mfma32 selects the 4-wave MFMA kernel instead of the ping-pong one (for
// comparisons).
bool prefer_mfma32() {
    const char* e = std::getenv("FA_KERNEL");
    return e && std::strcmp(e, "mfma32") == 0;
}

// FA_DECODE=0 keeps short-query problems on the prefill kernels (for comparisons).
bool decode_enabled() {
    const char* e = std::getenv("FA_DECODE");
    return !(e && e[0] == '0');
}

}  // namespace

static fa_status make_plan_impl(const fa_call& call, bool with_tables, bool sizes_only,
                                fa_plan* out) {
    if (!call.dims || !out) return FA_ERR_NULLPTR;
    const fa_dims& d = *call.dims;
    const int mode = call.sparse_mode;
    const bool tnd = call.layout == FA_LAYOUT_TND;

    if (d.dtype < FA_DTYPE_F32 || d.dtype > FA_DTYPE_BF16) return FA_ERR_PARAM_INVALID;
    if (call.layout < FA_LAYOUT_BNSD || call.layout > FA_LAYOUT_TND) return FA_ERR_PARAM_INVALID;
    if (mode < 0 || mode > 8) return FA_ERR_PARAM_INVALID;
    if (d.B < 0 || d.N < 1 || d.D < 1) return FA_ERR_PARAM_INVALID;
    if (d.B > (int64_t(1) << 24) || d.N > (int64_t(1) << 16)) return FA_ERR_UNSUPPORTED;
    if ((mode == 7 || mode == 8) && !tnd) return FA_ERR_PARAM_INVALID;
    if (!sizes_only) {
        if (call.check_scale && !(std::isfinite(call.scale) && call.scale > 0.0f))
            return FA_ERR_PARAM_INVALID;
        if (call.alibi_mode != FA_ALIBI_RIGHT && call.alibi_mode != FA_ALIBI_SQRT &&
            call.alibi_mode != FA_ALIBI_LEFT)
            return FA_ERR_PARAM_INVALID;
        if (call.has_alibi && d.D > 128) return FA_ERR_PARAM_INVALID;
        if (call.has_alibi && (mode == 7 || mode == 8)) return FA_ERR_PARAM_INVALID;
        if (mode == 1 && !call.has_mask) return FA_ERR_NULLPTR;
    }
    if (mode == 1 && tnd) return FA_ERR_UNSUPPORTED;
    if (d.D > 128) return FA_ERR_UNSUPPORTED;
    const fa_paged_kv* pk = call.paged;
    if (pk) {
        if (pk->cache_layout != FA_CACHE_NORM && pk->cache_layout != FA_CACHE_NHSD) return FA_ERR_PARAM_INVALID;
        if (pk->reserved != 0) return FA_ERR_PARAM_INVALID;
        if (pk->block_size < 1 || pk->num_blocks < 1 || pk->max_blocks_per_seq < 1) return FA_ERR_PARAM_INVALID;
        if (pk->block_size > (int64_t(1) << 24) || pk->num_blocks > INT32_MAX ||
            pk->max_blocks_per_seq > (int64_t(1) << 24))
            return FA_ERR_UNSUPPORTED;
        // Cache elements (and so every page offset) must stay well inside int64.
        if (double(pk->num_blocks) * double(pk->block_size) * double(d.N) * double(d.D) > std::ldexp(1.0, 60))
            return FA_ERR_UNSUPPORTED;
    }

    const int64_t B = d.B;
    std::vector<int64_t> sq(B), skv(B), qs(B), ks(B);
    if (tnd) {
        if (B > 0 && (!call.actual_seq_qlen || !call.actual_seq_kvlen)) return FA_ERR_NULLPTR;
        int64_t pq = 0, pk = 0;
        for (int64_t b = 0; b < B; ++b) {
            const int64_t cq = call.actual_seq_qlen[b], ck = call.actual_seq_kvlen[b];
            if (cq < pq || ck < pk) return FA_ERR_PARAM_INVALID;  // cumulative ends only grow
            qs[b] = pq;
            ks[b] = pk;
            sq[b] = cq - pq;
            skv[b] = ck - pk;
            if (sq[b] >= FA_MAX_SEQ || skv[b] >= FA_MAX_SEQ) return FA_ERR_UNSUPPORTED;
            pq = cq;
            pk = ck;
        }
        if (pq != d.T_q || pk != d.T_kv) return FA_ERR_PARAM_INVALID;
        if (d.T_q >= (int64_t(1) << 31) || d.T_kv >= (int64_t(1) << 31)) return FA_ERR_UNSUPPORTED;
    } else {
        if (d.Sq < 0 || d.Skv < 0) return FA_ERR_PARAM_INVALID;
        if (d.Sq >= FA_MAX_SEQ || d.Skv >= FA_MAX_SEQ) return FA_ERR_UNSUPPORTED;
        for (int64_t b = 0; b < B; ++b) {
            sq[b] = d.Sq;
            skv[b] = d.Skv;
            qs[b] = ks[b] = 0;
        }
    }
    // Element counts must stay well inside int64.
    {
        const double rows = tnd ? double(d.T_q) : double(B) * double(d.Sq);
        const double keys = tnd ? double(d.T_kv) : double(B) * double(d.Skv);
        const double big = std::ldexp(1.0, 60);
        if (rows * double(d.N) * double(d.D) > big || keys * double(d.N) * double(d.D) > big)
            return FA_ERR_UNSUPPORTED;
    }
    int64_t max_sq = 0, max_skv = 0;
    for (int64_t b = 0; b < B; ++b) {
        max_sq = std::max(max_sq, sq[b]);
        max_skv = std::max(max_skv, skv[b]);
    }
    // The block table must reach the last key of the longest sequence.
    if (pk && max_skv > pk->max_blocks_per_seq * pk->block_size) return FA_ERR_PARAM_INVALID;

    // Mode-specific arguments.
    const int64_t pre = call.pre_tokens, nxt = call.next_tokens;
    const bool band_mode = mode == 0 || mode == 4 || mode == 7 || mode == 8;
    const int64_t huge = int64_t(1) << 62;
    int64_t band_b = -1;
    if (mode == 7 || mode == 8) {
        for (int64_t b = 0; b < B; ++b) {
            if (sq[b] > 0 && skv[b] > 0) {
                band_b = b;
                if (mode == 8) break;
            }
        }
    }
    if (!sizes_only) {
        if (band_mode && (pre < -huge || nxt < -huge)) return FA_ERR_PARAM_INVALID;
        if (mode == 0) {
            if (nxt < 0 && !(pre >= -nxt && -nxt < max_skv)) return FA_ERR_PARAM_INVALID;
            if (pre < 0 && !(nxt >= -pre && -pre < max_sq)) return FA_ERR_PARAM_INVALID;
        }
        if (mode == 4 && clamp64(pre, -huge, huge) < -clamp64(nxt, -huge, huge))  // pre + next < 0
            return FA_ERR_PARAM_INVALID;
        if (mode == 7) {
            for (int64_t b = 0; b < B; ++b) {
                if (b == band_b) {
                    if (!(pre >= skv[b] && sq[b] - skv[b] <= nxt && nxt <= 0))
                        return FA_ERR_PARAM_INVALID;
                } else if (sq[b] > skv[b]) {
                    return FA_ERR_PARAM_INVALID;
                }
            }
        }
        if (mode == 8 && band_b >= 0) {
            if (!(pre >= skv[band_b] && nxt >= sq[band_b] - skv[band_b])) return FA_ERR_PARAM_INVALID;
        }
        if (mode == 5 || mode == 6) {
            if (B > 0 && !call.prefix) return FA_ERR_NULLPTR;
            for (int64_t b = 0; b < B; ++b)
                if (call.prefix[b] < 0) return FA_ERR_PARAM_INVALID;
        }
    }

    fa_plan p;
    p.B = int32_t(B);
    p.N = int32_t(d.N);
    p.D = int32_t(d.D);
    p.kernel = FA_KERNEL_GENERIC;
    p.bm = FA_GEN_BM;
    p.bn = FA_GEN_BN;
    // Paged K / V through the MFMA kernels: 64-key tiles inside one page, page offsets in
    // 32 bits, at most FA_PP_MAX_PAGES pages per sequence.
    bool paged_mfma_ok = true;
    if (pk) {
        const int64_t bs = pk->block_size;
        paged_mfma_ok = (bs & (bs - 1)) == 0 && bs >= FA_PP_BN && ceil_div(max_skv, bs) <= FA_PP_MAX_PAGES &&
                        bs * d.N * d.D * 2 < (int64_t(1) << 32);
    }
    if (mfma_eligible(d.dtype, d.N, d.D) && max_sq <= FA_DEC_ROWS && mode != 1 && paged_mfma_ok &&
        decode_enabled() && B > 0) {
        p.kernel = FA_KERNEL_DECODE;
        p.bm = FA_DEC_ROWS;
        p.bn = FA_DEC_BN;
    } else if (pk) {
        // Paged K / V: the ping-pong kernel when its tiles fit whole pages, a sequence has at
        // most FA_PP_MAX_PAGES pages and a page is under 4 GiB; else the generic kernel (any
        // block size, explicit masks too).
        const int64_t bs = pk->block_size;
        const bool pow2 = (bs & (bs - 1)) == 0;
        const int64_t page_bytes = bs * d.N * d.D * 2;
        if (mfma_eligible(d.dtype, d.N, d.D) && mode != 1 && pow2 && bs >= FA_PP_BN &&
            ceil_div(max_skv, bs) <= FA_PP_MAX_PAGES && page_bytes < (int64_t(1) << 32)) {
            p.kernel = FA_KERNEL_PP;
            p.bm = FA_PP_BM;
            p.bn = FA_PP_BN;
        }
    } else if (mfma_eligible(d.dtype, d.N, d.D)) {
        if (!prefer_mfma32()) {
            p.kernel = FA_KERNEL_PP;
            p.bm = FA_PP_BM;
            p.bn = FA_PP_BN;
        } else {
            p.kernel = FA_KERNEL_MFMA32;
            p.bm = FA_MFMA32_BM;
            p.bn = FA_MFMA32_BN;
        }
    }
    for (int64_t b = 0; b < B; ++b) {
        p.rows_total += sq[b];
        p.kv_total += skv[b];
    }
    p.empty = p.rows_total == 0;

    // Geometry per batch (see fa_mask.h for the a / c / f rule table).
    const int32_t prei = int32_t(clamp64(pre, -FA_LIM, FA_LIM));
    const int32_t nxti = int32_t(clamp64(nxt, -FA_LIM, FA_LIM));
    p.geoms.resize(B);
    for (int64_t b = 0; b < B; ++b) {
        fa_geom g{};
        g.q_start = int32_t(qs[b]);
        g.kv_start = pk ? 0 : int32_t(ks[b]);   // a paged sequence starts at key 0 of its pages
        g.sq = int32_t(sq[b]);
        g.skv = int32_t(skv[b]);
        const int32_t off = g.skv - g.sq;
        int m = mode;
        if (m == 7) m = (b == band_b) ? 4 : 3;
        if (m == 8) m = (b == band_b) ? 4 : 2;
        g.f = -FA_BIG;
        switch (m) {
            case 0: g.a = -prei; g.c = nxti; break;
            case 1: g.a = -FA_BIG; g.c = FA_BIG; break;
            case 2: g.a = -FA_BIG; g.c = 0; break;
            case 3: g.a = -FA_BIG; g.c = off; break;
            case 4: g.a = off - prei; g.c = off + nxti; break;
            default: {  // 5, 6
                g.a = -FA_BIG;
                g.c = off;
                const int64_t pl = sizes_only ? 0 : std::min<int64_t>(call.prefix[b], g.skv);
                g.f = int32_t(pl) - 1;
                break;
            }
        }
        p.geoms[b] = g;
    }
    if (B > 0) p.geom0 = p.geoms[0];

    // Strides (elements).
    const int64_t N = d.N, D = d.D;
    if (call.layout == FA_LAYOUT_BNSD) {
        p.q_bs = N * d.Sq * D; p.q_hs = d.Sq * D; p.q_rs = D;
        p.kv_bs = N * d.Skv * D; p.kv_hs = d.Skv * D; p.kv_rs = D;
    } else if (call.layout == FA_LAYOUT_BSND) {
        p.q_bs = d.Sq * N * D; p.q_hs = D; p.q_rs = N * D;
        p.kv_bs = d.Skv * N * D; p.kv_hs = D; p.kv_rs = N * D;
    } else {
        p.q_bs = 0; p.q_hs = D; p.q_rs = N * D;
        p.kv_bs = 0; p.kv_hs = D; p.kv_rs = N * D;
    }
    if (pk) {
        const int64_t bs = pk->block_size;
        p.paged = true;
        p.kv_bs = 0;
        if (pk->cache_layout == FA_CACHE_NORM) {   // [num_blocks, block_size, N, D]
            p.page_stride = bs * N * D; p.kv_hs = D; p.kv_rs = N * D;
        } else {                                   // [num_blocks, N, block_size, D]
            p.page_stride = N * bs * D; p.kv_hs = bs * D; p.kv_rs = D;
        }
        p.bt_stride = pk->max_blocks_per_seq;
        p.block_size = int32_t(bs);
        p.log2_block_size = -1;
        if ((bs & (bs - 1)) == 0)
            for (int32_t e = 0; e < 31; ++e)
                if ((int64_t(1) << e) == bs) p.log2_block_size = e;
        p.num_pages = int32_t(pk->num_blocks);
    }
    if (tnd) {
        p.lse_bs = 0; p.lse_hs = d.T_q;
    } else {
        p.lse_bs = N * d.Sq; p.lse_hs = d.Sq;
    }
    if (mode == 1) {
        const bool bb = call.mask_bcast && call.mask_bcast[0] != 0;
        const bool hb = call.mask_bcast && call.mask_bcast[1] != 0;
        const int64_t nm = hb ? 1 : N;
        p.m_rs = d.Skv;
        p.m_hs = hb ? 0 : d.Sq * d.Skv;
        p.m_bs = bb ? 0 : nm * d.Sq * d.Skv;
        if (p.kernel == FA_KERNEL_PP && !tnd) {
            // The ping-pong kernel visits only the kv tiles the pre-pass found a visible entry in.
            p.dense_tiles = true;
            p.m_bcast_b = bb ? 1 : 0;
            p.m_bcast_h = hb ? 1 : 0;
            p.mask_heads = int32_t(nm);
            p.mask_slices = int32_t((bb ? 1 : B) * nm);
            p.dense_nqt = int32_t(ceil_div(d.Sq, FA_PP_BM));
            p.dense_nkt = int32_t(ceil_div(d.Skv, FA_PP_BN));
        }
    }

    // Work items.
    p.table = tnd || mode == 5 || mode == 6;
    p.n_qtiles_total = 0;
    p.n_kvtiles_max = 0;
    for (int64_t b = 0; b < B; ++b) {
        p.n_qtiles_total += ceil_div(sq[b], p.bm);
        p.n_kvtiles_max = std::max(p.n_kvtiles_max, ceil_div(skv[b], p.bn));
    }
    // The skip costs a uniform test per tile, which measured about 0.5% on long causal items
    // (2 x 32 x 8192^2, 128-tile items) and gained 1-8% where edge tiles are a larger share of
    // each item: a band with a lower bound (modes 0 and 4, the band batch of 7 / 8) or items of
    // at most 64 kv tiles (varlen with sequences up to 4096 keys: +1.2%). Dense masks and alibi keep the plain kernel.
    if (p.kernel == FA_KERNEL_PP && mode != 1 && !call.has_alibi) {
        bool lower = false;
        for (const fa_geom& g : p.geoms) lower = lower || int64_t(g.sq) - 1 + g.a > 0;   // some row's lo > 0
        p.edge_skip = lower || p.n_kvtiles_max <= 64;
        if (const char* ee = std::getenv("FA_EDGE"))   // 0 | 1: override (comparisons and tests)
            p.edge_skip = std::atoi(ee) != 0;
    }
    auto item_cost = [&](int64_t b, int64_t qt, int64_t* full) -> int64_t {
        const fa_geom& g = p.geoms[b];
        const int32_t i0 = int32_t(qt * p.bm);
        const int32_t i1 = std::min<int32_t>(i0 + p.bm, g.sq) - 1;
        const fa_kv_range r = fa_tile_kv_range(g, i0, i1, p.bn);
        if (full) {
            // fa_tile_full is the conjunction of one bound on the tile's first column and two
            // on its last, so the full tiles of a q tile are one contiguous run: find its ends
            // from both sides. Only the few tiles that a mask edge crosses are partial, so
            // both scans stop after a handful of steps even for a very long kv range.
            *full = 0;
            if (mode != 1) {
                int32_t lo = r.begin, hi = r.end;
                while (lo < hi && !fa_tile_full(g, i0, i1, lo * p.bn, p.bn)) ++lo;
                while (hi > lo && !fa_tile_full(g, i0, i1, (hi - 1) * p.bn, p.bn)) --hi;
                *full = hi - lo;
            }
        }
        return r.end - r.begin;
    };
    if (p.kernel == FA_KERNEL_DECODE) {
        // Split-KV decode: sequence b's kv tiles (by its length, not its visible range, so the
        // workspace-size query plans the same) are cut into ns_b splits of at most C tiles, one
        // workgroup per (split, head). C comes from a model of the launch: a workgroup costs
        // its tiles plus FA_DEC_WG_COST, the chip holds FA_DEC_SLOTS of them at once (per CU,
        // what the kernel's LDS allows), the makespan is the larger of the total cost over the
        // slots and the longest workgroup (whole rounds when all are equal), and splitting adds
        // the merge kernel's FA_DEC_MERGE_COST. Table mode (per-batch geometry) launches the
        // (batch, split) entries longest first.
        const int64_t slots = FA_DEC_SLOTS * (d.D == 64 ? 2 : 1);
        std::vector<int64_t> tiles(B);
        int64_t max_tiles = 0;
        for (int64_t b = 0; b < B; ++b) {
            tiles[b] = sq[b] > 0 ? ceil_div(skv[b], FA_DEC_BN) : 0;
            max_tiles = std::max(max_tiles, tiles[b]);
        }
        auto splits_of = [](int64_t t, int64_t c) { return t <= c ? int64_t(1) : ceil_div(t, c); };
        auto estimate = [&](int64_t c) {
            double sum = 0.0, longest = 0.0, first = -1.0;
            int64_t busy = 0;
            bool split = false, equal = true;
            for (int64_t b = 0; b < B; ++b) {
                if (tiles[b] == 0) continue;
                const int64_t ns = splits_of(tiles[b], c);
                const double len = double(ceil_div(tiles[b], ns) + FA_DEC_WG_COST);
                sum += double(d.N * ns) * len;
                busy += d.N * ns;
                longest = std::max(longest, len);
                split = split || ns > 1;
                if (first < 0.0) first = len;
                equal = equal && len == first;
            }
            double t = std::max(sum / double(slots), longest);
            if (equal && busy > 0) t = std::max(t, double(ceil_div(busy, slots)) * first);
            return t + (split ? double(FA_DEC_MERGE_COST) : 0.0);
        };
        int64_t chunk = std::max<int64_t>(max_tiles, 1);
        const char* ce = std::getenv("FA_DEC_CHUNK");   // tiles per split (comparisons)
        if (ce) {
            chunk = std::max<int64_t>(1, std::atoll(ce));
        } else if (B * d.N < 8 * slots) {
            // Fewer splits win ties: each candidate must beat the best so far by 1%.
            double best = estimate(chunk);
            for (int64_t k = 2; k <= FA_DEC_MAX_SPLITS; ++k) {
                const int64_t c = ceil_div(max_tiles, k);
                if (c < FA_DEC_MIN_TILES) break;
                const double e = estimate(c);
                if (e < 0.99 * best) {
                    best = e;
                    chunk = c;
                }
            }
        }
        // Entries, splits per batch and the partial-result slots of split batches.
        std::vector<int32_t> ns_b(B);
        int64_t entries = 0, split_slots = 0;
        p.n_split = 1;
        for (int64_t b = 0; b < B; ++b) {
            ns_b[b] = int32_t(splits_of(tiles[b], chunk));
            entries += ns_b[b];
            if (ns_b[b] > 1) split_slots += ns_b[b];
            p.n_split = std::max(p.n_split, ns_b[b]);
        }
        p.dec_merge = split_slots > 0;
        p.n_items = entries;
        size_t off = 0;
        if (p.table) {
            p.ws_items_offset = align256(size_t(B) * sizeof(fa_geom));
            p.ws_dec_batch_offset = align256(p.ws_items_offset + size_t(entries) * 2 * sizeof(int32_t));
            off = align256(p.ws_dec_batch_offset + size_t(B) * 2 * sizeof(int32_t));
            p.ws_table_bytes = p.empty ? 0 : off;
            if (with_tables && !sizes_only) {
                std::vector<std::pair<int64_t, int64_t>> order;   // (tiles of the split, entry)
                std::vector<int32_t> raw;
                order.reserve(entries);
                raw.reserve(2 * entries);
                p.dec_batch.assign(2 * B, 0);
                int32_t base = 0;
                for (int64_t b = 0; b < B; ++b) {
                    p.dec_batch[2 * b] = ns_b[b] > 1 ? base : 0;
                    p.dec_batch[2 * b + 1] = ns_b[b];
                    if (ns_b[b] > 1) base += ns_b[b];
                    const int64_t len = ceil_div(tiles[b], ns_b[b]);
                    for (int32_t sp = 0; sp < ns_b[b]; ++sp) {
                        order.push_back({len, int64_t(raw.size() / 2)});
                        raw.push_back(int32_t(b));
                        raw.push_back(sp);
                    }
                }
                std::stable_sort(order.begin(), order.end(),
                                 [](const std::pair<int64_t, int64_t>& x,
                                    const std::pair<int64_t, int64_t>& y) { return x.first > y.first; });
                p.items.resize(2 * order.size());
                for (size_t n = 0; n < order.size(); ++n) {
                    p.items[2 * n] = raw[2 * order[n].second];
                    p.items[2 * n + 1] = raw[2 * order[n].second + 1];
                }
            }
        } else {
            p.ws_table_bytes = 0;
        }
        if (p.dec_merge) {
            const size_t rows = size_t(split_slots) * size_t(d.N) * FA_DEC_ROWS;
            p.ws_opart_offset = off;
            off = align256(off + rows * size_t(d.D) * sizeof(float));
            p.ws_lse_offset = off;
            off = align256(off + rows * sizeof(float));
        }
        p.ws_bytes = p.empty ? 0 : off;
    } else if (p.table) {
        p.n_items = p.n_qtiles_total;
        if (with_tables && !sizes_only) {
            std::vector<std::pair<int64_t, int64_t>> order;  // (cost, index)
            std::vector<int32_t> raw;
            order.reserve(p.n_items);
            raw.reserve(2 * p.n_items);
            for (int64_t b = 0; b < B; ++b) {
                const int64_t nqt = ceil_div(sq[b], p.bm);
                for (int64_t qt = 0; qt < nqt; ++qt) {
                    order.push_back({item_cost(b, qt, nullptr), int64_t(raw.size() / 2)});
                    raw.push_back(int32_t(b));
                    raw.push_back(int32_t(qt));
                }
            }
            // Varlen (TND) launches sequence-major: sequences by total cost, heaviest first, and
            // in each its q tiles heaviest first. The workgroups an XCD runs at once then share
            // one or two sequences' K/V in its L2 (longest-first over all sequences spreads them
            // over many sequences and re-reads K/V from HBM about four times). Prefix modes on
            // fixed-length batches launch longest first: their sequences are all long, and the
            // balance of the global order matters more there. FA_TABLE_ORDER=seq|lpt forces.
            const char* to = std::getenv("FA_TABLE_ORDER");
            bool seq_major = tnd;
            if (to && std::strcmp(to, "seq") == 0) seq_major = true;
            if (to && std::strcmp(to, "lpt") == 0) seq_major = false;
            if (seq_major) {
                std::vector<int64_t> tot(B, 0);
                for (const auto& o : order) tot[raw[2 * o.second]] += o.first;
                std::stable_sort(order.begin(), order.end(),
                                 [&](const std::pair<int64_t, int64_t>& x, const std::pair<int64_t, int64_t>& y) {
                                     const int32_t bx = raw[2 * x.second], by = raw[2 * y.second];
                                     if (bx != by) return tot[bx] != tot[by] ? tot[bx] > tot[by] : bx < by;
                                     return x.first > y.first;
                                 });
            } else {
                // Longest first; ties keep batch-major order.
                std::stable_sort(order.begin(), order.end(),
                                 [](const std::pair<int64_t, int64_t>& x,
                                    const std::pair<int64_t, int64_t>& y) { return x.first > y.first; });
            }
            p.items.resize(2 * order.size());
            for (size_t n = 0; n < order.size(); ++n) {
                p.items[2 * n] = raw[2 * order[n].second];
                p.items[2 * n + 1] = raw[2 * order[n].second + 1];
            }
        }
        p.ws_items_offset = align256(size_t(B) * sizeof(fa_geom));
        p.ws_bytes = p.empty ? 0 : p.ws_items_offset + size_t(p.n_items) * 2 * sizeof(int32_t);
        p.ws_table_bytes = p.ws_bytes;
    } else {
        p.n_qtiles_fixed = int32_t(ceil_div(d.Sq, p.bm));
        p.n_items = B * p.n_qtiles_fixed;
        p.ws_bytes = 0;
        if (p.dense_tiles && !p.empty && d.Skv > 0)
            p.ws_bytes = fa_dense_ws_layout(p.mask_slices, p.dense_nqt, p.dense_nkt, &p.ws_cls_offset,
                                            &p.ws_list_offset, &p.ws_bits_offset, &p.ws_perm_offset);
        if (B > 0 && p.n_qtiles_fixed > 1 && !sizes_only)
            p.reverse_qt = item_cost(0, p.n_qtiles_fixed - 1, nullptr) > item_cost(0, 0, nullptr);
        const char* xm = std::getenv("FA_XCD_MAJOR");
        p.xcd_major = ((B * d.N) % 8 == 0 && !(xm && xm[0] == '0')) ? 1 : 0;
        if (p.xcd_major && B > 0 && !sizes_only && p.kernel != FA_KERNEL_DECODE) {
            // Model one XCD's dispatch (every XCD sees the same pattern): its 32 CUs take the
            // next workgroup in launch order when free; an item costs its kv tiles plus a fixed
            // two. Pair-major order (one (batch, head) after another, heaviest q tile first) keeps
            // one pair's K/V in the XCD's L2; rank-major (the heaviest q tile of every pair, then
            // the next) balances better when a pair has few, very unequal q tiles. Take rank-major
            // when the model says it finishes more than 5% sooner (FA_XCD_ORDER=pair|rank forces).
            const int64_t ppx = B * d.N / 8;
            const int32_t nq = p.n_qtiles_fixed;
            const int slots = 32 * ((p.kernel == FA_KERNEL_PP && d.D == 128) ? 1 : 2);
            std::vector<int64_t> cost(nq);
            for (int32_t r = 0; r < nq; ++r)
                cost[r] = item_cost(0, p.reverse_qt ? nq - 1 - r : r, nullptr) + 2;
            auto makespan = [&](bool rank_major) {
                std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
                for (int i = 0; i < slots; ++i) free_at.push(0);
                int64_t end = 0;
                for (int64_t sl = 0; sl < ppx * nq; ++sl) {
                    const int32_t r = rank_major ? int32_t(sl / ppx) : int32_t(sl % nq);
                    const int64_t t = free_at.top() + cost[r];
                    free_at.pop();
                    free_at.push(t);
                    end = std::max(end, t);
                }
                return end;
            };
            // Workgroups are dispatched in launch order, so a workgroup that cannot start yet holds
            // back the ones after it: in pair-major order, where neighbouring items differ a lot in
            // cost (causal: the heaviest q tile of a pair next to its lightest), compute units
            // measured idle for 4-32 us between items. When the item costs of a pair spread
            // widely (coefficient of variation above 0.35; band masks stay near 0.2), take the
            // rank-major order, whose neighbours cost the same.
            double cs = 0.0, cs2 = 0.0;
            for (int32_t r = 0; r < nq; ++r) {
                cs += double(cost[r]);
                cs2 += double(cost[r]) * double(cost[r]);
            }
            const double mean = cs / std::max(nq, 1), var = std::max(cs2 / std::max(nq, 1) - mean * mean, 0.0);
            // Mode 1's costs come from the mask on the device; its pre-pass launches each slice's
            // q tiles most visited first, so pair-major neighbours differ as much as causal ones.
            const bool spread = nq > 1 && (p.dense_tiles || std::sqrt(var) > 0.35 * mean);
            bool rank = ppx > 1 && nq > 1 && (spread || makespan(true) * 20 < makespan(false) * 19);
            const char* xo = std::getenv("FA_XCD_ORDER");   // pair | rank (grouped) | rank1 (plain)
            if (xo && (std::strcmp(xo, "rank") == 0 || std::strcmp(xo, "rank1") == 0)) rank = true;
            if (xo && std::strcmp(xo, "pair") == 0) rank = false;
            // Rank-major runs within groups of four pairs when the XCD's pairs split that way: the
            // neighbours stay equal in cost, but an XCD works on four pairs' K/V at a time instead of
            // all of its pairs'. Same box against plain rank-major: causal_8192 equal or +0.4% with
            // 888 MB of L2 misses per launch instead of 1389; causal_2048 +2%.
            if (rank) p.xcd_major = (ppx % 4 == 0 && ppx > 4) ? 3 : 2;
            if (xo && std::strcmp(xo, "rank1") == 0) p.xcd_major = 2;
        }
    }

    if (with_tables && !sizes_only) {
        for (int64_t b = 0; b < B; ++b) {
            const int64_t nqt = ceil_div(sq[b], p.bm);
            for (int64_t qt = 0; qt < nqt; ++qt) {
                int64_t full = 0;
                p.kv_tiles_visited += item_cost(b, qt, &full);
                p.kv_tiles_full += full;
                p.kv_tiles_total += ceil_div(skv[b], p.bn);
            }
        }
    }
    *out = std::move(p);
    return FA_OK;
}

size_t fa_dense_ws_layout(int64_t slices, int64_t nqt, int64_t nkt, size_t* cls_off, size_t* list_off,
                          size_t* bits_off, size_t* perm_off) {
    const size_t tiles = size_t(slices) * size_t(nqt) * size_t(nkt);
    *cls_off = 0;
    *list_off = align256(tiles * sizeof(uint16_t));
    *bits_off = align256(*list_off + size_t(slices) * size_t(nqt) * size_t(nkt + 1) * sizeof(uint32_t));
    *perm_off = align256(*bits_off + tiles * 512 * sizeof(uint32_t));
    return align256(*perm_off + size_t(slices) * size_t(nqt) * sizeof(int32_t));
}

fa_status fa_make_plan(const fa_call& call, bool with_tables, fa_plan* plan) {
    return make_plan_impl(call, with_tables, false, plan);
}

fa_status fa_make_plan_sizes(const fa_call& call, fa_plan* plan) {
    return make_plan_impl(call, false, true, plan);
}

void fa_plan_workspace_image(const fa_plan& plan, std::vector<unsigned char>* image) {
    image->assign(plan.ws_table_bytes, 0);
    if (plan.ws_table_bytes == 0) return;
    std::memcpy(image->data(), plan.geoms.data(), plan.geoms.size() * sizeof(fa_geom));
    if (!plan.items.empty())
        std::memcpy(image->data() + plan.ws_items_offset, plan.items.data(),
                    plan.items.size() * sizeof(int32_t));
    if (!plan.dec_batch.empty())
        std::memcpy(image->data() + plan.ws_dec_batch_offset, plan.dec_batch.data(),
                    plan.dec_batch.size() * sizeof(int32_t));
}

// ---------------------------------------------------------------------------------------
// Host-only entry points of the C ABI.
// ---------------------------------------------------------------------------------------

extern "C" fa_status fa_fwd_workspace_size(const fa_dims* dims, int32_t layout,
                                           int32_t sparse_mode, const int64_t* actual_seq_qlen,
                                           const int64_t* actual_seq_kvlen, size_t* bytes) {
    if (!dims || !bytes) return FA_ERR_NULLPTR;
    fa_call c;
    c.dims = dims;
    c.layout = layout;
    c.sparse_mode = sparse_mode;
    c.actual_seq_qlen = actual_seq_qlen;
    c.actual_seq_kvlen = actual_seq_kvlen;
    fa_plan p;
    const fa_status st = fa_make_plan_sizes(c, &p);
    if (st != FA_OK) return st;
    *bytes = p.ws_bytes;
    return FA_OK;
}

extern "C" fa_status fa_fwd_mask_workspace_size(const fa_dims* dims, int32_t layout,
                                                const int64_t* mask_bcast, size_t* bytes) {
    if (!dims || !bytes) return FA_ERR_NULLPTR;
    fa_call c;
    c.dims = dims;
    c.layout = layout;
    c.sparse_mode = 1;
    c.mask_bcast = mask_bcast;
    fa_plan p;
    const fa_status st = fa_make_plan_sizes(c, &p);
    if (st != FA_OK) return st;
    *bytes = p.ws_bytes;
    return FA_OK;
}

extern "C" fa_status fa_fwd_paged_workspace_size(const fa_dims* dims, int32_t layout,
                                                 int32_t sparse_mode, const int64_t* actual_seq_qlen,
                                                 const int64_t* actual_seq_kvlen,
                                                 const fa_paged_kv* paged, size_t* bytes) {
    if (!dims || !bytes || !paged) return FA_ERR_NULLPTR;
    fa_call c;
    c.dims = dims;
    c.layout = layout;
    c.sparse_mode = sparse_mode;
    c.actual_seq_qlen = actual_seq_qlen;
    c.actual_seq_kvlen = actual_seq_kvlen;
    c.paged = paged;
    fa_plan p;
    const fa_status st = fa_make_plan_sizes(c, &p);
    if (st != FA_OK) return st;
    *bytes = p.ws_bytes;
    return FA_OK;
}

extern "C" fa_status fa_tile_shape(const fa_dims* dims, int32_t layout,
                                   const int64_t* actual_seq_qlen,
                                   const int64_t* actual_seq_kvlen, int32_t* block_m,
                                   int32_t* block_n, int64_t* n_qtiles_total,
                                   int64_t* n_kvtiles_max) {
    if (!dims || !block_m || !block_n || !n_qtiles_total || !n_kvtiles_max) return FA_ERR_NULLPTR;
    fa_call c;
    c.dims = dims;
    c.layout = layout;
    c.sparse_mode = 3;
    c.actual_seq_qlen = actual_seq_qlen;
    c.actual_seq_kvlen = actual_seq_kvlen;
    fa_plan p;
    const fa_status st = fa_make_plan_sizes(c, &p);
    if (st != FA_OK) return st;
    *block_m = p.bm;
    *block_n = p.bn;
    *n_qtiles_total = p.n_qtiles_total;
    *n_kvtiles_max = p.n_kvtiles_max;
    return FA_OK;
}

extern "C" fa_status fa_plan_stats_get(const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                                       int64_t pre_tokens, int64_t next_tokens,
                                       const int64_t* actual_seq_qlen,
                                       const int64_t* actual_seq_kvlen, const int64_t* prefix,
                                       int32_t has_alibi, int32_t has_mask, float scale,
                                       fa_plan_stats* out) {
    if (!dims || !out) return FA_ERR_NULLPTR;
    fa_call c;
    c.dims = dims;
    c.layout = layout;
    c.sparse_mode = sparse_mode;
    c.pre_tokens = pre_tokens;
    c.next_tokens = next_tokens;
    c.actual_seq_qlen = actual_seq_qlen;
    c.actual_seq_kvlen = actual_seq_kvlen;
    c.prefix = prefix;
    c.has_alibi = has_alibi != 0;
    c.has_mask = has_mask != 0;
    c.scale = scale;
    fa_plan p;
    const fa_status st = fa_make_plan(c, true, &p);
    if (st != FA_OK) return st;
    out->kernel = p.kernel;
    out->block_m = p.bm;
    out->block_n = p.bn;
    out->work_items = p.n_items;
    out->kv_tiles_visited = p.kv_tiles_visited;
    out->kv_tiles_full = p.kv_tiles_full;
    out->kv_tiles_total = p.kv_tiles_total;
    out->workspace_bytes = p.ws_bytes;
    out->launch_order = p.kernel == FA_KERNEL_DECODE ? 0 : (p.table ? 4 : p.xcd_major);
    out->edge_skip = p.edge_skip ? 1 : 0;
    return FA_OK;
}

extern "C" const char* fa_status_str(fa_status status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_NULLPTR: return "FA_ERR_NULLPTR: a required pointer is NULL";
        case FA_ERR_PARAM_INVALID: return "FA_ERR_PARAM_INVALID: an argument breaks a stated rule";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: valid but not built";
        case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace too small";
        default: return "unknown fa_status";
    }
}
