// fa_plan.h - host-side validation and planning for fa_fwd / fa_mask_probe.
//
// Pure C++17, no HIP include, so it can be built and tested on a machine without a GPU.
#ifndef FA_PLAN_H_
#define FA_PLAN_H_

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/fa.h"
#include "fa_mask.h"

// Everything fa_fwd receives that the host can look at (device pointers only as flags).
struct fa_call {
    const fa_dims* dims = nullptr;
    int32_t layout = 0;
    int32_t sparse_mode = 0;
    int64_t pre_tokens = 0, next_tokens = 0;
    const int64_t* actual_seq_qlen = nullptr;
    const int64_t* actual_seq_kvlen = nullptr;
    const int64_t* prefix = nullptr;
    bool has_alibi = false;
    int32_t alibi_mode = FA_ALIBI_RIGHT;
    bool has_mask = false;
    const int64_t* mask_bcast = nullptr;
    float scale = 1.0f;
    bool check_scale = true;
    const fa_paged_kv* paged = nullptr;   // K / V read from paged caches (fa_fwd_paged)
};

// Kernel families and their tiles.
enum { FA_KERNEL_GENERIC = 0, FA_KERNEL_PP = 1, FA_KERNEL_MFMA32 = 2, FA_KERNEL_DECODE = 3 };
constexpr int FA_PP_BM = 256;       // 8 waves x 32 rows, two groups in ping-pong
constexpr int FA_PP_BN = 64;
constexpr int FA_MFMA32_BM = 128;   // 4 waves x 32 rows
constexpr int FA_MFMA32_BN = 64;
constexpr int FA_GEN_BM = 64;
constexpr int FA_GEN_BN = 16;
// Split-KV decode (every sequence has at most FA_DEC_ROWS query rows): one workgroup per
// (batch, kv split, head), 64-key tiles. The planner's launch model, in kv tiles: a workgroup
// costs its tiles plus FA_DEC_WG_COST (its fixed start-up and combine, measured at about
// three tiles' time), FA_DEC_SLOTS workgroups run at once with D = 128 (twice that with
// D = 64: the kernel's LDS allows one or two per CU), the merge kernel costs
// FA_DEC_MERGE_COST; splits hold at least FA_DEC_MIN_TILES tiles, at most
// FA_DEC_MAX_SPLITS per sequence.
constexpr int FA_DEC_ROWS = 16;
constexpr int FA_DEC_BN = 64;
constexpr int FA_DEC_WG_COST = 3;
constexpr int FA_DEC_MERGE_COST = 3;
constexpr int FA_DEC_SLOTS = 256;
constexpr int FA_DEC_MIN_TILES = 8;
constexpr int FA_DEC_MAX_SPLITS = 64;
// Paged K / V in the ping-pong kernel: pages of a power-of-two size >= 64 (a 64-key tile never
// straddles two pages) and at most this many pages per sequence.
constexpr int FA_PP_MAX_PAGES = 2048;

struct fa_plan {
    int32_t kernel = FA_KERNEL_GENERIC;
    int32_t bm = 0, bn = 0;
    int32_t B = 0, N = 0, D = 0;
    int64_t rows_total = 0;     // query rows over all batches (per head)
    int64_t kv_total = 0;       // key rows over all batches (per head)
    bool empty = false;         // nothing to compute or write
    // Geometry: one entry per batch; geom0 when every batch shares it.
    std::vector<fa_geom> geoms;
    fa_geom geom0{};
    bool table = false;         // per-batch geometry + work-item list travel in the workspace
    std::vector<int32_t> items; // (b, q tile) pairs in launch order (table mode)
    int64_t n_items = 0;        // work items per head
    int32_t n_qtiles_fixed = 0; // q tiles per batch (fixed-length mode)
    int32_t reverse_qt = 0;     // fixed-length mode: launch the last q tiles first
    int32_t xcd_major = 0;      // fixed-length mode, B * N % 8 == 0: XCD-major launch order,
                                // 1 = pair-major, 2 = rank-major, 3 = rank-major in groups of
                                // four pairs (see fa_decode_item)
    int64_t n_qtiles_total = 0; // batch-major q tiles over all batches
    int64_t n_kvtiles_max = 0;
    size_t ws_bytes = 0;
    size_t ws_table_bytes = 0;  // leading part of the workspace the host uploads (geometry, items)
    size_t ws_items_offset = 0;
    // Split-KV decode. n_items counts (batch, split) entries; fixed-length mode splits every
    // batch n_split ways (entry e = b * n_split + split), table mode lists the entries in
    // `items` (longest first) and per batch (first partial slot, splits) in `dec_batch`.
    // Batches with more than one split write fp32 partial O / LSE for the merge kernel.
    int32_t n_split = 1;
    bool dec_merge = false;
    std::vector<int32_t> dec_batch;
    size_t ws_dec_batch_offset = 0;
    size_t ws_opart_offset = 0, ws_lse_offset = 0;
    // Strides in elements.
    int64_t q_bs = 0, q_hs = 0, q_rs = 0;
    int64_t kv_bs = 0, kv_hs = 0, kv_rs = 0;
    int64_t lse_bs = 0, lse_hs = 0;
    int64_t m_bs = 0, m_hs = 0, m_rs = 0;
    // Paged K / V (kv_bs is 0 and every sequence starts at key 0 of its own pages).
    bool paged = false;
    int64_t page_stride = 0;    // elements from one page to the next
    int64_t bt_stride = 0;      // block_table row length
    int32_t block_size = 0;
    int32_t log2_block_size = -1;   // -1 unless block_size is a power of two
    int32_t num_pages = 0;
    // Dense mask (sparse mode 1) on the ping-pong kernel: a pre-pass classifies every (q tile,
    // kv tile) of each mask slice and packs its mask bits; the kernel walks a per-q-tile list of
    // the tiles that hold a visible entry. Slices are the mask's own [B or 1, N or 1] entries.
    bool dense_tiles = false;
    int32_t mask_slices = 0, mask_heads = 0;    // slices = (B or 1) x (N or 1); heads = N or 1
    int32_t m_bcast_b = 0, m_bcast_h = 0;
    int32_t dense_nqt = 0, dense_nkt = 0;       // q tiles (256 rows) and kv tiles (64 keys) per slice
    size_t ws_cls_offset = 0, ws_list_offset = 0, ws_bits_offset = 0, ws_perm_offset = 0;
    // Statistics (per head).
    int64_t kv_tiles_visited = 0, kv_tiles_full = 0, kv_tiles_total = 0;
    // Ping-pong kernel variant in which a wave skips the softmax of a kv tile none of its rows
    // sees (band edges, causal diagonals): chosen where such tiles are a large share of the
    // work items, see fa_make_plan.
    bool edge_skip = false;
};

// Validates `call` against the pages' rules and this ABI; on success fills `plan`.
// with_tables: also build the work-item list and tile statistics.
fa_status fa_make_plan(const fa_call& call, bool with_tables, fa_plan* plan);

// Size-only planning for the workspace-size query: checks sizes and layout, not the
// mode-specific arguments (pre/next, prefix, mask), and builds no work-item list. In mode 1
// the mask is taken as unbroadcast unless call.mask_bcast is given.
fa_status fa_make_plan_sizes(const fa_call& call, fa_plan* plan);

// Bytes of the mode-1 pre-pass tables for `slices` mask slices of nqt x nkt tiles, and their
// offsets from the start of the workspace: the tile classes (uint16), the per-q-tile lists
// (count, then one uint32 entry per visited tile), the packed mask bits (512 uint32 per tile)
// and each slice's q tiles in launch order (int32, most visited tiles first).
size_t fa_dense_ws_layout(int64_t slices, int64_t nqt, int64_t nkt, size_t* cls_off, size_t* list_off,
                          size_t* bits_off, size_t* perm_off);

// Serialises the per-batch geometry and work items into a host image of the leading
// ws_table_bytes of the workspace.
void fa_plan_workspace_image(const fa_plan& plan, std::vector<unsigned char>* image);

#endif  // FA_PLAN_H_
