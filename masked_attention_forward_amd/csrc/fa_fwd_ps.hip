// fa_fwd_ps.hip - persistent forward kernel for gfx950: one workgroup per CU walks a list of
// work items and streams their K/V tiles back to back.
//
// The arithmetic is the ping-pong kernel's (fa_kernels.hip, fa_fwd_pp): FlashAttention-style
// tiling with an online softmax ("Ý Tưởng Tiling & Online Softmax Trong FlashAttention",
// knowledge goals), the mask of "sparseMode介绍" turned into per-row column intervals
// (fa_mask.h), and the alibi bias of "压缩mask". A workgroup of 512 threads owns 256 query rows
// of an item; groups A (waves 0-3) and B (waves 4-7) alternate a softmax phase (VALU) with a
// matrix phase (O^T += V^T P^T, then S^T = K Q^T of the next tile) one phase apart, so each
// SIMD runs one wave's MFMAs under its partner's exponentials.
//
// What is persistent: the positions p = 0, 1, ... of the tile stream run over every kv tile of
// every item of the workgroup's list, in order. The loads of the four-set LDS ring run three
// phases ahead of the stream, so the next item's first K/V tiles arrive while the current item
// finishes; the matrix phase after an item's last tile computes S^T of the next item's first
// tile, with that item's Q loaded into registers during the softmax phase before it; and the
// softmax phase of an item's first tile first writes out the previous item (O / l through a
// dedicated LDS staging area, and the LSE). So no phase drains between items, no workgroup is
// launched per item, and the only idle phase of a workgroup is its last one.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_fwd_common.h"

namespace {

constexpr int PS_THREADS = 512;

// One item of a workgroup's list (all wave-uniform). Only a few of its fields stay live across
// the stream; the rest is recomputed from the list position when needed.
struct ps_item {
    int n;          // position in the workgroup's list
    int b, h, qt;
    int i0;         // first query row
    int kbeg, nt;   // kv tiles [kbeg, kbeg + nt)
    int kv_lim;     // keys at and past this are never read
    fa_geom g;
};

// A K/V tile of the stream: element offset of its item's sequence in K and V (they share a
// layout), kv tile, and the item's key limit (0: an empty load).
struct ld_tile {
    int64_t off;
    int kt;
    int lim;
};

typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
typedef const __attribute__((address_space(4))) float* cfloat_ptr;

template <int D, bool IS_BF16, int AL>
__global__ __attribute__((amdgpu_flat_work_group_size(PS_THREADS, PS_THREADS),
                          amdgpu_waves_per_eu(2, 2))) void
fa_fwd_ps(const fa_kargs a, const fa_ps_args ps) {
    static_assert(D == 64 || D == 128, "MFMA path covers D = 64 and 128");
    static_assert(AL >= 0 && AL <= 2, "alibi kind: 0 none, 1 linear, 2 square root");
    constexpr bool ALIBI = AL != 0;
    using io = mfma_io<IS_BF16>;
    constexpr int BM = PP_BM, BN = PP_BN, NT = PS_THREADS;
    constexpr int KCH = D / 8;                   // 16-byte chunks per K / V row
    constexpr int KSTEPS = D / 16;               // k-steps of S^T = K Q^T
    constexpr int DBLK = D / 32;                 // 32-row blocks of O^T
    constexpr int TILE_CHUNKS = BN * KCH;        // 16-byte chunks per K or V tile
    constexpr int LOADS = TILE_CHUNKS / NT;      // direct loads per thread and tile
    constexpr int BATCH = 2 * LOADS;             // loads per thread and set (V and K)
    static_assert(LOADS >= 1 && LOADS <= 2 && TILE_CHUNKS % NT == 0, "tile shape");

    __shared__ u32x4 lds_k0[TILE_CHUNKS], lds_k1[TILE_CHUNKS], lds_k2[TILE_CHUNKS], lds_k3[TILE_CHUNKS];
    __shared__ u32x4 lds_v0[TILE_CHUNKS], lds_v1[TILE_CHUNKS], lds_v2[TILE_CHUNKS], lds_v3[TILE_CHUNKS];
    // O staging: a 32-row slot per wave of a group. The two groups write out items in different
    // phases (B one phase behind A, a barrier between), so waves w and w + 4 share slot w % 4.
    __shared__ u32x4 lds_o[4 * 32 * KCH];
    FA_POISON_LDS(lds_k0, lds_k1, lds_k2, lds_k3, lds_v0, lds_v1, lds_v2, lds_v3, lds_o);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int ln = lane & 31;
    const int wave_u = fa_uniform(wave);
    const int grp = wave_u >> 2;   // 0: group A, 1: group B (one phase behind)
    const int lrow = wave * 32 + ln;
    // The lane index as a value the compiler cannot see through: addresses of the rarely taken
    // item-boundary paths derive from it at the point of use, so they are not hoisted out of the
    // stream loop to hold vector registers for its whole length.
    auto lane_opaque = [&]() __attribute__((always_inline)) {
        int l = lane;
        asm volatile("" : "+v"(l));
        return l;
    };
    const int q_rs = int(a.q_rs), kv_rs = int(a.kv_rs);
    const float sl2 = a.scale_log2;

    // Arguments used only at item boundaries are read again from the kernel argument segment
    // there (scalar loads through a pointer the compiler cannot see through), instead of
    // holding scalar registers for the whole stream.
    typedef const __attribute__((address_space(4))) fa_kargs* ckargs_ptr;
    typedef const __attribute__((address_space(4))) fa_ps_args* cps_ptr;
    auto kseg = [&]() __attribute__((always_inline)) {
        const __attribute__((address_space(4))) char* p =
            (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(p));
        return p;
    };
    auto kargs = [&]() __attribute__((always_inline)) { return (ckargs_ptr)kseg(); };
    // The schedule argument follows the fa_kargs argument in the segment (both 8-byte aligned).
    static_assert(sizeof(fa_kargs) % 8 == 0 && alignof(fa_ps_args) <= 8, "kernel argument layout");
    auto psargs = [&]() __attribute__((always_inline)) { return (cps_ptr)(kseg() + sizeof(fa_kargs)); };
    auto fdiv = [](uint32_t n, uint32_t mul, uint32_t shr) __attribute__((always_inline)) -> int {
        return int((mul ? __umulhi(n, mul) : n) >> shr);
    };

    // ---------------------------------------------------------------------------------------
    // The workgroup's list (see fa_ps_args). Table reads go through the constant address space:
    // scalar loads, which no phase has to wait for behind the vector loads in flight.
    // ---------------------------------------------------------------------------------------
    auto item_at = [&](int n, ps_item& it) __attribute__((always_inline)) -> bool {
        const cps_ptr sp = psargs();
        fa_ps_args P;   // adjacent fields: one batch of scalar loads
        P.W = sp->W;
        P.xcd = sp->xcd;
        P.n_list = sp->n_list;
        P.nq = sp->nq;
        P.nq_mul = sp->nq_mul;
        P.nq_shr = sp->nq_shr;
        P.n_mul = sp->n_mul;
        P.n_shr = sp->n_shr;
        P.N = sp->N;
        P.reverse_qt = sp->reverse_qt;
        P.table = sp->table;
        const int w = blockIdx.x;
        const int x = P.xcd ? (w & 7) : 0;
        const int j = P.xcd ? (w >> 3) : w;
        const int pos = (n & 1) ? P.W - 1 - j : j;
        const int idx = n * P.W + pos;
        if (idx >= P.n_list) return false;
        int b, h, qt;
        const ckargs_ptr ka = kargs();
        if (P.table) {
            const int e = fdiv(uint32_t(idx), P.n_mul, P.n_shr);
            h = idx - e * P.N;
            b = ((cint_ptr)ka->items)[2 * e];
            qt = ((cint_ptr)ka->items)[2 * e + 1];
        } else {
            const int pl = fdiv(uint32_t(idx), P.nq_mul, P.nq_shr);
            const int r = idx - pl * P.nq;
            const int pair = P.xcd ? pl * 8 + x : pl;
            b = fdiv(uint32_t(pair), P.n_mul, P.n_shr);
            h = pair - b * P.N;
            qt = P.reverse_qt ? P.nq - 1 - r : r;
        }
        it.n = n;
        it.b = b;
        it.h = h;
        it.qt = qt;
        if (P.table) {
            cint_ptr gp = (cint_ptr)(ka->geoms + b);
            it.g.q_start = gp[0];
            it.g.kv_start = gp[1];
            it.g.sq = gp[2];
            it.g.skv = gp[3];
            it.g.a = gp[4];
            it.g.c = gp[5];
            it.g.f = gp[6];
            it.g.pad = 0;
        } else {
            it.g.q_start = ka->geom0.q_start;
            it.g.kv_start = ka->geom0.kv_start;
            it.g.sq = ka->geom0.sq;
            it.g.skv = ka->geom0.skv;
            it.g.a = ka->geom0.a;
            it.g.c = ka->geom0.c;
            it.g.f = ka->geom0.f;
            it.g.pad = 0;
        }
        it.i0 = qt * BM;
        const fa_kv_range kr = fa_tile_kv_range(it.g, it.i0, min(it.i0 + BM, it.g.sq) - 1, BN);
        it.kbeg = kr.begin;
        it.nt = kr.end - kr.begin;
        it.kv_lim = min(kr.end * BN, it.g.skv);
        return true;
    };

    // Items without a visible key (no kv tile) are written here and leave the tile stream:
    // O = 0 and LSE = -inf for this wave's rows.
    auto write_empty = [&](const ps_item& it) __attribute__((always_inline)) {
        const int lo = lane_opaque();
        const int wrow0 = it.i0 + wave_u * 32;
        const int row = wrow0 + (lo & 31);
        const ckargs_ptr ka = kargs();
        if (row < it.g.sq && lo < 32) ka->lse[it.b * ka->lse_bs + it.h * ka->lse_hs + it.g.q_start + row] = -INFINITY;
        uint16_t* obase = static_cast<uint16_t*>(ka->o) + it.b * ka->q_bs + it.h * ka->q_hs +
                          (int64_t(it.g.q_start) + wrow0) * q_rs;
        constexpr int RPI = 64 / KCH;
        const int c = lo % KCH;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int r = i * RPI + lo / KCH;
            if (wrow0 + r < it.g.sq)
                __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, reinterpret_cast<u32x4*>(obase + int64_t(r) * q_rs + 8 * c));
        }
    };

    // First item with a kv tile at list position n or later (-1: none); with `zeros`, the empty
    // items passed on the way are written out.
    auto find_next = [&](int n, bool zeros, ps_item& it) __attribute__((always_inline)) -> int {
        for (;; ++n) {
            if (!item_at(n, it)) return -1;
            if (it.nt > 0) return n;
            if (zeros) write_empty(it);
        }
    };

    // ---------------------------------------------------------------------------------------
    // Per-item state of the softmax stage: list position, kv tiles, and this wave's range of
    // tile starts j0 that need no per-element masking (fa_tile_full over the wave's rows).
    // ---------------------------------------------------------------------------------------
    int n_cur = 0, c_kbeg = 0, c_nt = 0, t_cur = 0, n_nxt = -1, full_lo = 0, full_hi = -1;
    int row_lo = 0, row_hi = -1, rowb = 0;   // per lane; rowb: the row plus the alibi bias origin
    float slope2 = 0.f;
    auto enter_item = [&](const ps_item& it) __attribute__((always_inline)) {
        n_cur = it.n;
        c_kbeg = it.kbeg;
        c_nt = it.nt;
        t_cur = 0;
        const int row = it.i0 + lrow;
        row_lo = fa_row_lo(it.g, row);
        row_hi = fa_row_hi(it.g, row);
        const int w0 = it.i0 + wave_u * 32;
        const int w1 = min(w0 + 31, it.g.sq - 1);
        // fa_tile_full(g, w0, w1, j0, BN) <=> full_lo <= j0 <= full_hi.
        full_lo = w1 + it.g.a;
        full_hi = min(max(w0 + it.g.c, it.g.f) - BN + 1, it.g.skv - BN);
        const int off = it.g.skv - it.g.sq;
        const ckargs_ptr ka = kargs();
        rowb = row + (AL == 1 && ka->alibi_left ? 0 : off);
        if (ALIBI) slope2 = ((cfloat_ptr)ka->slopes)[it.h] * kLog2e;
    };

    // The next item's Q goes HBM -> LDS into this wave's staging slot with direct loads
    // (physical 16-byte chunk P of the slot holds row P / KCH, logical chunk (P % KCH) ^ (row %
    // KCH)), and from there into registers once it has landed. No register is a load's target, so
    // the compiler adds no wait for it anywhere; the waits are explicit where Q is read.
    u32x4 qop[KSTEPS];
    u32x4* const q_slot = lds_o + (wave_u & 3) * 32 * KCH;
    auto load_q = [&](const ps_item& it) __attribute__((always_inline)) {
        const ckargs_ptr ka = kargs();
        const int r0 = it.i0 + wave_u * 32;
        const int nrows = min(32, it.g.sq - r0);
        const uint16_t* qp = static_cast<const uint16_t*>(ka->q) + it.b * ka->q_bs + it.h * ka->q_hs +
                             (int64_t(it.g.q_start) + r0) * q_rs;
        const __amdgpu_buffer_rsrc_t rq = fa_rsrc(qp, nrows > 0 ? ((nrows - 1) * q_rs + D) * 2 : 0);
        const int lo = lane_opaque();
#pragma unroll
        for (int i = 0; i < KCH / 2; ++i) {
            const int P = i * 64 + lo;
            const int r = P / KCH;
            const int c = (P % KCH) ^ (r & (KCH - 1));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_t*)(q_slot + i * 64), 16, (r * q_rs + 8 * c) * 2, 0,
                                                     0, 0);
        }
    };
    // The first item's Q straight into registers: waves w and w + 4 share a staging slot, and the
    // prologue waits for every load anyway.
    auto load_q_regs = [&](const ps_item& it) __attribute__((always_inline)) {
        const ckargs_ptr ka = kargs();
        const uint16_t* qp = static_cast<const uint16_t*>(ka->q) + it.b * ka->q_bs + it.h * ka->q_hs +
                             (int64_t(it.g.q_start) + it.i0) * q_rs;
        const __amdgpu_buffer_rsrc_t rq = fa_rsrc(qp, ((min(it.g.sq - it.i0, BM) - 1) * q_rs + D) * 2);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) qop[t] = fa_bload(rq, (lrow * q_rs + 16 * t + 8 * hl) * 2);
    };
    auto read_q = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            const int lo = lane_opaque();
            const int l = lo & 31;
            qop[t] = q_slot[l * KCH + ((2 * t + (lo >> 5)) ^ (l & (KCH - 1)))];
        }
    };

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x16 oacc[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) oacc[db] = f32x16{};

    // O = O / l and LSE = ln2 (m + log2 l) of item `it` (rows with nothing visible give 0 and
    // -inf), then a fresh softmax state. O goes out as whole rows: the wave stages its 32 x D
    // tile in its LDS slot and reads it back one row per KCH lanes (chunk c of row r stored at
    // c ^ (r % KCH)); its reads complete before the phase barrier, which orders them before the
    // partner group's use of the slot.
    auto write_out = [&](int n) __attribute__((always_inline)) {
        ps_item it;
        item_at(n, it);
        const int lo = lane_opaque();
        const int l32 = lo & 31, h2 = lo >> 5;
        const int wrow0 = it.i0 + wave_u * 32;
        const int row = wrow0 + l32;
        const float l_tot = pair_sum(l_run);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const ckargs_ptr ka = kargs();
        if (row < it.g.sq && h2 == 0)
            ka->lse[it.b * ka->lse_bs + it.h * ka->lse_hs + it.g.q_start + row] =
                l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
        char* stage = reinterpret_cast<char*>(lds_o + (wave_u & 3) * 32 * KCH);
        constexpr int ROWB = KCH * 16;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int c = 4 * db + gi;
                const u32x2 w = {io::pack(oacc[db][4 * gi + 0] * inv, oacc[db][4 * gi + 1] * inv),
                                 io::pack(oacc[db][4 * gi + 2] * inv, oacc[db][4 * gi + 3] * inv)};
                *reinterpret_cast<u32x2*>(stage + l32 * ROWB + (c ^ (l32 & (KCH - 1))) * 16 + 8 * h2) = w;
            }
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        uint16_t* obase = static_cast<uint16_t*>(ka->o) + it.b * ka->q_bs + it.h * ka->q_hs +
                          (int64_t(it.g.q_start) + wrow0) * q_rs;
        constexpr int RPI = 64 / KCH;
        const int c = lo % KCH;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int r = i * RPI + lo / KCH;
            const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * ROWB + (c ^ (r & (KCH - 1))) * 16);
            if (wrow0 + r < it.g.sq)
                __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(obase + int64_t(r) * q_rs + 8 * c));
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int db = 0; db < DBLK; ++db) oacc[db] = f32x16{};
        m_run = -INFINITY;
        l_run = 0.f;
    };

    // ---------------------------------------------------------------------------------------
    // The loader: K/V tiles of the stream, in order. Its cursor is the next K tile; a V tile is
    // loaded one iteration after the K tile of the same position. Descriptors of the coming
    // matrix phase's loads are prepared in the softmax phase (scalar work and branches there),
    // so the matrix phase only issues them.
    // ---------------------------------------------------------------------------------------
    int n_ld = -1, t_ld = 0, l_kbeg = 0, l_nt = 0, l_lim = 0;
    int64_t l_off = 0;
    auto ld_enter = [&](const ps_item& it) __attribute__((always_inline)) {
        n_ld = it.n;
        t_ld = 0;
        l_kbeg = it.kbeg;
        l_nt = it.nt;
        l_lim = it.kv_lim;
        const ckargs_ptr ka = kargs();
        l_off = int64_t(it.b) * ka->kv_bs + int64_t(it.h) * ka->kv_hs + int64_t(it.g.kv_start) * kv_rs;
    };
    // The cursor's tile, then the cursor one tile on.
    auto ld_take = [&]() __attribute__((always_inline)) -> ld_tile {
        ld_tile r{l_off, 0, 0};
        if (__builtin_expect(n_ld >= 0, 1)) {
            r.kt = l_kbeg + t_ld;
            r.lim = l_lim;
            if (__builtin_expect(++t_ld == l_nt, 0)) {
                ps_item it;
                const int n = find_next(n_ld + 1, false, it);
                n_ld = -1;
                if (n >= 0) ld_enter(it);
            }
        }
        return r;
    };

    // HBM -> LDS for this thread's share of one K or V tile (physical chunk 64 (LOADS wave + p) +
    // lane, i.e. row P / KCH, logical chunk un-swizzled); rows at and past lim read as zeros.
    auto dl_offset = [&](int p) __attribute__((always_inline)) {
        const int P = (wave * LOADS + p) * 64 + lane;
        const int j = P / KCH;
        return (j * kv_rs + fa_swz<KCH>(j, P % KCH) * 8) * 2;
    };
    const int dl0 = dl_offset(0), dl1 = LOADS > 1 ? dl_offset(1) : 0;
    auto dload = [&](const void* tensor, const ld_tile& tl, u32x4* dst) __attribute__((always_inline)) {
        const uint16_t* base = static_cast<const uint16_t*>(tensor) + tl.off;
        const int kt = tl.kt, lim = tl.lim;
        const int j0 = kt * BN;
        const int rows = min(BN, lim - j0);
        const __amdgpu_buffer_rsrc_t r =
            fa_rsrc(base + int64_t(j0) * kv_rs, rows > 0 ? ((rows - 1) * kv_rs + D) * 2 : 0);
#pragma unroll
        for (int p = 0; p < LOADS; ++p)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + (wave_u * LOADS + p) * 64), 16,
                                                     p == 0 ? dl0 : dl1, 0, 0, 0);
    };

    const int src = lane & 15;
    const int dlo = 16 * ((lane >> 4) & 1) + 4 * (src & 3);
    int v_off[2][DBLK];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        const int j = 8 * h2 + 4 * hl + (src >> 2);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const int d0 = 32 * db + dlo;
            v_off[h2][db] = (j * KCH + fa_swz<KCH>(j, d0 >> 3)) * 16 + (d0 & 7) * 2;
        }
    }
    int k_off[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) k_off[t] = ln * KCH + fa_swz<KCH>(ln, 2 * t + hl);

    f32x16 sacc[2];   // S^T of the tile waiting for its softmax
    u32x4 pop[4];     // P^T of the tile waiting for its PV product

    auto qk = [&](const u32x4* kb) __attribute__((always_inline)) {
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const u32x4 kop = kb[k_off[t] + 32 * jb * KCH];
                sacc[jb] = io::mma(kop, qop[t], sacc[jb]);
            }
        }
    };

    // Softmax of tile t_cur of the current item: mask, scale (+ alibi), online update, P^T
    // packed for the PV product; the O^T rescale happens here too (no MFMA of this wave is
    // using the accumulators).
    auto softmax = [&]() __attribute__((always_inline)) {
        const int j0 = (c_kbeg + t_cur) * BN;
        const bool full = j0 >= full_lo && j0 <= full_hi;
        if (!full) {
            const int lo_rel = row_lo - j0 - 4 * hl;
            const int hi_rel = row_hi - j0 - 4 * hl;
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const int r = e & 15;
                const int kc = 32 * (e >> 4) + 8 * (r >> 2) + (r & 3);
                sacc[e >> 4][r] = (kc >= lo_rel && kc <= hi_rel) ? sacc[e >> 4][r] : -INFINITY;
            }
        }
        float s[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) s[e] = sacc[e >> 4][e & 15];
        if (AL == 1) {
            const float base = slope2 * float(j0 + 4 * hl - rowb);
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const int r = e & 15;
                const int kc = 32 * (e >> 4) + 8 * (r >> 2) + (r & 3);
                s[e] = fmaf(s[e], sl2, fmaf(slope2, float(kc), base));
            }
        } else if (AL == 2) {
            // Square-root bias: -slope sign(d) sqrt(|d|), d = i + (Skv - Sq) - j (v_sqrt_f32,
            // within 1 ulp: d is an integer below 2^24).
            const float dbase = float(rowb - j0 - 4 * hl);
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const int r = e & 15;
                const int kc = 32 * (e >> 4) + 8 * (r >> 2) + (r & 3);
                const float dd = dbase - float(kc);
                s[e] = fmaf(s[e], sl2, -slope2 * copysignf(__builtin_amdgcn_sqrtf(fabsf(dd)), dd));
            }
        }
        // p = 2^(s - m) for the maximum m in use; returns this lane's sum of the 32 values.
        float p[32];
        auto expo = [&](float m_use) __attribute__((always_inline)) {
            float l4[4];
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                p[e] = ALIBI ? __builtin_amdgcn_exp2f(s[e] - m_use) : __builtin_amdgcn_exp2f(fmaf(s[e], sl2, -m_use));
                l4[e & 3] = e < 4 ? p[e] : l4[e & 3] + p[e];
            }
            return (l4[0] + l4[1]) + (l4[2] + l4[3]);
        };
        // As in fa_fwd_pp: once the row has a maximum, exponentiate against it as it stands while
        // every lane's sum of the tile's 32 values stays at most 2^15 (so every p does, within
        // fp16's range); otherwise
        // the exact update (tile maximum; rescale when it grows by more than 2^8). This kernel
        // walks tiles upwards, and an alibi bias then raises the maximum tile by tile: alibi
        // kernels always take the exact update.
        bool exact = ALIBI || __any(m_run == -INFINITY);
        float lsum = 0.f;
        if (!exact) {
            lsum = expo(m_run);
            exact = __any(!(lsum <= 32768.f));
        }
        float alpha = 1.f;
        bool need = false;
        if (exact) {
            float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int e = 0; e < 32; ++e) m4[e & 3] = fmaxf(m4[e & 3], s[e]);
            float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
            if (!ALIBI) mx *= sl2;
            mx = pair_max(mx);
            need = mx > m_run + 8.f;
            alpha = need ? exp2f(m_run - mx) : 1.f;
            m_run = need ? mx : m_run;
            lsum = expo(m_run == -INFINITY ? 0.f : m_run);
        }
        l_run = fmaf(l_run, alpha, lsum);
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int base = 16 * (t4 >> 1) + 8 * (t4 & 1);
            pop[t4] = u32x4{io::pack(p[base + 0], p[base + 1]), io::pack(p[base + 2], p[base + 3]),
                            io::pack(p[base + 4], p[base + 5]), io::pack(p[base + 6], p[base + 7])};
        }
        if (__any(need)) {
#pragma unroll
            for (int db = 0; db < DBLK; ++db) oacc[db] *= alpha;
        }
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) asm volatile("" : : "v"(pop[t4]));
        asm volatile("" : : "v"(l_run));
    };

    constexpr int NPRE = DBLK;
    u32x4 vpre[NPRE];
    auto vread = [&](const char* vbase, int t, int db) __attribute__((always_inline)) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vbase + v_off[0][db] + t * 16 * KCH * 16));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vbase + v_off[1][db] + t * 16 * KCH * 16));
        return u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                     __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
    };
    auto prefetch = [&](const u32x4* vb) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < NPRE; ++db) vpre[db] = vread(reinterpret_cast<const char*>(vb), 0, db);
    };
    // O^T += V^T P^T from V buffer vb, then S^T of the next stream position from K buffer kb; the
    // tile loads go into the gaps of the first MFMAs (fa_fwd_pp's schedule).
    auto matmul = [&](const u32x4* kb, const u32x4* vb, auto&& between) __attribute__((always_inline)) {
        const char* vbase = reinterpret_cast<const char*>(vb);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
                oacc[db] = io::mma(t == 0 ? vpre[db] : vread(vbase, t, db), pop[t], oacc[db]);
        between();
        qk(kb);
        constexpr int NPV = 4 * DBLK, NQK = 2 * KSTEPS;
        constexpr int NDMA = 2 * LOADS;
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < NPV + NQK; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (i < 16) __builtin_amdgcn_sched_group_barrier(0x004, 4, 0);
#pragma unroll
            for (int p = 0; p < NDMA; ++p)
                if (i == 5 + 6 * (p / LOADS) + p % LOADS) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        }
    };

    ld_tile lv{0, 0, 0};   // the last K load: this position's V comes next

    // One stream position t: softmax phase, then matrix phase. Set u = {V(u), K(u+1)} lives in
    // buffer u % 4; both groups load set t + 3 during MM(t), into the buffer of set t - 1, and
    // wait at the end of MM(t) until only that batch is in flight (fa_fwd_pp's ring).
    auto iter = [&](auto s_tag) __attribute__((always_inline)) {
        constexpr int S = decltype(s_tag)::value;   // t % 4
        constexpr int F = (S + 3) % 4;
        const u32x4* k_cur = S == 0 ? lds_k0 : (S == 1 ? lds_k1 : (S == 2 ? lds_k2 : lds_k3));
        const u32x4* v_cur = S == 0 ? lds_v0 : (S == 1 ? lds_v1 : (S == 2 ? lds_v2 : lds_v3));
        u32x4* k_fill = F == 0 ? lds_k0 : (F == 1 ? lds_k1 : (F == 2 ? lds_k2 : lds_k3));
        u32x4* v_fill = F == 0 ? lds_v0 : (F == 1 ? lds_v1 : (F == 2 ? lds_v2 : lds_v3));
        // A new item begins: write out the finished one, take the next.
        if (__builtin_expect(t_cur == c_nt, 0)) {
            write_out(n_cur);
            ps_item it;
            item_at(n_nxt, it);
            enter_item(it);
        }
        // The item's last tile: the next item's Q for the coming S^T (its first tile) arrives
        // under this softmax and goes into registers after it.
        const bool last = t_cur == c_nt - 1;
        if (__builtin_expect(last, 0)) {
            ps_item nx;
            n_nxt = find_next(n_cur + 1, true, nx);
            if (n_nxt >= 0) load_q(nx);
        }
        softmax();
        if (__builtin_expect(last && n_nxt >= 0, 0)) {
            __builtin_amdgcn_s_waitcnt(fa_vmcnt(0));
            asm volatile("" ::: "memory");
            read_q();
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): qop is in registers
        }
        ++t_cur;
        // This iteration's loads: V of the last K load's position, K of the cursor.
        const ld_tile lvv = lv;
        const ld_tile lkk = ld_take();
        lv = lkk;
        asm volatile("" : : "s"(lvv.kt), "s"(lkk.kt), "s"(lvv.lim), "s"(lkk.lim), "s"(lvv.off), "s"(lkk.off));
        prefetch(v_cur);
        fa_lds_barrier_pending<2 * NPRE>();
        __builtin_amdgcn_s_setprio(1);
        matmul(k_cur, v_cur, [&]() __attribute__((always_inline)) {
            dload(a.v, lvv, v_fill);
            dload(a.k, lkk, k_fill);
        });
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_s_waitcnt(fa_vmcnt(BATCH));
        fa_lds_barrier();
    };

    // Stream length: the kv tiles of every item of the list (empty items are written here).
    int n_first;
    {
        ps_item it;
        n_first = find_next(0, true, it);
    }
    int P = 0;
    {
        ps_item it;
        for (int n = n_first; n >= 0; n = find_next(n + 1, false, it)) {
            item_at(n, it);
            P += it.nt;
        }
    }

    if (P > 0) {
        {
            ps_item it;
            item_at(n_first, it);
            enter_item(it);
            load_q_regs(it);
            ld_enter(it);
        }
        // K(0) goes into buffer 3's K half; sets 0, 1, 2 into buffers 0, 1, 2.
        const ld_tile k0 = ld_take();
        dload(a.k, k0, lds_k3);
        dload(a.v, k0, lds_v0);
        const ld_tile k1 = ld_take();
        dload(a.k, k1, lds_k0);
        dload(a.v, k1, lds_v1);
        const ld_tile k2 = ld_take();
        dload(a.k, k2, lds_k1);
        dload(a.v, k2, lds_v2);
        const ld_tile k3 = ld_take();
        dload(a.k, k3, lds_k2);
        lv = k3;
        __builtin_amdgcn_s_waitcnt(0);
        fa_lds_barrier();
        if (grp == 0) {
            qk(lds_k3);
            fa_lds_barrier();
        } else {
            fa_lds_barrier();
            qk(lds_k3);
            fa_lds_barrier();
        }
        using s0 = std::integral_constant<int, 0>;
        using s1 = std::integral_constant<int, 1>;
        using s2 = std::integral_constant<int, 2>;
        using s3 = std::integral_constant<int, 3>;
        int t = 0;
        for (; t + 4 <= P; t += 4) {
            iter(s0{});
            iter(s1{});
            iter(s2{});
            iter(s3{});
        }
        if (t < P) {
            iter(s0{});
            if (t + 1 < P) {
                iter(s1{});
                if (t + 2 < P) iter(s2{});
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the loop
        write_out(n_cur);
        ps_item it;
        find_next(n_cur + 1, true, it);   // empty items after the last one with tiles
        // Group A ran one phase ahead: its last barrier matches B's final matrix phase.
        if (grp == 0) fa_lds_barrier();
    }
}

template <int D, bool BF>
void launch_d(const fa_kargs& a, const fa_ps_args& ps, int al, unsigned grid, hipStream_t s) {
    const dim3 block(PS_THREADS);
    switch (al) {
        case 0: fa_fwd_ps<D, BF, 0><<<dim3(grid), block, 0, s>>>(a, ps); break;
        case 1: fa_fwd_ps<D, BF, 1><<<dim3(grid), block, 0, s>>>(a, ps); break;
        default: fa_fwd_ps<D, BF, 2><<<dim3(grid), block, 0, s>>>(a, ps); break;
    }
}

}  // namespace

void launch_fwd_ps(const fa_kargs& a, const fa_ps_args& ps, int D, bool bf16, int alibi, unsigned grid,
                   hipStream_t s) {
    if (D == 128) {
        if (bf16) launch_d<128, true>(a, ps, alibi, grid, s);
        else launch_d<128, false>(a, ps, alibi, grid, s);
    } else {
        if (bf16) launch_d<64, true>(a, ps, alibi, grid, s);
        else launch_d<64, false>(a, ps, alibi, grid, s);
    }
}
