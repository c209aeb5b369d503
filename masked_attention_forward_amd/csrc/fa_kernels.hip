// fa_kernels.hip - masked attention forward kernels for gfx950 (MI355X) and the device half
// of the C ABI (fa_fwd, fa_fwd_paged, fa_mask_probe).
//
// The method is FlashAttention-style tiling with an online softmax ("Ý Tưởng Tiling & Online
// Softmax Trong FlashAttention", knowledge goals): K/V blocks stream past a block of query
// rows that keeps a running row maximum m and running sum l, so the Sq x Skv score matrix
// never exists. The mask family is "sparseMode介绍" (sparseMode 0..8), turned into per-row
// column intervals by fa_mask.h; the alibi bias is "压缩mask"'s per-head slope times a
// right-aligned relative position.
//
// Kernels:
//  * fa_fwd_pp (default for fp16 / bf16, D in {64, 128}): 512-thread workgroups own 256 query
//    rows (8 waves x 32 rows). Two groups of four waves alternate phases at workgroup barriers:
//    while one group runs its MFMAs (O^T += V^T P^T, then S^T = K Q^T for the next tile) the
//    other runs the softmax on the VALU, and waves w and w + 4 share a SIMD, so every SIMD
//    overlaps one wave's matrix work with the other's exponentials.
//  * fa_fwd_mfma (same inputs; selected with FA_KERNEL=mfma32): 256-thread workgroups of 128
//    rows, two per CU, software-pipelined within each wave instead of across waves.
//    Both MFMA kernels compute S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16}, so each lane
//    holds one query row (and 32 of the tile's 64 keys): softmax statistics are lane-local plus
//    one exchange with lane^32, and P^T is taken straight from the S^T accumulators. K and V
//    tiles go from HBM straight into XOR-swizzled LDS with buffer loads; the V^T operand is
//    read with ds_read_b64_tr_b16 transpose reads.
//  * fa_decode_split + fa_decode_merge (every sequence has at most 16 query rows): each
//    workgroup takes one (batch, kv split, head); 16x16x32 MFMAs with the query rows as the 16
//    columns, K straight from HBM into registers, V through swizzled per-wave LDS buffers; the
//    merge combines the splits' (O, LSE). The planner sizes the splits from a launch model.
//  * fa_fwd_generic: any dtype (fp32 included), D <= 128. One thread per query row, fp32
//    throughout (P is never rounded), K/V tiles of 16 keys staged in LDS.
// All visit only kv tiles that hold a visible entry (fa_tile_kv_range) and skip per-element
// masking on tiles that are fully visible (fa_tile_full).
//
// Paged K / V (fa_fwd_paged): K and V come from the caches that fa_scatter_kv_cache fills
// ("aclnnScatterPaKvCache", layouts "Norm" and "NHSD"), key j of sequence b in page
// block_table[b][j / block_size]. The ping-pong kernel takes it when pages hold a power of two
// >= 64 keys (one page per 64-key tile: only the tile's base address changes); the generic
// kernel takes every other page size and explicit masks.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "fa_device.h"
#include "fa_fwd_common.h"
#include "fa_mask.h"
#include "fa_plan.h"

namespace {

// ------------------------------------------------------------------------------------------
// MFMA kernel
// ------------------------------------------------------------------------------------------

constexpr int MF_BM = FA_MFMA32_BM;   // 128 query rows per workgroup (4 waves x 32 rows)
constexpr int MF_BN = FA_MFMA32_BN;   // 64 keys per kv tile
constexpr int MF_THREADS = 256;

// 32 query rows per wave, two workgroups per CU (two waves per SIMD, which take turns on the
// matrix core and the VALU). K and V tiles go from HBM straight into LDS with buffer loads
// (no register staging; rows past the last needed key read as zero), double-buffered and
// prefetched one tile ahead. S^T = K Q^T puts one query row in each lane; P comes straight
// from the S^T accumulators; the V^T operand of O^T += V^T P^T is read from the row-major V
// tile with ds_read_b64_tr_b16 (lane i of each 16-lane group receives element i%4 of the
// chunks addressed by lanes i/4, 4+i/4, 8+i/4, 12+i/4), so no transpose pass is needed.
template <int D, bool IS_BF16, int AL, bool DENSE>
__global__ __attribute__((amdgpu_flat_work_group_size(MF_THREADS, MF_THREADS),
                          amdgpu_waves_per_eu(2, 2))) void
fa_fwd_mfma(const fa_kargs a) {
    static_assert(D == 64 || D == 128, "MFMA path covers D = 64 and 128");
    static_assert(AL >= 0 && AL <= 2, "alibi kind: 0 none, 1 linear, 2 square root");
    constexpr bool ALIBI = AL != 0;
    using io = mfma_io<IS_BF16>;
    constexpr int BM = MF_BM, BN = MF_BN, NT = MF_THREADS;
    constexpr int KCH = D / 8;                   // 16-byte chunks per K / V row
    constexpr int KSTEPS = D / 16;               // k-steps of S^T = K Q^T
    constexpr int DBLK = D / 32;                 // 32-row blocks of O^T
    constexpr int TILE_CHUNKS = BN * KCH;        // 16-byte chunks per K or V tile
    constexpr int LOADS = TILE_CHUNKS / NT;      // direct loads per thread and tile
    static_assert(LOADS >= 1 && TILE_CHUNKS % NT == 0, "tile shape");

    // Two separate buffers per operand (not one array indexed by parity) so the compiler can
    // see that the prefetch DMA into one buffer never overlaps reads of the other and does not
    // wait for it before those reads.
    __shared__ u32x4 lds_k0[TILE_CHUNKS], lds_k1[TILE_CHUNKS];
    __shared__ u32x4 lds_v0[TILE_CHUNKS], lds_v1[TILE_CHUNKS];
    FA_POISON_LDS(lds_k0, lds_k1, lds_v0, lds_v1);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;     // which half of the wave
    const int ln = lane & 31;

    int b, h, qt;
    fa_geom g;
    fa_decode_item(a, b, h, qt, g);
    const int i0 = qt * BM;
    const int i_last = min(i0 + BM, g.sq) - 1;
    const fa_kv_range kr = fa_tile_kv_range(g, i0, i_last, BN);
    const int n_tiles = kr.end - kr.begin;
    const int kv_lim = min(kr.end * BN, g.skv);   // keys past this are never needed

    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.q_bs + h * a.q_hs +
                         (int64_t(g.q_start) + i0) * a.q_rs;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.kv_bs + h * a.kv_hs +
                         int64_t(g.kv_start) * a.kv_rs;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + b * a.kv_bs + h * a.kv_hs +
                         int64_t(g.kv_start) * a.kv_rs;
    const int q_rs = int(a.q_rs), kv_rs = int(a.kv_rs);

    // This lane's query row; Q^T is the B operand: lane holds d = 16 t + 8 hl .. + 7.
    const int lrow = wave * 32 + ln;
    const int row = i0 + lrow;
    const bool row_ok = row < g.sq;
    u32x4 qop[KSTEPS];
    {
        const __amdgpu_buffer_rsrc_t rq = fa_rsrc(qp, ((min(g.sq - i0, BM) - 1) * q_rs + D) * 2);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) qop[t] = fa_bload(rq, (lrow * q_rs + 16 * t + 8 * hl) * 2);
    }
    const int row_lo = fa_row_lo(g, row);
    const int row_hi = fa_row_hi(g, row);
    const int wrow0 = i0 + wave * 32;
    const int wlast = min(wrow0 + 31, g.sq - 1);   // last valid row of this wave
    const float sl2 = a.scale_log2;
    float slope2 = 0.f;
    if (ALIBI) slope2 = a.slopes[h] * kLog2e;
    const int off = g.skv - g.sq;
    const int aoff = a.alibi_left ? 0 : off;   // diagonal of the linear alibi bias
    const uint8_t* mrow = nullptr;
    if (DENSE) mrow = a.mask + b * a.m_bs + h * a.m_hs + int64_t(row_ok ? row : 0) * a.m_rs;

    float m_run = -INFINITY;   // running max, log2 domain (scale folded in)
    float l_run = 0.f;         // this lane's half of the running sum
    f32x16 oacc[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) oacc[db] = f32x16{};

    // HBM -> LDS for one K or V tile: lane l of the wave's p-th load fills physical chunk
    // P = 64 (LOADS wave + p) + l, i.e. row P / KCH, so it fetches that row's logical chunk.
    // The per-lane source offsets are the same for every tile (only the buffer base moves).
    // (Kept as scalars: a lambda capturing a local array here made the host compiler drop
    // this kernel's launch stub.)
    static_assert(LOADS <= 4, "at most four direct loads per thread and tile");
    const int wave_u = fa_uniform(wave);
    auto dl_offset = [&](int p) {
        const int P = (wave * LOADS + p) * 64 + lane;
        const int j = P / KCH;
        return (j * kv_rs + fa_swz<KCH>(j, P % KCH) * 8) * 2;
    };
    const int dl0 = dl_offset(0), dl1 = LOADS > 1 ? dl_offset(1) : 0;
    const int dl2 = LOADS > 2 ? dl_offset(2) : 0, dl3 = LOADS > 3 ? dl_offset(3) : 0;
    auto dload = [&](const uint16_t* base, int kt, u32x4* dst) {
        const int j0 = kt * BN;
        const int rows = min(BN, kv_lim - j0);
        const __amdgpu_buffer_rsrc_t r =
            fa_rsrc(base + int64_t(j0) * kv_rs, rows > 0 ? ((rows - 1) * kv_rs + D) * 2 : 0);
#pragma unroll
        for (int p = 0; p < LOADS; ++p) {
            const int off = p == 0 ? dl0 : (p == 1 ? dl1 : (p == 2 ? dl2 : dl3));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + (wave_u * LOADS + p) * 64), 16, off,
                                                     0, 0, 0);
        }
    };

    // Per-lane LDS byte offsets of the V^T operand halves (see the transpose-read note above):
    // group lanes address rows 16 t + 8 h2 + 4 hl + (lane%16)/4 and columns
    // 32 db + 16 ((lane/16)%2) + 4 (lane%4).
    const int src = lane & 15;
    const int dlo = 16 * ((lane >> 4) & 1) + 4 * (src & 3);
    int v_off[2][DBLK];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        const int j = 8 * h2 + 4 * hl + (src >> 2);   // + 16 t
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const int d0 = 32 * db + dlo;
            v_off[h2][db] = (j * KCH + fa_swz<KCH>(j, d0 >> 3)) * 16 + (d0 & 7) * 2;
        }
    }
    int k_off[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) k_off[t] = ln * KCH + fa_swz<KCH>(ln, 2 * t + hl);   // + 32 jb rows

    // S^T of one kv tile from K buffer kb (keys x rows): lane holds row `row`, keys
    // 32 jb + 8 (r/4) + 4 hl + r%4 of the tile in sacc[jb][r].
    auto qk = [&](const u32x4* kb, f32x16 (&sacc)[2]) {
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

    // Tile `it` (its S^T already in s_cur): start the HBM -> LDS loads of K(it+2) and V(it+1),
    // issue the MFMAs of S^T(it+1) (into s_nxt, when NEXT) so they run while this tile's
    // softmax is on the VALU, then O += P V(it). K(t) and V(t) live in buffer t % 2.
    auto step = [&](auto next_tag, int it, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2], const u32x4* k_next,
                    const u32x4* v_cur, u32x4* k_fill, u32x4* v_fill) {
            constexpr bool NEXT = decltype(next_tag)::value;
            const int kt = kr.begin + it;
            if (it + 2 < n_tiles) dload(kp, kt + 2, k_fill);
            if (it + 1 < n_tiles) dload(vp, kt + 1, v_fill);
            const int j0 = kt * BN;
            // Per-element masking (partial tiles only) before the next tile's MFMAs are issued.
            const bool full = !DENSE && fa_tile_full(g, wrow0, wlast, j0, BN);
            if (!full) {
                if (DENSE) {
#pragma unroll
                    for (int e = 0; e < 32; ++e) {
                        const int r = e & 15;
                        const int j = j0 + 32 * (e >> 4) + 8 * (r >> 2) + 4 * hl + (r & 3);
                        const bool vis = row_ok && j < g.skv && mrow[j] == 0;
                        s_cur[e >> 4][r] = vis ? s_cur[e >> 4][r] : -INFINITY;
                    }
                } else {
                    const int lo_rel = row_lo - j0 - 4 * hl;
                    const int hi_rel = row_hi - j0 - 4 * hl;
#pragma unroll
                    for (int e = 0; e < 32; ++e) {
                        const int r = e & 15;
                        const int kc = 32 * (e >> 4) + 8 * (r >> 2) + (r & 3);
                        s_cur[e >> 4][r] = (kc >= lo_rel && kc <= hi_rel) ? s_cur[e >> 4][r] : -INFINITY;
                    }
                }
            }
            if constexpr (NEXT) qk(k_next, s_nxt);
            float s[32];
#pragma unroll
            for (int e = 0; e < 32; ++e) s[e] = s_cur[e >> 4][e & 15];
            // Row maximum over this lane's 32 keys in four independent chains (short dependency
            // chains keep the VALU busy), then across the lane pair.
            float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            if (AL == 1) {
                const float base = slope2 * float(j0 + 4 * hl - row - aoff);
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    const int r = e & 15;
                    const int kc = 32 * (e >> 4) + 8 * (r >> 2) + (r & 3);
                    s[e] = fmaf(s[e], sl2, fmaf(slope2, float(kc), base));
                    m4[e & 3] = fmaxf(m4[e & 3], s[e]);
                }
            } else if (AL == 2) {
                // Square-root bias: -slope sign(d) sqrt(|d|), d = i + (Skv - Sq) - j (v_sqrt_f32,
                // within 1 ulp: d is an integer below 2^24).
                const float dbase = float(row + off - j0 - 4 * hl);
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    const int r = e & 15;
                    const int kc = 32 * (e >> 4) + 8 * (r >> 2) + (r & 3);
                    const float dd = dbase - float(kc);
                    s[e] = fmaf(s[e], sl2, -slope2 * copysignf(__builtin_amdgcn_sqrtf(fabsf(dd)), dd));
                    m4[e & 3] = fmaxf(m4[e & 3], s[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 32; ++e) m4[e & 3] = fmaxf(m4[e & 3], s[e]);
            }
            float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
            if (!ALIBI) mx *= sl2;
            mx = pair_max(mx);
            // Rescale only when the row maximum grows by more than 2^8: p stays <= 256, and the
            // final O / l and LSE do not depend on which maximum was used.
            const bool need = mx > m_run + 8.f;
            const float alpha = need ? exp2f(m_run - mx) : 1.f;
            m_run = need ? mx : m_run;
            const float m_use = m_run == -INFINITY ? 0.f : m_run;
            float p[32];
            float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                p[e] = ALIBI ? __builtin_amdgcn_exp2f(s[e] - m_use)
                             : __builtin_amdgcn_exp2f(fmaf(s[e], sl2, -m_use));
                l4[e & 3] += p[e];
            }
            l_run = fmaf(l_run, alpha, (l4[0] + l4[1]) + (l4[2] + l4[3]));
            // P^T as the B operand: k-step t takes accumulator entries 8 (t%2) .. +7 of block t/2.
            u32x4 pop[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int base = 16 * (t >> 1) + 8 * (t & 1);
                pop[t] = u32x4{io::pack(p[base + 0], p[base + 1]), io::pack(p[base + 2], p[base + 3]),
                               io::pack(p[base + 4], p[base + 5]), io::pack(p[base + 6], p[base + 7])};
            }
            // Keep the softmax above the rescale branch below (otherwise it sinks towards its
            // only use, the PV MFMAs, and lands outside the block it is interleaved with).
#pragma unroll
            for (int t = 0; t < 4; ++t) asm volatile("" : : "v"(pop[t]));
            asm volatile("" : : "v"(l_run));
            // Interleave: the MFMAs of the next tile's S^T (when NEXT) with this tile's softmax
            // VALU work, K operand reads running four ahead.
            if constexpr (NEXT) {
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < 2 * KSTEPS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                    if (i + 4 < 2 * KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            if (__any(need)) {
#pragma unroll
                for (int db = 0; db < DBLK; ++db) oacc[db] *= alpha;
            }
            // O^T (d x rows) += V^T P^T; the V^T operand is two transpose reads. Consecutive
            // MFMAs go to different accumulators (t outer, db inner) so none waits on the last.
            const char* vbase = reinterpret_cast<const char*>(v_cur);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int db = 0; db < DBLK; ++db) {
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(vbase + v_off[0][db] + t * 16 * KCH * 16));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(vbase + v_off[1][db] + t * 16 * KCH * 16));
                    const u32x4 vop = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                       __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
                    oacc[db] = io::mma(vop, pop[t], oacc[db]);
                }
            }
            // PV: keep the transpose reads two MFMAs ahead.
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
            for (int i = 0; i < 4 * DBLK; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                if (i + 2 < 4 * DBLK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
            }
            __builtin_amdgcn_s_waitcnt(0);   // this thread's loads have landed in LDS
            __syncthreads();
    };

    if (n_tiles > 0) {
        using yes = std::integral_constant<bool, true>;
        using no = std::integral_constant<bool, false>;
        dload(kp, kr.begin, lds_k0);
        dload(vp, kr.begin, lds_v0);
        if (n_tiles > 1) dload(kp, kr.begin + 1, lds_k1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        f32x16 sA[2], sB[2];
        qk(lds_k0, sA);
        __syncthreads();   // K buffer 0 is refilled with K(2) during tile 0
        int it = 0;
        for (; it + 2 < n_tiles; it += 2) {
            step(yes{}, it, sA, sB, lds_k1, lds_v0, lds_k0, lds_v1);
            step(yes{}, it + 1, sB, sA, lds_k0, lds_v1, lds_k1, lds_v0);
        }
        if (it + 1 < n_tiles) {
            step(yes{}, it, sA, sB, lds_k1, lds_v0, lds_k0, lds_v1);
            step(no{}, it + 1, sB, sA, lds_k0, lds_v1, lds_k1, lds_v0);
        } else {
            step(no{}, it, sA, sB, lds_k1, lds_v0, lds_k0, lds_v1);
        }
    }

    // Epilogue: O = O / l, LSE = ln2 (m + log2 l); rows with nothing visible give 0 and -inf.
    const float l_tot = pair_sum(l_run);
    if (row_ok) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (hl == 0) {
            a.lse[b * a.lse_bs + h * a.lse_hs + g.q_start + row] =
                l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
        }
        uint16_t* op = static_cast<uint16_t*>(a.o) + b * a.q_bs + h * a.q_hs +
                       (int64_t(g.q_start) + row) * a.q_rs;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int d = 32 * db + 8 * gi + 4 * hl;
                const u32x2 w = {io::pack(oacc[db][4 * gi + 0] * inv, oacc[db][4 * gi + 1] * inv),
                                 io::pack(oacc[db][4 * gi + 2] * inv, oacc[db][4 * gi + 3] * inv)};
                *reinterpret_cast<u32x2*>(op + d) = w;
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// MFMA ping-pong kernel (the fast path).
//
// A 512-thread workgroup owns 256 query rows, 32 per wave; waves w and w + 4 share a SIMD.
// Group A (waves 0-3) and group B (waves 4-7) run the same sequence of phases,
//     QK(0) | SM(0) | MM(0) | SM(1) | MM(1) | ... | SM(n-1) | MM(n-1)
// with B one phase behind A and a workgroup barrier between phases. SM(t) is the masked
// online softmax of kv tile t (VALU only); MM(t) is O^T += V(t)^T P(t)^T followed by
// S^T(t+1) = K(t+1) Q^T (matrix core only). In every phase one group runs MFMAs while its
// partner on the same SIMD runs the softmax, so the exponentials hide under the matrix work
// instead of alternating with it.
//
// Tile data: set u = {K(u), V(u-1)} is what MM(u-1) reads, in phase 2u of A and 2u + 1 of B.
// Two LDS buffers hold sets u and u + 1; set u + 2 goes HBM -> LDS (direct buffer loads)
// into the buffer of set u as soon as both groups are done with it, two phases before it is
// needed. Each group issues its half of the loads at the start of the phase in which set
// u + 2 becomes writable and waits for them (vmcnt) at the end of the following phase.
// Phase barriers order LDS only, so loads stay in flight across them.
// ------------------------------------------------------------------------------------------

template <int D, bool IS_BF16, int AL, bool DENSE, bool PAGED = false, bool EDGE = false>
__global__ __attribute__((amdgpu_flat_work_group_size(PP_THREADS, PP_THREADS),
                          amdgpu_waves_per_eu(2, 2))) void
fa_fwd_pp(const fa_kargs a) {
    static_assert(D == 64 || D == 128, "MFMA path covers D = 64 and 128");
    static_assert(AL >= 0 && AL <= 2, "alibi kind: 0 none, 1 linear, 2 square root");
    constexpr bool ALIBI = AL != 0;
    using io = mfma_io<IS_BF16>;
    constexpr int BM = PP_BM, BN = PP_BN, NT = PP_THREADS;
    constexpr int KCH = D / 8;                   // 16-byte chunks per K / V row
    constexpr int KSTEPS = D / 16;               // k-steps of S^T = K Q^T
    constexpr int DBLK = D / 32;                 // 32-row blocks of O^T
    constexpr int TILE_CHUNKS = BN * KCH;        // 16-byte chunks per K or V tile
    constexpr int LOADS = TILE_CHUNKS / NT;      // direct loads per thread and tile
    constexpr int BATCH = 2 * LOADS;             // loads per thread and set (V and K)
    static_assert(LOADS >= 1 && LOADS <= 2 && TILE_CHUNKS % NT == 0, "tile shape");

    __shared__ u32x4 lds_k0[TILE_CHUNKS], lds_k1[TILE_CHUNKS], lds_k2[TILE_CHUNKS], lds_k3[TILE_CHUNKS];
    __shared__ u32x4 lds_v0[TILE_CHUNKS], lds_v1[TILE_CHUNKS], lds_v2[TILE_CHUNKS], lds_v3[TILE_CHUNKS];
    FA_POISON_LDS(lds_k0, lds_k1, lds_k2, lds_k3, lds_v0, lds_v1, lds_v2, lds_v3);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int ln = lane & 31;
    const int wave_u = fa_uniform(wave);
    const int grp = wave_u >> 2;   // 0: group A, 1: group B (one phase behind)

    int b, h, qt;
    fa_geom g;
    fa_decode_item(a, b, h, qt, g);
    // Dense mask: the q tile of launch rank qt is the pre-pass's choice (most visited tiles first;
    // a dense mask has no reverse order, so the rank is qt itself).
    int ms = 0;
    if constexpr (DENSE) {
        ms = (a.m_bcast_b ? 0 : b) * a.m_heads + (a.m_bcast_h ? 0 : h);
        if (a.tile_perm) qt = fa_uniform(a.tile_perm[int64_t(ms) * a.dense_nqt + qt]);
    }
    const int i0 = qt * BM;
    const int i_last = min(i0 + BM, g.sq) - 1;
    const fa_kv_range kr = fa_tile_kv_range(g, i0, i_last, BN);
    int n_tiles = kr.end - kr.begin;
    int kv_lim = min(kr.end * BN, g.skv);
    // Kernels with an alibi bias walk the item's kv tiles from the last to the first: the bias
    // rises with the key index, so the row maximum then shows up in the first tiles and the
    // softmax's fast path (see there) holds for the rest. Positions t >= n_tiles map past the
    // range on either side; their loads read nothing.
    constexpr bool REV = ALIBI && !DENSE;
    auto kt_of = [&](int t) __attribute__((always_inline)) { return REV ? kr.end - 1 - t : kr.begin + t; };
    // Dense mask: the kv tiles come from the pre-pass's list for this q tile (a count, then per
    // visited tile kt | full-wave bits << 24), and the per-element mask from its packed bits.
    // Entries are read by scalar loads through the constant address space (the tables do not
    // change during the kernel); past the count an entry is FA_DENSE_END, a tile past every key
    // whose loads read nothing.
    const __attribute__((address_space(4))) uint32_t* trec = nullptr;
    const uint32_t* tbits = nullptr;
    if constexpr (DENSE) {
        n_tiles = 0;
        kv_lim = g.skv;
        if (a.tile_list) {
            const int64_t r = int64_t(ms) * a.dense_nqt + qt;
            trec = (const __attribute__((address_space(4))) uint32_t*)(a.tile_list + r * (a.dense_nkt + 1));
            tbits = a.tile_bits + r * a.dense_nkt * 512 + wave * 64 + lane;
            n_tiles = fa_uniform(int(trec[0]));
        }
    }
    auto ent = [&](int t) __attribute__((always_inline)) -> uint32_t {
        if constexpr (DENSE) return t < n_tiles ? trec[1 + t] : FA_DENSE_END;
        else return 0u;
    };

    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.q_bs + h * a.q_hs +
                         (int64_t(g.q_start) + i0) * a.q_rs;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.kv_bs + h * a.kv_hs +
                         int64_t(g.kv_start) * a.kv_rs;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + b * a.kv_bs + h * a.kv_hs +
                         int64_t(g.kv_start) * a.kv_rs;
    const int q_rs = int(a.q_rs), kv_rs = int(a.kv_rs);

    const int lrow = wave * 32 + ln;
    const int row = i0 + lrow;
    const bool row_ok = row < g.sq;
    u32x4 qop[KSTEPS];
    {
        const __amdgpu_buffer_rsrc_t rq = fa_rsrc(qp, ((min(g.sq - i0, BM) - 1) * q_rs + D) * 2);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) qop[t] = fa_bload(rq, (lrow * q_rs + 16 * t + 8 * hl) * 2);
    }
    const int row_lo = fa_row_lo(g, row);
    const int row_hi = fa_row_hi(g, row);
    const int wrow0 = i0 + wave * 32;
    const int wlast = min(wrow0 + 31, g.sq - 1);
    const float sl2 = a.scale_log2;
    float slope2 = 0.f;
    if (ALIBI) slope2 = a.slopes[h] * kLog2e;
    // Load these now: a scalar load left to the loop would be waited for there with
    // lgkmcnt(0), which also waits for every LDS read in flight.
    asm volatile("" : : "s"(sl2), "v"(slope2));
    const int off = g.skv - g.sq;
    const int aoff = a.alibi_left ? 0 : off;   // diagonal of the linear alibi bias

    // Paged K / V: a 64-key tile lies inside one page (pages hold 2^lbs >= 64 keys). Page ids
    // come straight from the block table with scalar loads, issued at the start of a softmax
    // phase and landed before its closing LDS reads: no VALU work (which would compete with the
    // other group's softmax on the same SIMD) and no wait inside a matrix phase.
    // (The table is read through the constant address space: it does not change during the
    // kernel, and uniform loads from there are scalar.)
    int lbs = 0, n_pages = 0, pg_last = 0, bs_mask = 0;
    uint32_t pg_bytes = 0;
    const __attribute__((address_space(4))) int32_t* bt_row = nullptr;
    if constexpr (PAGED) {
        lbs = a.log2_block_size;
        bs_mask = (1 << lbs) - 1;
        n_pages = a.num_pages;
        pg_bytes = uint32_t(a.page_stride) * 2u;
        bt_row = (const __attribute__((address_space(4))) int32_t*)(a.block_table + b * a.bt_stride);
        pg_last = n_tiles > 0 ? (kv_lim - 1) >> lbs : 0;   // last table entry this item reads
        asm volatile("" : : "s"(lbs), "s"(n_pages), "s"(pg_bytes), "s"(bs_mask));
    }
    // Page id of key tile kt (-1 past the item's range: that load reads nothing).
    auto page_of = [&](int kt) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            const int pg = bt_row[max(min((kt * BN) >> lbs, pg_last), 0)];
            return kt < kr.end && kt >= kr.begin ? pg : -1;
        } else {
            return 0;
        }
    };
    int pg_v_next = 0, pg_k_next = 0;   // page ids of the next iteration's V and K loads
    // Dense mask: entries of the next iteration's V and K loads, of the current and next tile,
    // and the current tile's mask bits.
    uint32_t e_v_next = 0u, e_k_next = 0u, e_cur = 0u, e_nxt = 0u, hid_cur = 0u;

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x16 oacc[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) oacc[db] = f32x16{};

    // HBM -> LDS for this thread's share of one K or V tile (physical chunk
    // 64 (LOADS wave + p) + lane, i.e. row P / KCH, logical chunk un-swizzled).
    auto dl_offset = [&](int p) __attribute__((always_inline)) {
        const int P = (wave * LOADS + p) * 64 + lane;
        const int j = P / KCH;
        return (j * kv_rs + fa_swz<KCH>(j, P % KCH) * 8) * 2;
    };
    const int dl0 = dl_offset(0), dl1 = LOADS > 1 ? dl_offset(1) : 0;
    // Tile kt of K or V; `page` is its page id (paged K / V only). Rows past kv_lim, and every
    // row of a page id outside [0, num_pages), read as zeros.
    auto dload = [&](const uint16_t* base, int kt, int page, u32x4* dst) __attribute__((always_inline)) {
        const int j0 = max(kt, 0) * BN;
        int rows = REV && kt < kr.begin ? 0 : min(BN, kv_lim - j0);
        const uint16_t* tile = base + int64_t(j0) * kv_rs;
        if constexpr (PAGED) {
            // Page bytes and in-page offsets fit 32 bits (checked on the host): one 32 x 32 -> 64
            // bit product per tile.
            rows = unsigned(page) < unsigned(n_pages) ? rows : 0;
            tile = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(base) +
                                                     uint64_t(uint32_t(page)) * pg_bytes +
                                                     uint32_t((j0 & bs_mask) * kv_rs) * 2u);
        }
        const __amdgpu_buffer_rsrc_t r = fa_rsrc(tile, rows > 0 ? ((rows - 1) * kv_rs + D) * 2 : 0);
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

    // EDGE: true when no row of this wave sees a key of the item's tile t. The rows' intervals
    // [lo, hi] rise with the row, so the wave's visible keys lie in [lo(first row), hi(last
    // row)]. Such a wave skips the tile's softmax and hands a zero P^T to its PV product (its
    // MFMAs still run: a branch around them costs the fused matrix phase its register
    // allocation). The planner picks this variant where such tiles are a large share of the
    // items (band edges, short causal items); the test costs long items about 0.5%.
    const int u_row0 = i0 + wave_u * 32, u_last = min(u_row0 + 31, g.sq - 1);
    const int w_lo = fa_row_lo(g, u_row0), w_hi = fa_row_hi(g, u_last);
    auto wave_empty = [&](int t) __attribute__((always_inline)) {
        if constexpr (DENSE || !EDGE) {
            return false;
        } else {
            const int j0 = kt_of(t) * BN;
            return u_row0 >= g.sq || w_hi < j0 || w_lo > j0 + BN - 1;
        }
    };

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

    // SM(t): mask, scale (+ alibi), online softmax update, P^T packed for the PV product. The
    // O^T rescale happens here too: no MFMA of this wave is using the accumulators.
    // es: the dense-mask entry of tile t; hidden: its packed mask bits for this lane.
    auto softmax = [&](int t, uint32_t es, uint32_t hidden) __attribute__((always_inline)) {
        if (wave_empty(t)) {
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) pop[t4] = u32x4{0u, 0u, 0u, 0u};
            return;
        }
        const int j0 = DENSE ? int(es & FA_DENSE_KT) * BN : kt_of(t) * BN;
        const bool full = DENSE ? ((es >> (24 + wave_u)) & 1u) != 0u : fa_tile_full(g, wrow0, wlast, j0, BN);
        if (!full) {
            if (DENSE) {
                // Bit e hides this lane's key 32 (e / 16) + 8 ((e / 4) % 4) + 4 hl + e % 4 of the tile.
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    sacc[e >> 4][e & 15] = (hidden >> e) & 1u ? -INFINITY : sacc[e >> 4][e & 15];
            } else {
                const int lo_rel = row_lo - j0 - 4 * hl;
                const int hi_rel = row_hi - j0 - 4 * hl;
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    const int r = e & 15;
                    const int kc = 32 * (e >> 4) + 8 * (r >> 2) + (r & 3);
                    sacc[e >> 4][r] = (kc >= lo_rel && kc <= hi_rel) ? sacc[e >> 4][r] : -INFINITY;
                }
            }
        }
        float s[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) s[e] = sacc[e >> 4][e & 15];
        if (AL == 1) {
            const float base = slope2 * float(j0 + 4 * hl - row - aoff);
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const int r = e & 15;
                const int kc = 32 * (e >> 4) + 8 * (r >> 2) + (r & 3);
                s[e] = fmaf(s[e], sl2, fmaf(slope2, float(kc), base));
            }
        } else if (AL == 2) {
            // Square-root bias: -slope sign(d) sqrt(|d|), d = i + (Skv - Sq) - j (v_sqrt_f32,
            // within 1 ulp: d is an integer below 2^24).
            const float dbase = float(row + off - j0 - 4 * hl);
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
        // Fast path: once the row has a maximum, exponentiate against it as it stands. The final
        // O / l and LSE do not depend on which maximum was used, only on p staying finite and
        // within the range fp32 and the 16-bit P hold; a lane sum of at most 2^15 bounds every
        // p by 2^15, which fp16 holds (its largest finite value is 65504; an overflow to inf, or
        // a NaN, fails the test too). Otherwise the wave takes the exact path: the tile's row
        // maximum, and the rescale when it grows by more than 2^8.
        // An alibi bias rises with the key index: walked upwards (a dense mask's tile list) the
        // row maximum would grow from tile to tile and the fast path mostly fail, so that case
        // takes the exact path.
        bool exact = (ALIBI && DENSE) || __any(m_run == -INFINITY);
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
        // The softmax belongs to this phase: keep it from sinking past the barrier.
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) asm volatile("" : : "v"(pop[t4]));
        asm volatile("" : : "v"(l_run));
    };

    // The V^T operands of the first NPRE PV MFMAs are read at the end of the preceding softmax
    // phase, so a matrix phase starts with MFMAs instead of waiting for LDS.
    constexpr int NPRE = DBLK;   // (t = 0, db = 0 .. DBLK-1)
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
    // MM(t): O^T += V^T P^T from V buffer vb, then S^T of the next tile from K buffer kb. After
    // the last tile the S^T product reads a stale K buffer and its result is never used.
    auto matmul = [&](const u32x4* kb, const u32x4* vb, auto&& between) __attribute__((always_inline)) {
        const char* vbase = reinterpret_cast<const char*>(vb);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
                oacc[db] = io::mma(t == 0 ? vpre[db] : vread(vbase, t, db), pop[t], oacc[db]);
        between();
        qk(kb);
        // LDS reads run about three MFMAs ahead: two per PV MFMA (its two V^T halves) and one
        // per S^T MFMA. The tile loads of `between` (scalar address arithmetic, M0 and the DMA
        // issue) go into the gaps of the first MFMAs: left free, the scheduler puts them all
        // ahead of the first MFMA, which then starts late.
        constexpr int NPV = 4 * DBLK, NQK = 2 * KSTEPS;
        constexpr int NDMA = 2 * LOADS;
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < NPV + NQK; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (i < 16) __builtin_amdgcn_sched_group_barrier(0x004, 4, 0);
            // V tile after MFMAs 5.., K tile after MFMAs 11..: each address chain has a few
            // MFMA gaps to run in.
#pragma unroll
            for (int p = 0; p < NDMA; ++p)
                if (i == 5 + 6 * (p / LOADS) + p % LOADS) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        }
    };

    // Set u = {V(u), K(u+1)} is what MM(u) reads; it lives in buffer u % 4. Both groups issue
    // their share of set t + 3 during MM(t) (into the buffer of set t - 1, which MM(t-1) of both
    // groups has finished with) and wait at the end of MM(t) until only the newest batch is in
    // flight. For group A that phase is slot 2t+2, for B slot 2t+3; set u is first read by A's
    // prefetch in slot 2u+1, after both waits (slots 2u-2 and 2u-1) and their barriers, giving
    // each batch three phases to land. Every batch is the same number of loads per thread (an
    // empty range past the last tile: nothing read, zeros written to the free buffer), and both
    // groups issue and wait at the same points of the program.
    auto iter = [&](auto s_tag, int t) __attribute__((always_inline)) {
        constexpr int S = decltype(s_tag)::value;   // t % 4
        constexpr int F = (S + 3) % 4;              // buffer of set t + 3 (and of set t - 1)
        const u32x4* k_cur = S == 0 ? lds_k0 : (S == 1 ? lds_k1 : (S == 2 ? lds_k2 : lds_k3));
        const u32x4* v_cur = S == 0 ? lds_v0 : (S == 1 ? lds_v1 : (S == 2 ? lds_v2 : lds_v3));
        u32x4* k_fill = F == 0 ? lds_k0 : (F == 1 ? lds_k1 : (F == 2 ? lds_k2 : lds_k3));
        u32x4* v_fill = F == 0 ? lds_v0 : (F == 1 ? lds_v1 : (F == 2 ? lds_v2 : lds_v3));
        // Page ids of this iteration's loads were fetched one iteration ago; fetch the next ones.
        const int pg_v = pg_v_next, pg_k = pg_k_next;
        if constexpr (PAGED) {
            pg_v_next = page_of(kt_of(t + 4));
            pg_k_next = page_of(kt_of(t + 5));
        }
        // Dense mask: entries of V(t + 3) and K(t + 4) were fetched one iteration ago (V(t + 4) is
        // this iteration's K), tile t + 1's two. Fetch K(t + 5) and tile t + 2.
        const uint32_t e_v = e_v_next, e_k = e_k_next, e_s = e_cur;
        uint32_t e_far = 0u;
        if constexpr (DENSE) {
            e_v_next = e_k_next;
            e_k_next = ent(t + 5);
            e_far = ent(t + 2);
        }
        softmax(t, e_s, hid_cur);
        // Tile t + 1's mask bits for the next softmax, when this wave masks it: the load has the
        // matrix phase to land (its closing wait covers every load issued before the tile batch).
        if constexpr (DENSE) {
            if (e_nxt != FA_DENSE_END && !((e_nxt >> (24 + wave_u)) & 1u))
                hid_cur = __builtin_nontemporal_load(tbits + int64_t(e_nxt & FA_DENSE_KT) * 512);
            e_cur = e_nxt;
            e_nxt = e_far;
        }
        // The scalar loads land here, while no LDS read is in flight.
        if constexpr (PAGED) asm volatile("" : : "s"(pg_v_next), "s"(pg_k_next));
        if constexpr (DENSE) asm volatile("" : : "s"(e_v_next), "s"(e_k_next), "s"(e_nxt));
        prefetch(v_cur);
        fa_lds_barrier_pending<2 * NPRE>();   // the prefetched V^T reads may still be in flight
        __builtin_amdgcn_s_setprio(1);
        matmul(k_cur, v_cur, [&]() __attribute__((always_inline)) {
            dload(vp, DENSE ? int(e_v & FA_DENSE_KT) : kt_of(t + 3), pg_v, v_fill);
            dload(kp, DENSE ? int(e_k & FA_DENSE_KT) : kt_of(t + 4), pg_k, k_fill);
        });
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_s_waitcnt(fa_vmcnt(BATCH));
        fa_lds_barrier();
    };

    if (n_tiles > 0) {
        // K(0) goes into buffer 3's K half (set 3 is not loaded before iteration 0's matrix
        // phase, after both groups have used K(0)); sets 0, 1, 2 into buffers 0, 1, 2.
        const int pg0 = page_of(kt_of(0)), pg1 = page_of(kt_of(1));
        const int pg2 = page_of(kt_of(2)), pg3 = page_of(kt_of(3));
        pg_v_next = pg3;
        pg_k_next = page_of(kt_of(4));
        int kt0 = kt_of(0), kt1 = kt_of(1), kt2 = kt_of(2), kt3 = kt_of(3);
        if constexpr (DENSE) {
            const uint32_t e0 = ent(0), e1 = ent(1), e2 = ent(2), e3 = ent(3);
            kt0 = int(e0 & FA_DENSE_KT);
            kt1 = int(e1 & FA_DENSE_KT);
            kt2 = int(e2 & FA_DENSE_KT);
            kt3 = int(e3 & FA_DENSE_KT);
            e_v_next = e3;
            e_k_next = ent(4);
            e_cur = e0;
            e_nxt = e1;
            if (!((e0 >> (24 + wave_u)) & 1u)) hid_cur = __builtin_nontemporal_load(tbits + int64_t(kt0) * 512);
        }
        dload(kp, kt0, pg0, lds_k3);
        dload(vp, kt0, pg0, lds_v0);
        dload(kp, kt1, pg1, lds_k0);
        dload(vp, kt1, pg1, lds_v1);
        dload(kp, kt2, pg2, lds_k1);
        dload(vp, kt2, pg2, lds_v2);
        dload(kp, kt3, pg3, lds_k2);
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
        // Full trips of four, then a tail with nested guards: every path into an iteration runs
        // the earlier iterations (and their waits), which the compiler's own wait analysis must
        // be able to see.
        int t = 0;
        for (; t + 4 <= n_tiles; t += 4) {
            iter(s0{}, t);
            iter(s1{}, t + 1);
            iter(s2{}, t + 2);
            iter(s3{}, t + 3);
        }
        if (t < n_tiles) {
            iter(s0{}, t);
            if (t + 1 < n_tiles) {
                iter(s1{}, t + 1);
                if (t + 2 < n_tiles) iter(s2{}, t + 2);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the loop
    }

    // Epilogue: O = O / l, LSE = ln2 (m + log2 l); rows with nothing visible give 0 and -inf.
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (row_ok && hl == 0) {
        a.lse[b * a.lse_bs + h * a.lse_hs + g.q_start + row] =
            l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
    // O goes out as whole rows: each wave stages its 32 x D tile (bf16 / fp16) in half of one
    // K or V buffer and reads it back one row per KCH lanes, so every store instruction writes
    // 64 / KCH complete rows. A lane's accumulators hold one query row and 4-element runs of
    // columns, which stored directly would give row-strided 8-byte pieces. Group A runs this
    // while group B's last matrix phase reads set S = (n_tiles - 1) % 4 and the last (empty)
    // tile loads fill set S + 3, so A takes set S + 1, whose loads landed phases ago; group B
    // runs it after its final wait, when every load and read is done, and takes set S + 2.
    // Rows are KCH 16-byte chunks, chunk c of row r stored at c ^ (r % KCH).
    {
        const int set = (((n_tiles - 1) & 3) + 1 + grp) & 3;
        u32x4* kset = set == 0 ? lds_k0 : (set == 1 ? lds_k1 : (set == 2 ? lds_k2 : lds_k3));
        u32x4* vset = set == 0 ? lds_v0 : (set == 1 ? lds_v1 : (set == 2 ? lds_v2 : lds_v3));
        char* stage = reinterpret_cast<char*>(((wave_u & 2) ? vset : kset) + (wave_u & 1) * (TILE_CHUNKS / 2));
        constexpr int ROWB = KCH * 16;   // bytes of a staged row
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int c = 4 * db + gi;   // chunk of columns 32 db + 8 gi .. + 7; this lane has half hl
                const u32x2 w = {io::pack(oacc[db][4 * gi + 0] * inv, oacc[db][4 * gi + 1] * inv),
                                 io::pack(oacc[db][4 * gi + 2] * inv, oacc[db][4 * gi + 3] * inv)};
                *reinterpret_cast<u32x2*>(stage + ln * ROWB + (c ^ (ln & (KCH - 1))) * 16 + 8 * hl) = w;
            }
        }
        // LDS operations of one wave complete in order; this keeps the compiler from moving the
        // reads above the writes (other lanes' data).
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        uint16_t* obase = static_cast<uint16_t*>(a.o) + b * a.q_bs + h * a.q_hs + (int64_t(g.q_start) + wrow0) * a.q_rs;
        constexpr int RPI = 64 / KCH;   // rows per read / store instruction
        const int c = lane % KCH;
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
            const int r = it * RPI + lane / KCH;
            const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * ROWB + (c ^ (r & (KCH - 1))) * 16);
            // Non-temporal: O is not read again here, so it need not displace K / V in the caches.
            if (wrow0 + r < g.sq) __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(obase + int64_t(r) * q_rs + 8 * c));
        }
    }
    // Group A ran one phase ahead: its last barrier matches B's final MM phase.
    if (n_tiles > 0 && grp == 0) fa_lds_barrier();
}

// ------------------------------------------------------------------------------------------
// Split-KV decode: at most 16 query rows per (batch, head). One workgroup per (batch, head,
// split of the visible kv tiles); its four waves take every fourth tile of the split, each
// with its own online-softmax state, and combine at the end; fa_decode_merge combines the
// splits with LSE = log2-sum-exp2 of the split LSEs and O = sum of 2^(LSE_s - LSE) O_s.
//
// MFMA 16x16x32: S^T = K Q^T with K as the A operand straight from HBM (16 bytes per lane,
// rows past the tile's valid keys read as zeros) and the query rows as the 16 columns. Key
// rows are permuted inside the 64-key tile so that each lane's S^T values are exactly its P
// operand of O = P V (rows: queries, k: keys): block bb, A row r holds key
// 32 (bb / 2) + 8 (r / 4) + 4 (bb % 2) + r % 4. V goes to a per-wave LDS buffer with direct
// loads and comes back as the B operand (8 consecutive keys of one column per lane) through
// ds_read_b64_tr_b16, whose 16-lane groups return element i % 4 of the vector addressed by
// lane 4 e + i / 4 as element e of lane i.
// ------------------------------------------------------------------------------------------

constexpr int DC_THREADS = 256;
constexpr int DC_BN = FA_DEC_BN;     // keys per tile
constexpr int DC_ROWS = FA_DEC_ROWS; // query rows (the MFMA's 16 columns)

struct fa_decode_args {
    float* o_part;          // [split slots, N, 16, D]: each split's O / l (batches with splits)
    float* lse_part;        // [split slots, N, 16]: each split's log2(sum) + max, log2 domain
    const int32_t* batch;   // table mode: per batch (first slot, splits); else nullptr
    int32_t n_split;        // fixed-length mode: splits of every batch
};

// Work of decode workgroup w: entry e = w / N (a (batch, split) pair), head w % N; the
// batch's split count and its first partial-result slot. Slot (base + split) * N + h holds
// this workgroup's partial result when ns > 1.
struct fa_dec_work {
    int b, h, split, ns, base;
};

__device__ __forceinline__ fa_dec_work fa_decode_work(const fa_kargs& a, const fa_decode_args& dc, int w) {
    fa_dec_work r;
    r.h = w % a.N;
    const int e = w / a.N;
    if (a.items) {
        typedef const __attribute__((address_space(4))) int32_t* cptr;
        r.b = fa_uniform(((cptr)a.items)[2 * e]);
        r.split = fa_uniform(((cptr)a.items)[2 * e + 1]);
        r.base = fa_uniform(((cptr)dc.batch)[2 * r.b]);
        r.ns = fa_uniform(((cptr)dc.batch)[2 * r.b + 1]);
    } else {
        r.b = e / dc.n_split;
        r.split = e % dc.n_split;
        r.ns = dc.n_split;
        r.base = r.b * dc.n_split;
    }
    return r;
}

template <int D, bool IS_BF16, int AL, bool PAGED>
__global__ __launch_bounds__(DC_THREADS) void fa_decode_split(const fa_kargs a, const fa_decode_args dc) {
    static_assert(D == 64 || D == 128, "MFMA decode covers D = 64 and 128");
    using io = mfma_io<IS_BF16>;
    using mm = mfma16_io<IS_BF16>;
    constexpr int KD = D / 32;                 // k-steps of S^T = K Q^T
    constexpr int NK = 4 * KD;                 // K operand loads per tile (4 blocks of 16 keys)
    constexpr int ROW_B = D * 2;               // bytes of a key row
    constexpr int NV = DC_BN * ROW_B / 1024;   // 1 KB direct loads per V tile
    constexpr int RPL = 1024 / ROW_B;          // V rows per direct load
    constexpr int DB = D / 16;                 // 16-column blocks of O
    constexpr int TILE_U4 = DC_BN * D / 8;     // 16-byte chunks of a tile
    __shared__ u32x4 lds_v[4 * 2 * TILE_U4];   // per wave, two V tiles
    FA_POISON_LDS(lds_v);

    const int lane = threadIdx.x & 63;
    const int wave = fa_uniform(threadIdx.x >> 6);
    const int n = lane & 15;    // query row (S^T column / P and O row block index)
    const int gq = lane >> 4;   // 16-lane group

    const fa_dec_work wk = fa_decode_work(a, dc, blockIdx.x);
    const int b = wk.b, h = wk.h, split = wk.split;
    const fa_geom g = fa_geom_of(a, b);
    if (g.sq <= 0) return;
    const int rows = min(g.sq, DC_ROWS);
    const fa_kv_range kr = fa_tile_kv_range(g, 0, rows - 1, DC_BN);
    const int n_tiles = kr.end - kr.begin;
    const int tps = (n_tiles + wk.ns - 1) / wk.ns;
    const int t0 = min(kr.begin + split * tps, kr.end);
    const int t1 = min(t0 + tps, kr.end);
    const int kv_lim = min(kr.end * DC_BN, g.skv);

    const int q_rs = int(a.q_rs), kv_rs = int(a.kv_rs);
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.q_bs + h * a.q_hs + int64_t(g.q_start) * a.q_rs;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.kv_bs + h * a.kv_hs + int64_t(g.kv_start) * a.kv_rs;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + b * a.kv_bs + h * a.kv_hs + int64_t(g.kv_start) * a.kv_rs;

    // Q^T operand: lane (gq, n) holds query row n, columns 32 kd + 8 gq .. + 7 (rows past Sq
    // read as zeros: their offsets are past the buffer's end because q_rs >= D).
    u32x4 qop[KD];
    {
        const __amdgpu_buffer_rsrc_t rq = fa_rsrc(qp, ((rows - 1) * q_rs + D) * 2);
#pragma unroll
        for (int kd = 0; kd < KD; ++kd) qop[kd] = fa_bload(rq, (n * q_rs + 32 * kd + 8 * gq) * 2);
    }
    const int row_lo = fa_row_lo(g, n), row_hi = fa_row_hi(g, n);
    const float sl2 = a.scale_log2;
    float slope2 = 0.f;
    if (AL != 0) slope2 = a.slopes[h] * kLog2e;
    const int off = g.skv - g.sq;
    const int aoff = a.alibi_left ? 0 : off;

    // Paged K / V: page ids by scalar loads (the table is read-only during the kernel).
    int lbs = 0, n_pages = 0, bs_mask = 0, pg_last = 0;
    uint32_t pg_bytes = 0;
    const __attribute__((address_space(4))) int32_t* bt_row = nullptr;
    if constexpr (PAGED) {
        lbs = a.log2_block_size;
        bs_mask = (1 << lbs) - 1;
        n_pages = a.num_pages;
        pg_bytes = uint32_t(a.page_stride) * 2u;
        bt_row = (const __attribute__((address_space(4))) int32_t*)(a.block_table + b * a.bt_stride);
        pg_last = n_tiles > 0 ? (kv_lim - 1) >> lbs : 0;
    }

    // Per-lane operand offsets.
    int k_off[4][KD];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
        const int key = 32 * (bb >> 1) + 8 * (n >> 2) + 4 * (bb & 1) + (n & 3);
#pragma unroll
        for (int kd = 0; kd < KD; ++kd) k_off[bb][kd] = (key * kv_rs + 32 * kd + 8 * gq) * 2;
    }
    // V tile in LDS: rows of D / 8 16-byte chunks; with D = 128, chunk c of row r sits at
    // c ^ vswz(r), vswz(r) = 4 (r % 4) + (r / 4) % 4, so that the transpose reads (per 16 lanes four
    // consecutive rows at two chunks) spread over all banks. With SQ_LDS_BANK_CONFLICT the
    // unswizzled tile spent 86% of its LDS cycles in conflicts; a read loop of this pattern
    // measured none with this swizzle. D = 64 keeps the plain layout. The swizzle depends on row
    // bits 0-3 only, so rows 32 apart share it.
    auto vswz = [](int r) { return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : 0; };
    int v_voff[4];   // source offset of this lane's 16 bytes in direct load p (by p % 4; + p RPL rows)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = lane * 16 / ROW_B, c = ((lane * 16) % ROW_B) / 16;
        v_voff[q] = r * kv_rs * 2 + ((c ^ vswz(q * RPL + r)) * 16);
    }
    int v_rd[2][DB];   // [half][column block]: LDS byte offset of this lane's transpose read (+ 32 kk rows)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int r = 8 * gq + 4 * hf + (n >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int byte = 32 * db + 8 * (n & 3);
            v_rd[hf][db] = r * ROW_B + (((byte >> 4) ^ vswz(r)) * 16) + (byte & 15);
        }
    }

    u32x4 kreg[2][NK];
    char* const vbuf = reinterpret_cast<char*>(lds_v) + wave * 2 * TILE_U4 * 16;

    // Loads of tile t into buffer BUF (t >= t1: nothing read, zeros written).
    auto issue = [&](auto buf_tag, int t) __attribute__((always_inline)) {
        constexpr int BUF = decltype(buf_tag)::value;
        const int j0 = t * DC_BN;
        int nrows = t < t1 ? min(DC_BN, kv_lim - j0) : 0;
        const uint16_t* kt = kp + int64_t(j0) * kv_rs;
        const uint16_t* vt = vp + int64_t(j0) * kv_rs;
        if constexpr (PAGED) {
            const int pg = bt_row[min(j0 >> lbs, pg_last)];
            nrows = unsigned(pg) < unsigned(n_pages) ? nrows : 0;
            const uint64_t o = uint64_t(uint32_t(pg)) * pg_bytes + uint32_t((j0 & bs_mask) * kv_rs) * 2u;
            kt = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(kp) + o);
            vt = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(vp) + o);
        }
        const int bytes = nrows > 0 ? ((nrows - 1) * kv_rs + D) * 2 : 0;
        const __amdgpu_buffer_rsrc_t rk = fa_rsrc(kt, bytes), rv = fa_rsrc(vt, bytes);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int kd = 0; kd < KD; ++kd) kreg[BUF][bb * KD + kd] = fa_bload(rk, k_off[bb][kd]);
        // V goes to LDS with the non-temporal hint (aux 2): decode reads each V row once, and the
        // hint measured 8-13% faster on every decode shape. The same hint on the K loads into
        // registers was slower.
#pragma unroll
        for (int p = 0; p < NV; ++p)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vbuf + (BUF * TILE_U4 + p * 64) * 16), 16,
                                                     v_voff[p & 3] + p * RPL * kv_rs * 2, 0, 0, 2);
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4{};

    auto compute = [&](auto buf_tag, int t) __attribute__((always_inline)) {
        constexpr int BUF = decltype(buf_tag)::value;
        const int j0 = t * DC_BN;
        f32x4 sacc[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            sacc[bb] = f32x4{};
#pragma unroll
            for (int kd = 0; kd < KD; ++kd) sacc[bb] = mm::mma(kreg[BUF][bb * KD + kd], qop[kd], sacc[bb]);
        }
        // Value (bb, e) of this lane: query row n, key j0 + 32 (bb / 2) + 8 gq + 4 (bb % 2) + e.
        const bool full = fa_tile_full(g, 0, rows - 1, j0, DC_BN);
        float sv[16];
        float mx = -INFINITY;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + 32 * (bb >> 1) + 8 * gq + 4 * (bb & 1) + e;
                float x = sacc[bb][e] * sl2;
                if (AL == 1) x = fmaf(slope2, float(j - n - aoff), x);
                if (AL == 2) {
                    const float dd = float(n + off - j);
                    x -= slope2 * copysignf(__builtin_amdgcn_sqrtf(fabsf(dd)), dd);
                }
                if (!full) x = (j >= row_lo && j <= row_hi) ? x : -INFINITY;
                sv[4 * bb + e] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // Rescale only when the row maximum grows by more than 2^8 (as in the forward kernels).
        const bool need = mx > m_run + 8.f;
        const float alpha = need ? exp2f(m_run - mx) : 1.f;
        m_run = need ? mx : m_run;
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float p[16];
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
            ls += p[i];
        }
        l_run = fmaf(l_run, alpha, ls);
        if (__any(need)) {
            // O rows are 4 gq + e: their factors live in lanes 4 gq + e.
            float ar[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ar[e] = __shfl(alpha, 4 * gq + e);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 4; ++e) oacc[db][e] *= ar[e];
        }
        u32x4 pop[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const float* lo = p + 8 * kk;   // block 2 kk: keys 32 kk + 8 gq + 0..3
            const float* hi = p + 8 * kk + 4;   // block 2 kk + 1: keys 32 kk + 8 gq + 4..7
            pop[kk] = u32x4{io::pack(lo[0], lo[1]), io::pack(lo[2], lo[3]), io::pack(hi[0], hi[1]),
                            io::pack(hi[2], hi[3])};
        }
        const char* vb = vbuf + BUF * TILE_U4 * 16;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(vb + 32 * kk * ROW_B + v_rd[0][db]));
                const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(vb + 32 * kk * ROW_B + v_rd[1][db]));
                const u32x4 vop = {__builtin_bit_cast(u32x2, x0)[0], __builtin_bit_cast(u32x2, x0)[1],
                                   __builtin_bit_cast(u32x2, x1)[0], __builtin_bit_cast(u32x2, x1)[1]};
                oacc[db] = mm::mma(pop[kk], vop, oacc[db]);
            }
        }
    };

    using b0 = std::integral_constant<int, 0>;
    using b1 = std::integral_constant<int, 1>;
    const int first = t0 + wave;
    const int cnt = first < t1 ? (t1 - first + 3) / 4 : 0;
    auto step = [&](auto buf_tag, int i) __attribute__((always_inline)) {
        constexpr int BUF = decltype(buf_tag)::value;
        issue(std::integral_constant<int, 1 - BUF>{}, first + 4 * (i + 1));
        __builtin_amdgcn_s_waitcnt(fa_vmcnt64(NK + NV));   // tile i's K registers and V tile landed
        asm volatile("" ::: "memory");
        compute(buf_tag, first + 4 * i);
    };
    if (cnt > 0) {
        issue(b0{}, first);
        int i = 0;
        for (; i + 2 <= cnt; i += 2) {
            step(b0{}, i);
            step(b1{}, i + 1);
        }
        if (i < cnt) step(b0{}, i);
        __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the loop
    }

    // Row statistics of this wave: l summed over the four lane groups (m is already shared).
    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);

    // Combine the four waves in LDS (the V buffers are free once every wave is past its loop).
    __syncthreads();
    float* cm = reinterpret_cast<float*>(lds_v);   // [4][16] m, then [4][16] l, then [4][16][D] O
    float* cl = cm + 4 * DC_ROWS;
    float* co = cl + 4 * DC_ROWS;
    if (gq == 0) {
        cm[wave * DC_ROWS + n] = m_run;
        cl[wave * DC_ROWS + n] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) co[(wave * DC_ROWS + 4 * gq + e) * D + 16 * db + n] = oacc[db][e];
    __syncthreads();
    for (int idx = threadIdx.x; idx < rows * D; idx += DC_THREADS) {
        const int r = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, cm[ww * DC_ROWS + r]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const float f = exp2f(cm[ww * DC_ROWS + r] - M);
                L = fmaf(cl[ww * DC_ROWS + r], f, L);
                O = fmaf(co[(ww * DC_ROWS + r) * D + d], f, O);
            }
        }
        const float o = L > 0.f ? O / L : 0.f;
        const float lse2 = L > 0.f ? M + log2f(L) : -INFINITY;
        if (wk.ns == 1) {
            uint16_t* op = static_cast<uint16_t*>(a.o) + b * a.q_bs + h * a.q_hs + (int64_t(g.q_start) + r) * a.q_rs;
            const uint32_t pk = io::pack(o, 0.f);
            op[d] = uint16_t(pk & 0xffffu);
            if (d == 0) a.lse[b * a.lse_bs + h * a.lse_hs + g.q_start + r] = lse2 * kLn2;
        } else {
            const int64_t slot = int64_t(wk.base + split) * a.N + h;
            dc.o_part[(slot * DC_ROWS + r) * D + d] = o;
            if (d == 0) dc.lse_part[slot * DC_ROWS + r] = lse2;
        }
    }
}

// Combines the splits of fa_decode_split: one workgroup per (batch, head), which returns at
// once when the batch has one split (fa_decode_split wrote its output); thread t takes row
// t / 16 and D / 16 consecutive columns, so every row and column is merged at once and each
// thread's loads over the splits are independent of one another.
template <typename T, int D>
__global__ __launch_bounds__(256) void fa_decode_merge(const fa_kargs a, const fa_decode_args dc) {
    constexpr int CPT = D / 16;   // columns per thread
    const int bh = blockIdx.x;
    const int h = bh % a.N, b = bh / a.N;
    int ns = dc.n_split, base = b * dc.n_split;
    if (dc.batch) {
        base = dc.batch[2 * b];
        ns = dc.batch[2 * b + 1];
    }
    if (ns <= 1) return;
    const fa_geom g = fa_geom_of(a, b);
    const int rows = min(g.sq, DC_ROWS);
    const int r = threadIdx.x >> 4, c0 = (threadIdx.x & 15) * CPT;
    if (r >= rows) return;
    // Split sp's partial result is slot (base + sp) * N + h: slots of one (batch, head) lie
    // N * 16 rows apart.
    const int64_t stride = int64_t(a.N) * DC_ROWS;
    const float* lp = dc.lse_part + int64_t(base) * stride + int64_t(h) * DC_ROWS + r;
    const float* opp = dc.o_part + (int64_t(base) * stride + int64_t(h) * DC_ROWS + r) * D + c0;
    float M = -INFINITY;
#pragma unroll 8
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, lp[sp * stride]);
    float L = 0.f;
    float O[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) O[j] = 0.f;
    if (M != -INFINITY) {
#pragma unroll 4
        for (int sp = 0; sp < ns; ++sp) {
            const float f = exp2f(lp[sp * stride] - M);
            L += f;
            const float4* src = reinterpret_cast<const float4*>(opp + sp * stride * D);
#pragma unroll
            for (int j = 0; j < CPT / 4; ++j) {
                const float4 x = src[j];
                O[4 * j + 0] = fmaf(x.x, f, O[4 * j + 0]);
                O[4 * j + 1] = fmaf(x.y, f, O[4 * j + 1]);
                O[4 * j + 2] = fmaf(x.z, f, O[4 * j + 2]);
                O[4 * j + 3] = fmaf(x.w, f, O[4 * j + 3]);
            }
        }
    }
    const int64_t qrow = int64_t(g.q_start) + r;
    T* op = static_cast<T*>(a.o) + b * a.q_bs + h * a.q_hs + qrow * a.q_rs + c0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) op[j] = T(L > 0.f ? O[j] / L : 0.f);
    if (c0 == 0) a.lse[b * a.lse_bs + h * a.lse_hs + qrow] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------------------------------
// Generic kernel: fp32 arithmetic, any dtype, D <= DMAX.
// ------------------------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ float to_f32(T x) {
    return float(x);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x) {
    return T(x);
}

constexpr int GN_BM = FA_GEN_BM;   // 64 query rows per workgroup (one wave)
constexpr int GN_BN = FA_GEN_BN;   // 16 keys per tile

template <typename T, int DMAX>
// alibi: 0 none, 1 linear (right- or left-aligned per a.alibi_left), 2 square root.
__global__ __launch_bounds__(GN_BM) void fa_fwd_generic(const fa_kargs a, int dense, int alibi) {
    // Q rows of this workgroup (padded by one float so each thread's row starts on its own
    // bank) and one K/V tile, all in fp32. Only the O accumulator lives in registers.
    __shared__ float qs[GN_BM][DMAX + 1];
    __shared__ float ks[GN_BN][DMAX];
    __shared__ float vs[GN_BN][DMAX];
    __shared__ int64_t roff[GN_BN];   // paged K / V: element offset of each key row of the tile
    const int tid = threadIdx.x;
    const int D = a.D;
    int b, h, qt;
    fa_geom g;
    fa_decode_item(a, b, h, qt, g);
    const int i0 = qt * GN_BM;
    const int i_last = min(i0 + GN_BM, g.sq) - 1;
    const fa_kv_range kr = fa_tile_kv_range(g, i0, i_last, GN_BN);
    const T* qp = static_cast<const T*>(a.q) + b * a.q_bs + h * a.q_hs + int64_t(g.q_start) * a.q_rs;
    const T* kp = static_cast<const T*>(a.k) + b * a.kv_bs + h * a.kv_hs + int64_t(g.kv_start) * a.kv_rs;
    const T* vp = static_cast<const T*>(a.v) + b * a.kv_bs + h * a.kv_hs + int64_t(g.kv_start) * a.kv_rs;

    for (int e = tid; e < GN_BM * DMAX; e += GN_BM) {
        const int r = e / DMAX, d = e % DMAX;
        const int i = i0 + r;
        qs[r][d] = (i < g.sq && d < D) ? to_f32(qp[int64_t(i) * a.q_rs + d]) : 0.f;
    }
    const int row = i0 + tid;
    const bool row_ok = row < g.sq;
    float o[DMAX];
#pragma unroll
    for (int d = 0; d < DMAX; ++d) o[d] = 0.f;
    const int row_lo = fa_row_lo(g, row), row_hi = fa_row_hi(g, row);
    const float slope = alibi ? a.slopes[h] : 0.f;
    const float slope2 = slope * kLog2e;
    const int off = g.skv - g.sq;
    const int aoff = a.alibi_left ? 0 : off;   // diagonal of the linear alibi bias
    // Scores are formed relative to the bias at a reference key jr of the row: its last
    // visible key when the slope is >= 0 (where a linear bias is largest), else its first. The
    // bias at jr is the same for every key of the row, so it cancels out of O; it goes into the
    // LSE at the end, in double. The part of each score that fp32 rounds is then only its
    // distance from the reference, which is small where the row's largest terms are: a bias of
    // slope x (a few thousand keys) no longer costs the LSE its last digits.
    const int jr = slope >= 0.f ? row_hi : row_lo;
    const int dr = row + off - jr;   // square-root bias: distance of jr from the diagonal
    double lse_shift = 0.0;
    if (alibi == 1) lse_shift = double(slope) * double(jr - row - aoff);
    if (alibi == 2) lse_shift = -double(slope) * copysign(sqrt(fabs(double(dr))), double(dr));
    const uint8_t* mrow = dense ? a.mask + b * a.m_bs + h * a.m_hs + int64_t(row_ok ? row : 0) * a.m_rs
                                : nullptr;
    float m = -INFINITY, l = 0.f;
    const bool paged = a.block_table != nullptr;
    const int32_t* bt = paged ? a.block_table + b * a.bt_stride : nullptr;
    for (int kt = kr.begin; kt < kr.end; ++kt) {
        const int j0 = kt * GN_BN;
        __syncthreads();   // previous tile fully consumed (and, first time, Q staged)
        if (paged) {
            // Key j lives in page bt[j / block_size], row j % block_size; -1 marks a row that
            // reads as zeros (past Skv, or a page id outside the cache).
            if (tid < GN_BN) {
                const int j = j0 + tid;
                int64_t o = -1;
                if (j < g.skv) {
                    const int pg = bt[j / a.block_size];
                    if (unsigned(pg) < unsigned(a.num_pages))
                        o = int64_t(pg) * a.page_stride + int64_t(j % a.block_size) * a.kv_rs;
                }
                roff[tid] = o;
            }
            __syncthreads();
        }
        for (int e = tid; e < GN_BN * DMAX; e += GN_BM) {
            const int r = e / DMAX, d = e % DMAX;
            const int j = j0 + r;
            const int64_t o = paged ? roff[r] : (j < g.skv ? int64_t(j) * a.kv_rs : -1);
            const bool ok = o >= 0 && d < D;
            ks[r][d] = ok ? to_f32(kp[o + d]) : 0.f;
            vs[r][d] = ok ? to_f32(vp[o + d]) : 0.f;
        }
        __syncthreads();
        // One key at a time: running max m, running sum l, O rescaled when m grows.
#pragma unroll 1
        for (int jj = 0; jj < GN_BN; ++jj) {
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < DMAX; ++d) dot = fmaf(qs[tid][d], ks[jj][d], dot);
            const int j = j0 + jj;
            const bool vis = dense ? (row_ok && j < g.skv && mrow[j] == 0) : (j >= row_lo && j <= row_hi);
            float sv = dot * a.scale_log2;
            if (alibi == 1) {
                sv = fmaf(slope2, float(j - jr), sv);   // bias(j) - bias(jr)
            } else if (alibi == 2) {
                // -slope (f(d) - f(dr)) with f(x) = sign(x) sqrt|x|, d = i + (Skv - Sq) - j. On one
                // side of the diagonal the difference of square roots is (|d| - |dr|) / (sqrt|d| +
                // sqrt|dr|), which keeps its relative accuracy when d is close to dr; across it the
                // two magnitudes add.
                const int d = row + off - j;
                const float qd = sqrtf(fabsf(float(d))), qr = sqrtf(fabsf(float(dr)));
                float diff;
                if ((d >= 0) == (dr >= 0)) {
                    const float den = qd + qr;
                    diff = den > 0.f ? float(abs(d) - abs(dr)) / den : 0.f;
                    diff = d >= 0 ? diff : -diff;
                } else {
                    diff = d >= 0 ? qd + qr : -(qd + qr);
                }
                sv = fmaf(-slope2, diff, sv);
            }
            sv = vis ? sv : -INFINITY;
            const float m_new = fmaxf(m, sv);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = exp2f(m - m_use);
            const float pj = exp2f(sv - m_use);
            l = fmaf(l, alpha, pj);
#pragma unroll
            for (int d = 0; d < DMAX; ++d) o[d] = fmaf(o[d], alpha, pj * vs[jj][d]);
            m = m_new;
        }
    }
    if (row_ok) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        // LSE = bias(jr) + ln 2 (m + log2 l), assembled in double and rounded once.
        a.lse[b * a.lse_bs + h * a.lse_hs + g.q_start + row] =
            l > 0.f ? float(lse_shift + (double(m) + log2(double(l))) * 0.6931471805599453) : -INFINITY;
        T* op = static_cast<T*>(a.o) + b * a.q_bs + h * a.q_hs + (int64_t(g.q_start) + row) * a.q_rs;
#pragma unroll
        for (int d = 0; d < DMAX; ++d)
            if (d < D) op[d] = from_f32<T>(o[d] * inv);
    }
}

// ------------------------------------------------------------------------------------------
// Mask probe kernels: the same mask code, no attention arithmetic.
// ------------------------------------------------------------------------------------------

__global__ void fa_probe_rows(const fa_kargs a, int64_t* counts, int dense) {
    const int b = blockIdx.x, h = blockIdx.y;
    const fa_geom g = fa_geom_of(a, b);
    for (int i = threadIdx.x; i < g.sq; i += blockDim.x) {
        int64_t cnt = 0;
        if (dense) {
            const uint8_t* mrow = a.mask + b * a.m_bs + h * a.m_hs + int64_t(i) * a.m_rs;
            for (int j = 0; j < g.skv; ++j) cnt += mrow[j] == 0;
        } else {
            const int lo = fa_row_lo(g, i), hi = fa_row_hi(g, i);
            cnt = hi >= lo ? hi - lo + 1 : 0;
        }
        counts[b * a.lse_bs + h * a.lse_hs + g.q_start + i] = cnt;
    }
}

__global__ void fa_probe_tiles(const fa_kargs a, uint8_t* tile_class, int64_t n_kv_max, int bm,
                               int bn) {
    const int qt = blockIdx.x, b = blockIdx.y;
    const fa_geom g = fa_geom_of(a, b);
    const int nqt = (g.sq + bm - 1) / bm;
    if (qt >= nqt) return;
    int64_t r = qt;
    for (int bb = 0; bb < b; ++bb) r += (fa_geom_of(a, bb).sq + bm - 1) / bm;
    const int i0 = qt * bm, i1 = min(i0 + bm, g.sq) - 1;
    const fa_kv_range kr = fa_tile_kv_range(g, i0, i1, bn);
    const int nkv = (g.skv + bn - 1) / bn;
    for (int kt = threadIdx.x; kt < n_kv_max; kt += blockDim.x) {
        uint8_t cls;
        if (kt >= nkv) cls = 3;
        else if (kt < kr.begin || kt >= kr.end) cls = 0;
        else cls = fa_tile_full(g, i0, i1, kt * bn, bn) ? 2 : 1;
        tile_class[r * n_kv_max + kt] = cls;
    }
}

// ------------------------------------------------------------------------------------------
// Dense mask (sparse mode 1) pre-pass for the ping-pong kernel. "sparseMode介绍", section
// sparseMode=1, hands the kernel a complete attenMask (non-zero = masked). The pre-pass reads it
// once and, per mask slice (batch or 1, head or 1), q tile of 256 rows and kv tile of 64 keys:
//  * packs the tile's mask bits in the order the kernel's lanes consume them: lane l of wave w
//    holds query row 32 w + l % 32 and, in bit e, key 32 (e / 16) + 8 ((e / 4) % 4) + 4 (l / 32)
//    + e % 4 (1 = hidden: masked, past Skv, or a row past Sq), so a lane reads one dword;
//  * classifies the tile: any visible entry, and per 32-row block whether every entry is
//    visible (that wave then skips per-element masking);
// then lists, per q tile, the kv tiles with a visible entry. The kernel loads no other tile.
// ------------------------------------------------------------------------------------------

struct fa_mask_args {
    const uint8_t* mask;
    int64_t m_bs, m_hs, m_rs;   // element strides of the mask (0 for a broadcast dimension)
    int32_t sq, skv;
    int32_t nqt, nkt;           // q tiles (256 rows) and kv tiles (64 keys) per slice
    int32_t m_heads;            // heads of the mask (N, or 1 when broadcast)
    uint16_t* cls;              // [slices, nqt, nkt]: bit 0 any visible, bits 8-15 full per block
    uint32_t* lists;            // [slices, nqt, 1 + nkt]: count, then kt | full bits << 24
    uint32_t* bits;             // [slices, nqt, nkt, 512]
    int32_t* perm;              // [slices, nqt]: q tiles in launch order (most visited tiles first)
};

constexpr int MC_TILES = 4;   // kv tiles per classify workgroup

// Hidden bits (1 = masked) of four mask bytes: bit c for byte c.
__device__ __forceinline__ uint32_t fa_nonzero_bytes(uint32_t x) {
    const uint32_t t = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;   // bit 7 of each byte: byte != 0
    return ((t >> 7) & 1u) | ((t >> 14) & 2u) | ((t >> 21) & 4u) | ((t >> 28) & 8u);
}

// One 256-thread workgroup per (MC_TILES kv tiles, q tile, slice); thread r takes row r of the
// q tile. ALIGNED: rows start on 16-byte boundaries (Skv % 16 == 0 and an aligned base), so a
// row's 64 bytes of a tile are four 16-byte loads; otherwise bytes are read one by one.
template <bool ALIGNED>
__global__ __launch_bounds__(256) void fa_mask_classify(const fa_mask_args m) {
    __shared__ uint32_t red[MC_TILES][8];   // per tile and 32-row block: bit 0 any visible, bit 1 all
    const int qt = blockIdx.y, ms = blockIdx.z;
    const int kt0 = blockIdx.x * MC_TILES;
    const int rho = threadIdx.x, lane = rho & 63, wv = rho >> 6;
    const int row = qt * FA_PP_BM + rho;
    const bool row_ok = row < m.sq;
    const uint8_t* mrow = m.mask + int64_t(ms / m.m_heads) * m.m_bs + int64_t(ms % m.m_heads) * m.m_hs +
                          int64_t(row_ok ? row : 0) * m.m_rs;
    const int64_t tile0 = (int64_t(ms) * m.nqt + qt) * m.nkt;
    for (int i = 0; i < MC_TILES; ++i) {
        const int kt = kt0 + i;
        if (kt >= m.nkt) break;
        const int j0 = kt * FA_PP_BN;
        // hid[hl], bit 4 (q / 2) + c: key 4 q + c of the tile (q = 0..15 its 4-byte words; word
        // q belongs to lane half hl = q % 2).
        uint32_t hid[2] = {0xFFFFFFFFu, 0xFFFFFFFFu};
        if (row_ok) {
            uint32_t w[16];
            if constexpr (ALIGNED) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    u32x4 x = {0u, 0u, 0u, 0u};
                    if (j0 + 16 * c < m.skv) x = *reinterpret_cast<const u32x4*>(mrow + j0 + 16 * c);
                    w[4 * c + 0] = x[0]; w[4 * c + 1] = x[1]; w[4 * c + 2] = x[2]; w[4 * c + 3] = x[3];
                }
            } else {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    uint32_t x = 0;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int j = j0 + 4 * q + c;
                        x |= uint32_t(j < m.skv ? mrow[j] : 0) << (8 * c);
                    }
                    w[q] = x;
                }
            }
            hid[0] = hid[1] = 0u;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int in = m.skv - (j0 + 4 * q);   // keys of this word inside the sequence
                const uint32_t past = in >= 4 ? 0u : (0xFu << (in > 0 ? in : 0)) & 0xFu;
                hid[q & 1] |= (fa_nonzero_bytes(w[q]) | past) << (4 * (q >> 1));
            }
        }
        uint32_t* dst = m.bits + (tile0 + kt) * 512 + (rho >> 5) * 64 + (rho & 31);
        dst[0] = hid[0];
        dst[32] = hid[1];
        const bool any = row_ok && (hid[0] != 0xFFFFFFFFu || hid[1] != 0xFFFFFFFFu);
        const bool all = !row_ok || (hid[0] == 0u && hid[1] == 0u);
        const uint64_t ba = __ballot(any), bf = __ballot(all);
        if (lane == 0) {
            red[i][2 * wv] = (uint32_t(ba) != 0u ? 1u : 0u) | (uint32_t(bf) == 0xFFFFFFFFu ? 2u : 0u);
            red[i][2 * wv + 1] = (uint32_t(ba >> 32) != 0u ? 1u : 0u) | (uint32_t(bf >> 32) == 0xFFFFFFFFu ? 2u : 0u);
        }
    }
    __syncthreads();
    if (rho < MC_TILES && kt0 + rho < m.nkt) {
        uint32_t any = 0u, full = 0u;
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
            any |= red[rho][blk] & 1u;
            full |= ((red[rho][blk] >> 1) & 1u) << blk;
        }
        m.cls[tile0 + kt0 + rho] = uint16_t(any | (full << 8));
    }
}

// One wave per (q tile, slice): the kv tiles with a visible entry, in order.
__global__ __launch_bounds__(64) void fa_mask_compact(const fa_mask_args m) {
    const int qt = blockIdx.x, ms = blockIdx.y, lane = threadIdx.x;
    const int64_t r = int64_t(ms) * m.nqt + qt;
    const uint16_t* c = m.cls + r * m.nkt;
    uint32_t* rec = m.lists + r * (m.nkt + 1);
    int base = 0;
    for (int k0 = 0; k0 < m.nkt; k0 += 64) {
        const int kt = k0 + lane;
        const uint32_t v = kt < m.nkt ? c[kt] : 0u;
        const uint64_t bal = __ballot(v & 1u);
        if (v & 1u) rec[1 + base + __popcll(bal & ((uint64_t(1) << lane) - 1))] = uint32_t(kt) | ((v >> 8) << 24);
        base += __popcll(bal);
    }
    if (lane == 0) rec[0] = uint32_t(base);
}

// Launch order of each slice's q tiles: most visited kv tiles first (ties by q tile), so the
// longest work items start first and the short ones fill the end. One workgroup per slice ranks
// every q tile against the others; past FA_ORDER_MAX q tiles the order stays the identity.
constexpr int FA_ORDER_MAX = 4096;

__global__ __launch_bounds__(256) void fa_mask_order(const fa_mask_args m) {
    __shared__ uint32_t cnt[FA_ORDER_MAX];
    const int ms = blockIdx.x;
    int32_t* perm = m.perm + int64_t(ms) * m.nqt;
    if (m.nqt > FA_ORDER_MAX) {
        for (int i = threadIdx.x; i < m.nqt; i += blockDim.x) perm[i] = i;
        return;
    }
    for (int i = threadIdx.x; i < m.nqt; i += blockDim.x) cnt[i] = m.lists[(int64_t(ms) * m.nqt + i) * (m.nkt + 1)];
    __syncthreads();
    for (int i = threadIdx.x; i < m.nqt; i += blockDim.x) {
        const uint32_t c = cnt[i];
        int rank = 0;
        for (int j = 0; j < m.nqt; ++j) rank += (cnt[j] > c || (cnt[j] == c && j < i)) ? 1 : 0;
        perm[rank] = i;
    }
}

// Mask probe of mode 1: tile classes of every (batch, head, q tile) from the pre-pass.
__global__ void fa_probe_tiles_dense(const fa_mask_args m, uint8_t* tile_class, int64_t n_kv_max, int N,
                                     int bcast_b, int bcast_h) {
    const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int ms = (bcast_b ? 0 : b) * m.m_heads + (bcast_h ? 0 : h);
    const uint16_t* c = m.cls + (int64_t(ms) * m.nqt + qt) * m.nkt;
    uint8_t* out = tile_class + ((int64_t(b) * N + h) * m.nqt + qt) * n_kv_max;
    for (int kt = threadIdx.x; kt < n_kv_max; kt += blockDim.x) {
        uint8_t cls = 3;
        if (kt < m.nkt) cls = !(c[kt] & 1u) ? 0 : ((c[kt] >> 8) == 0xFFu ? 2 : 1);
        out[kt] = cls;
    }
}

// ------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------

fa_kargs make_kargs(const fa_plan& p, const void* q, const void* k, const void* v, void* out,
                    float* lse, const float* slopes, const uint8_t* mask, void* workspace,
                    float scale) {
    fa_kargs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = out;
    a.lse = lse;
    a.slopes = slopes;
    a.mask = mask;
    if (p.table) {
        a.geoms = static_cast<const fa_geom*>(workspace);
        a.items = reinterpret_cast<const int32_t*>(static_cast<const char*>(workspace) + p.ws_items_offset);
    }
    a.geom0 = p.geom0;
    a.q_bs = p.q_bs; a.q_hs = p.q_hs; a.q_rs = p.q_rs;
    a.kv_bs = p.kv_bs; a.kv_hs = p.kv_hs; a.kv_rs = p.kv_rs;
    a.lse_bs = p.lse_bs; a.lse_hs = p.lse_hs;
    a.m_bs = p.m_bs; a.m_hs = p.m_hs; a.m_rs = p.m_rs;
    a.B = p.B;
    a.N = p.N;
    a.D = p.D;
    a.n_qtiles_fixed = p.n_qtiles_fixed;
    a.reverse_qt = p.reverse_qt;
    a.xcd_major = p.xcd_major;
    a.scale_log2 = scale * kLog2e;
    a.page_stride = p.page_stride;
    a.bt_stride = p.bt_stride;
    a.block_size = p.block_size;
    a.log2_block_size = p.log2_block_size;
    a.num_pages = p.num_pages;
    if (p.dense_tiles && p.ws_bytes > 0) {
        char* ws = static_cast<char*>(workspace);
        a.tile_list = reinterpret_cast<const uint32_t*>(ws + p.ws_list_offset);
        a.tile_bits = reinterpret_cast<const uint32_t*>(ws + p.ws_bits_offset);
        a.tile_perm = reinterpret_cast<const int32_t*>(ws + p.ws_perm_offset);
        a.dense_nqt = p.dense_nqt;
        a.dense_nkt = p.dense_nkt;
        a.m_heads = p.mask_heads;
        a.m_bcast_b = p.m_bcast_b;
        a.m_bcast_h = p.m_bcast_h;
    }
    return a;
}

fa_mask_args make_mask_args(const fa_plan& p, const uint8_t* mask, void* workspace) {
    fa_mask_args m{};
    char* ws = static_cast<char*>(workspace);
    m.mask = mask;
    m.m_bs = p.m_bs;
    m.m_hs = p.m_hs;
    m.m_rs = p.m_rs;
    m.sq = p.geom0.sq;
    m.skv = p.geom0.skv;
    m.nqt = p.dense_nqt;
    m.nkt = p.dense_nkt;
    m.m_heads = p.mask_heads;
    m.cls = reinterpret_cast<uint16_t*>(ws + p.ws_cls_offset);
    m.lists = reinterpret_cast<uint32_t*>(ws + p.ws_list_offset);
    m.bits = reinterpret_cast<uint32_t*>(ws + p.ws_bits_offset);
    m.perm = reinterpret_cast<int32_t*>(ws + p.ws_perm_offset);
    return m;
}

// The dense-mask pre-pass (classify, then list). with_lists = false: classes and bits only.
void launch_mask_prepass(const fa_mask_args& m, int slices, bool with_lists, hipStream_t s) {
    const bool aligned = (m.skv % 16) == 0 && (reinterpret_cast<uintptr_t>(m.mask) % 16) == 0;
    const dim3 grid(unsigned((m.nkt + MC_TILES - 1) / MC_TILES), unsigned(m.nqt), unsigned(slices));
    if (aligned) fa_mask_classify<true><<<grid, dim3(256), 0, s>>>(m);
    else fa_mask_classify<false><<<grid, dim3(256), 0, s>>>(m);
    if (with_lists) {
        fa_mask_compact<<<dim3(unsigned(m.nqt), unsigned(slices)), dim3(64), 0, s>>>(m);
        fa_mask_order<<<dim3(unsigned(slices)), dim3(256), 0, s>>>(m);
    }
}

// Compute units of the current device (cached per device).
int device_cus() {
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

// FA_PERSIST=1 runs the persistent kernel for the ping-pong kernel's problems without a dense
// mask or paged K/V.
bool persist_enabled() {
    const char* e = std::getenv("FA_PERSIST");
    return e && e[0] == '1';
}

// The persistent schedule (fa_fwd_ps.hip): one workgroup per compute unit, lists per XCD when
// the (batch, head) pairs split evenly over the 8 XCDs. Returns the grid size (0: not used).
unsigned persistent_schedule(const fa_plan& p, fa_ps_args* ps) {
    int cus = device_cus();
    if (cus < 8) return 0;
    // FA_PS_SLOTS: workgroups per launch instead of the compute unit count (comparisons).
    if (const char* e = std::getenv("FA_PS_SLOTS")) cus = std::max(8, std::atoi(e));
    *ps = fa_ps_args{};
    const int64_t pairs = int64_t(p.B) * p.N;
    ps->N = p.N;
    ps->reverse_qt = p.reverse_qt;
    ps->table = p.table ? 1 : 0;
    fa_magic_divisor(uint32_t(p.N), &ps->n_mul, &ps->n_shr);
    unsigned grid;
    if (!p.table && p.xcd_major) {
        ps->xcd = 1;
        ps->nq = p.n_qtiles_fixed;
        const int64_t n_list = pairs / 8 * p.n_qtiles_fixed;
        if (n_list >= (int64_t(1) << 31)) return 0;
        ps->n_list = int32_t(n_list);
        ps->W = int32_t(std::min<int64_t>(cus / 8, n_list));
        grid = unsigned(8 * ps->W);
    } else {
        ps->xcd = 0;
        ps->nq = p.table ? 1 : p.n_qtiles_fixed;
        const int64_t n_list = p.table ? p.n_items * p.N : pairs * p.n_qtiles_fixed;
        if (n_list >= (int64_t(1) << 31)) return 0;
        ps->n_list = int32_t(n_list);
        ps->W = int32_t(std::min<int64_t>(cus, n_list));
        grid = unsigned(ps->W);
    }
    fa_magic_divisor(uint32_t(std::max(ps->nq, 1)), &ps->nq_mul, &ps->nq_shr);
    return grid;
}

bool log_enabled() {
    const char* e = std::getenv("FA_LOG");
    return e && e[0] == '1';
}

fa_status upload_tables(const fa_plan& p, void* workspace, hipStream_t stream) {
    if (!p.table || p.ws_table_bytes == 0) return FA_OK;
    // The image is pageable host memory; hipMemcpyAsync stages it before returning.
    std::vector<unsigned char> image;
    fa_plan_workspace_image(p, &image);
    if (hipMemcpyAsync(workspace, image.data(), image.size(), hipMemcpyHostToDevice, stream) != hipSuccess)
        return FA_ERR_HIP;
    return FA_OK;
}

template <int D, bool BF>
void launch_mfma32_d(const fa_kargs& a, int al, bool dense, dim3 grid, hipStream_t s) {
    const dim3 block(MF_THREADS);
    switch (al * 2 + (dense ? 1 : 0)) {
        case 0: fa_fwd_mfma<D, BF, 0, false><<<grid, block, 0, s>>>(a); break;
        case 1: fa_fwd_mfma<D, BF, 0, true><<<grid, block, 0, s>>>(a); break;
        case 2: fa_fwd_mfma<D, BF, 1, false><<<grid, block, 0, s>>>(a); break;
        case 3: fa_fwd_mfma<D, BF, 1, true><<<grid, block, 0, s>>>(a); break;
        case 4: fa_fwd_mfma<D, BF, 2, false><<<grid, block, 0, s>>>(a); break;
        default: fa_fwd_mfma<D, BF, 2, true><<<grid, block, 0, s>>>(a); break;
    }
}

template <int D, bool BF>
void launch_pp_d(const fa_kargs& a, int al, bool dense, bool edge, dim3 grid, hipStream_t s) {
    const dim3 block(PP_THREADS);
    switch (al * 2 + (dense ? 1 : 0)) {
        case 0:
            if (edge) fa_fwd_pp<D, BF, 0, false, false, true><<<grid, block, 0, s>>>(a);
            else fa_fwd_pp<D, BF, 0, false><<<grid, block, 0, s>>>(a);
            break;
        case 1: fa_fwd_pp<D, BF, 0, true><<<grid, block, 0, s>>>(a); break;
        case 2: fa_fwd_pp<D, BF, 1, false><<<grid, block, 0, s>>>(a); break;
        case 3: fa_fwd_pp<D, BF, 1, true><<<grid, block, 0, s>>>(a); break;
        case 4: fa_fwd_pp<D, BF, 2, false><<<grid, block, 0, s>>>(a); break;
        default: fa_fwd_pp<D, BF, 2, true><<<grid, block, 0, s>>>(a); break;
    }
}

template <typename T>
void launch_generic_t(const fa_kargs& a, int D, int alibi, bool dense, dim3 grid, hipStream_t s) {
    const dim3 block(GN_BM);
    if (D <= 32) fa_fwd_generic<T, 32><<<grid, block, 0, s>>>(a, dense, alibi);
    else if (D <= 64) fa_fwd_generic<T, 64><<<grid, block, 0, s>>>(a, dense, alibi);
    else fa_fwd_generic<T, 128><<<grid, block, 0, s>>>(a, dense, alibi);
}

template <int D, bool BF, bool PAGED>
void launch_decode_d(const fa_kargs& a, const fa_decode_args& dc, int al, dim3 grid, hipStream_t s) {
    const dim3 block(DC_THREADS);
    switch (al) {
        case 0: fa_decode_split<D, BF, 0, PAGED><<<grid, block, 0, s>>>(a, dc); break;
        case 1: fa_decode_split<D, BF, 1, PAGED><<<grid, block, 0, s>>>(a, dc); break;
        default: fa_decode_split<D, BF, 2, PAGED><<<grid, block, 0, s>>>(a, dc); break;
    }
}

template <int D, bool BF>
void launch_pp_paged_d(const fa_kargs& a, int al, bool edge, dim3 grid, hipStream_t s) {
    const dim3 block(PP_THREADS);
    switch (al) {
        case 0:
            if (edge) fa_fwd_pp<D, BF, 0, false, true, true><<<grid, block, 0, s>>>(a);
            else fa_fwd_pp<D, BF, 0, false, true><<<grid, block, 0, s>>>(a);
            break;
        case 1: fa_fwd_pp<D, BF, 1, false, true><<<grid, block, 0, s>>>(a); break;
        default: fa_fwd_pp<D, BF, 2, false, true><<<grid, block, 0, s>>>(a); break;
    }
}

// Shared by fa_fwd and fa_fwd_paged: k / v are the tensors or the caches (block_table set).
fa_status run_fwd(const fa_call& c, const void* q, const void* k, const void* v, void* out, float* softmax_lse,
                  const float* alibi_slopes, const uint8_t* atten_mask, const int32_t* block_table,
                  void* workspace, size_t workspace_bytes, void* stream) {
    fa_plan p;
    fa_status st = fa_make_plan(c, true, &p);
    if (st != FA_OK) return st;
    if (!p.empty) {
        if (!q || !out || !softmax_lse) return FA_ERR_NULLPTR;
        if (p.kv_total > 0 && (!k || !v)) return FA_ERR_NULLPTR;
        if (p.paged && p.kv_total > 0 && !block_table) return FA_ERR_NULLPTR;
    }
    if (p.ws_bytes > 0) {
        if (!workspace) return FA_ERR_NULLPTR;
        if (workspace_bytes < p.ws_bytes) return FA_ERR_WORKSPACE;
    }
    if (p.empty) return FA_OK;
    const int64_t nblocks = p.n_items * p.N;
    if (nblocks >= (int64_t(1) << 31)) return FA_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (log_enabled()) {
        std::fprintf(stderr,
                     "[fa] kernel=%s bm=%d bn=%d items/head=%lld blocks=%lld kv tiles visited/full/"
                     "dense=%lld/%lld/%lld table=%d reverse=%d xcd_major=%d ws=%zu paged=%d\n",
                     p.kernel == FA_KERNEL_PP ? "pingpong"
                     : p.kernel == FA_KERNEL_MFMA32 ? "mfma32"
                     : p.kernel == FA_KERNEL_DECODE ? "decode" : "generic",
                     p.bm, p.bn,
                     (long long)p.n_items, (long long)nblocks, (long long)p.kv_tiles_visited,
                     (long long)p.kv_tiles_full, (long long)p.kv_tiles_total, int(p.table),
                     p.reverse_qt, p.xcd_major, p.ws_bytes, int(p.paged));
    }
    st = upload_tables(p, workspace, s);
    if (st != FA_OK) return st;
    if (p.dense_tiles && p.ws_bytes > 0) {
        (void)hipGetLastError();
        launch_mask_prepass(make_mask_args(p, atten_mask, workspace), p.mask_slices, true, s);
        if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    }
    fa_kargs a = make_kargs(p, q, k, v, out, softmax_lse, alibi_slopes, atten_mask, workspace, c.scale);
    a.alibi_left = c.alibi_mode == FA_ALIBI_LEFT ? 1 : 0;
    a.block_table = p.paged ? block_table : nullptr;
    const dim3 grid(static_cast<unsigned>(nblocks));
    const int alibi = alibi_slopes == nullptr ? 0 : (c.alibi_mode == FA_ALIBI_SQRT ? 2 : 1);
    const bool dense = c.sparse_mode == 1;
    const int32_t dtype = c.dims->dtype;
    (void)hipGetLastError();
    if (p.kernel == FA_KERNEL_DECODE) {
        fa_decode_args dc{};
        dc.n_split = p.n_split;
        if (p.table)
            dc.batch = reinterpret_cast<const int32_t*>(static_cast<const char*>(workspace) + p.ws_dec_batch_offset);
        if (p.dec_merge) {
            dc.o_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.ws_opart_offset);
            dc.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.ws_lse_offset);
        }
        const bool bf = dtype == FA_DTYPE_BF16;
        if (p.D == 128) {
            if (p.paged) {
                if (bf) launch_decode_d<128, true, true>(a, dc, alibi, grid, s);
                else launch_decode_d<128, false, true>(a, dc, alibi, grid, s);
            } else {
                if (bf) launch_decode_d<128, true, false>(a, dc, alibi, grid, s);
                else launch_decode_d<128, false, false>(a, dc, alibi, grid, s);
            }
        } else {
            if (p.paged) {
                if (bf) launch_decode_d<64, true, true>(a, dc, alibi, grid, s);
                else launch_decode_d<64, false, true>(a, dc, alibi, grid, s);
            } else {
                if (bf) launch_decode_d<64, true, false>(a, dc, alibi, grid, s);
                else launch_decode_d<64, false, false>(a, dc, alibi, grid, s);
            }
        }
        if (p.dec_merge) {
            const dim3 mgrid(static_cast<unsigned>(int64_t(p.B) * p.N)), mblock(256);
            if (p.D == 128) {
                if (bf) fa_decode_merge<__bf16, 128><<<mgrid, mblock, 0, s>>>(a, dc);
                else fa_decode_merge<_Float16, 128><<<mgrid, mblock, 0, s>>>(a, dc);
            } else {
                if (bf) fa_decode_merge<__bf16, 64><<<mgrid, mblock, 0, s>>>(a, dc);
                else fa_decode_merge<_Float16, 64><<<mgrid, mblock, 0, s>>>(a, dc);
            }
        }
    } else if (p.kernel == FA_KERNEL_PP && p.paged) {
        const bool bf = dtype == FA_DTYPE_BF16;
        if (p.D == 128) {
            if (bf) launch_pp_paged_d<128, true>(a, alibi, p.edge_skip, grid, s);
            else launch_pp_paged_d<128, false>(a, alibi, p.edge_skip, grid, s);
        } else {
            if (bf) launch_pp_paged_d<64, true>(a, alibi, p.edge_skip, grid, s);
            else launch_pp_paged_d<64, false>(a, alibi, p.edge_skip, grid, s);
        }
    } else if (p.kernel == FA_KERNEL_PP && !dense && persist_enabled() && [&] {
                   fa_ps_args ps;
                   const unsigned g = persistent_schedule(p, &ps);
                   if (g == 0) return false;
                   launch_fwd_ps(a, ps, p.D, dtype == FA_DTYPE_BF16, alibi, g, s);
                   return true;
               }()) {
        // launched above
    } else if (p.kernel == FA_KERNEL_PP) {
        const bool bf = dtype == FA_DTYPE_BF16;
        if (p.D == 128) {
            if (bf) launch_pp_d<128, true>(a, alibi, dense, p.edge_skip, grid, s);
            else launch_pp_d<128, false>(a, alibi, dense, p.edge_skip, grid, s);
        } else {
            if (bf) launch_pp_d<64, true>(a, alibi, dense, p.edge_skip, grid, s);
            else launch_pp_d<64, false>(a, alibi, dense, p.edge_skip, grid, s);
        }
    } else if (p.kernel == FA_KERNEL_MFMA32) {
        const bool bf = dtype == FA_DTYPE_BF16;
        if (p.D == 128) {
            if (bf) launch_mfma32_d<128, true>(a, alibi, dense, grid, s);
            else launch_mfma32_d<128, false>(a, alibi, dense, grid, s);
        } else {
            if (bf) launch_mfma32_d<64, true>(a, alibi, dense, grid, s);
            else launch_mfma32_d<64, false>(a, alibi, dense, grid, s);
        }
    } else {
        switch (dtype) {
            case FA_DTYPE_F32: launch_generic_t<float>(a, p.D, alibi, dense, grid, s); break;
            case FA_DTYPE_F16: launch_generic_t<_Float16>(a, p.D, alibi, dense, grid, s); break;
            default: launch_generic_t<__bf16>(a, p.D, alibi, dense, grid, s); break;
        }
    }
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    return FA_OK;
}

}  // namespace

extern "C" fa_status fa_fwd(const void* q, const void* k, const void* v, void* out,
                            float* softmax_lse, const fa_dims* dims, int32_t layout,
                            int32_t sparse_mode, int64_t pre_tokens, int64_t next_tokens,
                            const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                            const int64_t* prefix, const float* alibi_slopes, int32_t alibi_mode,
                            const uint8_t* atten_mask, const int64_t* mask_bcast, float scale,
                            void* workspace, size_t workspace_bytes, void* stream) {
    fa_call c;
    c.dims = dims;
    c.layout = layout;
    c.sparse_mode = sparse_mode;
    c.pre_tokens = pre_tokens;
    c.next_tokens = next_tokens;
    c.actual_seq_qlen = actual_seq_qlen;
    c.actual_seq_kvlen = actual_seq_kvlen;
    c.prefix = prefix;
    c.has_alibi = alibi_slopes != nullptr;
    c.alibi_mode = alibi_mode;
    c.has_mask = atten_mask != nullptr;
    c.mask_bcast = mask_bcast;
    c.scale = scale;
    return run_fwd(c, q, k, v, out, softmax_lse, alibi_slopes, atten_mask, nullptr, workspace, workspace_bytes,
                   stream);
}

// ------------------------------------------------------------------------------------------
// fa_fwd_noalloc: fa_fwd with the workspace in a fixed device array of this library.
// ------------------------------------------------------------------------------------------

namespace {

// The workspace of fa_fwd_noalloc: one copy per GPU, held until the process ends. In host code
// `scratch` names a host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only that address is
// ever passed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev`, which must be the current device.
fa_status scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

}  // namespace

extern "C" fa_status fa_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                    float* softmax_lse, const fa_dims* dims, int32_t layout,
                                    int32_t sparse_mode, int64_t pre_tokens, int64_t next_tokens,
                                    const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                                    const int64_t* prefix, const float* alibi_slopes, int32_t alibi_mode,
                                    const uint8_t* atten_mask, const int64_t* mask_bcast, float scale,
                                    void* stream) {
    fa_call c;
    c.dims = dims;
    c.layout = layout;
    c.sparse_mode = sparse_mode;
    c.pre_tokens = pre_tokens;
    c.next_tokens = next_tokens;
    c.actual_seq_qlen = actual_seq_qlen;
    c.actual_seq_kvlen = actual_seq_kvlen;
    c.prefix = prefix;
    c.has_alibi = alibi_slopes != nullptr;
    c.alibi_mode = alibi_mode;
    c.has_mask = atten_mask != nullptr;
    c.mask_bcast = mask_bcast;
    c.scale = scale;
    // Validate and size first: a problem whose workspace would not fit is refused before any
    // HIP call.
    fa_plan p;
    const fa_status st = fa_make_plan(c, false, &p);
    if (st != FA_OK) return st;
    if (p.ws_bytes > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (p.ws_bytes > 0) {
        // The stream's device must be the current one: that is the copy of `scratch` whose
        // address hipGetSymbolAddress returns.
        int cur = -1;
        hipDevice_t sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_HIP;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return FA_ERR_HIP;
        if (sdev != cur) return FA_ERR_PARAM_INVALID;
        const fa_status sa = scratch_address(cur, &ws);
        if (sa != FA_OK) return sa;
    }
    return run_fwd(c, q, k, v, out, softmax_lse, alibi_slopes, atten_mask, nullptr, ws,
                   ws ? size_t(FA_NOALLOC_SCRATCH_BYTES) : 0, stream);
}

extern "C" fa_status fa_fwd_paged(const void* q, const void* key_cache, const void* value_cache, void* out,
                                  float* softmax_lse, const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                                  int64_t pre_tokens, int64_t next_tokens, const int64_t* actual_seq_qlen,
                                  const int64_t* actual_seq_kvlen, const int64_t* prefix,
                                  const float* alibi_slopes, int32_t alibi_mode, const uint8_t* atten_mask,
                                  const int64_t* mask_bcast, const fa_paged_kv* paged, float scale,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (!paged) return FA_ERR_NULLPTR;
    fa_call c;
    c.dims = dims;
    c.layout = layout;
    c.sparse_mode = sparse_mode;
    c.pre_tokens = pre_tokens;
    c.next_tokens = next_tokens;
    c.actual_seq_qlen = actual_seq_qlen;
    c.actual_seq_kvlen = actual_seq_kvlen;
    c.prefix = prefix;
    c.has_alibi = alibi_slopes != nullptr;
    c.alibi_mode = alibi_mode;
    c.has_mask = atten_mask != nullptr;
    c.mask_bcast = mask_bcast;
    c.scale = scale;
    c.paged = paged;
    return run_fwd(c, q, key_cache, value_cache, out, softmax_lse, alibi_slopes, atten_mask, paged->block_table,
                   workspace, workspace_bytes, stream);
}

extern "C" fa_status fa_mask_probe(const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                                   int64_t pre_tokens, int64_t next_tokens,
                                   const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                                   const int64_t* prefix, const uint8_t* atten_mask,
                                   const int64_t* mask_bcast, int64_t* row_visible_counts,
                                   uint8_t* tile_class, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    fa_call c;
    c.dims = dims;
    c.layout = layout;
    c.sparse_mode = sparse_mode;
    c.pre_tokens = pre_tokens;
    c.next_tokens = next_tokens;
    c.actual_seq_qlen = actual_seq_qlen;
    c.actual_seq_kvlen = actual_seq_kvlen;
    c.prefix = prefix;
    c.has_mask = atten_mask != nullptr;
    c.mask_bcast = mask_bcast;
    c.check_scale = false;
    fa_plan p;
    fa_status st = fa_make_plan(c, true, &p);
    if (st != FA_OK) return st;
    // Mode 1 has a tile map where the forward runs the dense-mask pre-pass.
    if (sparse_mode == 1 && tile_class && !p.dense_tiles) return FA_ERR_UNSUPPORTED;
    if (!p.empty && !row_visible_counts) return FA_ERR_NULLPTR;
    if (p.ws_bytes > 0) {
        if (!workspace) return FA_ERR_NULLPTR;
        if (workspace_bytes < p.ws_bytes) return FA_ERR_WORKSPACE;
    }
    if (p.empty || p.B == 0) return FA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = upload_tables(p, workspace, s);
    if (st != FA_OK) return st;
    const fa_kargs a = make_kargs(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, atten_mask,
                                  workspace, 1.0f);
    (void)hipGetLastError();
    fa_probe_rows<<<dim3(p.B, p.N), dim3(256), 0, s>>>(a, row_visible_counts, sparse_mode == 1);
    if (sparse_mode == 1) {
        if (tile_class && p.ws_bytes > 0 && p.dense_nqt > 0) {
            const fa_mask_args m = make_mask_args(p, atten_mask, workspace);
            launch_mask_prepass(m, p.mask_slices, false, s);
            fa_probe_tiles_dense<<<dim3(unsigned(p.dense_nqt), unsigned(p.N), unsigned(p.B)), dim3(256), 0, s>>>(
                m, tile_class, p.n_kvtiles_max, p.N, p.m_bcast_b, p.m_bcast_h);
        }
    } else if (tile_class && p.n_kvtiles_max > 0) {
        int64_t max_nqt = 0;
        for (const fa_geom& g : p.geoms) max_nqt = std::max<int64_t>(max_nqt, (g.sq + p.bm - 1) / p.bm);
        if (max_nqt > 0)
            fa_probe_tiles<<<dim3(unsigned(max_nqt), p.B), dim3(256), 0, s>>>(a, tile_class, p.n_kvtiles_max,
                                                                            p.bm, p.bn);
    }
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    return FA_OK;
}

// ------------------------------------------------------------------------------------------
// Exp-throughput calibration. The online softmax evaluates one base-2 exponential per computed
// score (the tiling page's recurrence, with exp rewritten as exp2 of log2(e)-scaled scores);
// on this chip that is v_exp_f32, a transcendental issued at a fraction of the plain VALU rate.
// This kernel issues nothing else in its loop: every thread runs FA_EXP_CHAINS independent
// chains x <- 2^(-x) (the negation is a free source modifier), which converge to the root of
// x = 2^(-x), so the values stay finite and the result can be checked.
// ------------------------------------------------------------------------------------------

constexpr int FA_EXP_CHAINS = 8;
constexpr int FA_EXP_UNROLL = 16;
constexpr int FA_EXP_THREADS = 256;

__global__ __launch_bounds__(FA_EXP_THREADS) void fa_exp2_rate(float* out, int32_t iters) {
    float x[FA_EXP_CHAINS];
#pragma unroll
    for (int c = 0; c < FA_EXP_CHAINS; ++c) x[c] = 0.5f + 0.0625f * float(c) + 0.001f * float(threadIdx.x & 7);
    for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < FA_EXP_UNROLL; ++u) {
#pragma unroll
            for (int c = 0; c < FA_EXP_CHAINS; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < FA_EXP_CHAINS; ++c) s += x[c];
    out[size_t(blockIdx.x) * FA_EXP_THREADS + threadIdx.x] = s;
}

extern "C" fa_status fa_exp2_rate_probe(float* out, int32_t blocks, int32_t iters, int64_t* exps_per_launch,
                                        void* stream) {
    if (!out || !exps_per_launch) return FA_ERR_NULLPTR;
    if (blocks < 1 || iters < 1 || blocks > (1 << 20) || iters > (1 << 20)) return FA_ERR_PARAM_INVALID;
    *exps_per_launch = int64_t(blocks) * FA_EXP_THREADS * iters * FA_EXP_UNROLL * FA_EXP_CHAINS;
    (void)hipGetLastError();
    fa_exp2_rate<<<dim3(unsigned(blocks)), dim3(FA_EXP_THREADS), 0, static_cast<hipStream_t>(stream)>>>(out, iters);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
