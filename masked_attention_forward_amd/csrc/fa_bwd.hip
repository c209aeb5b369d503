// fa_bwd.hip - backward pass of masked attention for gfx950 (dQ, dK, dV) and its C ABI.
//
// The pages define the forward only; the backward is its derivative. With P recomputed from
// Q, K, the bias and the mask of the forward ("sparseMode介绍" sparseMode 0..8, "压缩mask"
// alibi) and the forward's LSE:
//
//     P_ij = exp(scale q_i.k_j + bias_ij - LSE_i) for visible (i, j), else 0
//     Delta_i = sum_d dO_id O_id                  (= sum_j P_ij dP_ij)
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - Delta),   dQ = scale dS K,   dK = scale dS^T Q
//
// Three kernels run in order: fa_bwd_delta (Delta from O and dO), one that owns a block of keys
// and loops over the query tiles that see it (dK, dV), and one that owns a block of query rows
// and loops over the kv tiles it sees (dQ). Every output element is written by exactly one
// workgroup: no atomics, bitwise deterministic.
//
//  * MFMA kernels (fp16 / bf16, D in {64, 128}, every mode but the explicit mask): eight waves
//    own 16 keys (dK dV) or 16 query rows (dQ) each, with 16x16x32 MFMAs. The products whose
//    contraction runs over rows or keys take their left operand straight from the accumulators
//    of the preceding product: tile rows are permuted so that a lane's four values of one
//    16 x 16 block and of its neighbour are the eight consecutive rows (keys) the next MFMA
//    wants (block b, row r holds 32 (b / 2) + 8 (r / 4) + 4 (b % 2) + r % 4). Their right
//    operand (8 consecutive rows of one column) comes from LDS through ds_read_b64_tr_b16.
//  * Generic kernels: any dtype, D <= 128, the explicit mask: one thread per query row (dQ) or
//    per key (dK, dV), fp32 throughout.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "fa_device.h"
#include "fa_mask.h"
#include "fa_plan.h"

namespace {

struct fa_bwd_args {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    const float* lse;
    float* delta;            // laid out like lse (workspace)
    float* lse2;             // lse * log2(e), laid out like lse (workspace)
    const float* slopes;
    const uint8_t* mask;
    const fa_geom* geoms;    // per-batch table (workspace) or nullptr
    fa_geom geom0;
    int64_t q_bs, q_hs, q_rs;
    int64_t kv_bs, kv_hs, kv_rs;
    int64_t lse_bs, lse_hs;
    int64_t m_bs, m_hs, m_rs;
    int32_t B, N, D;
    int32_t n_qt, n_kt;      // 64-row q tiles / 64-key kv tiles of the longest sequence
    int32_t alibi_left;
    int32_t rank_order;      // MFMA kernels: 1 = rank-major block order, 2 = in groups of four pairs (bw_block)
    float scale_log2;        // scale * log2(e)
    float scale;
};

constexpr int BW_THREADS = 256;
constexpr int BW_T = 64;        // rows per q tile, keys per kv tile
constexpr int GB_ROWS = 64;     // generic kernels: threads (rows or keys) per workgroup
constexpr int GB_T = 16;        // generic kernels: staged rows / keys per step

__device__ __forceinline__ fa_geom bw_geom(const fa_bwd_args& a, int b) {
    if (!a.geoms) return a.geom0;
    const fa_geom t = a.geoms[b];
    fa_geom g;
    g.q_start = fa_uniform(t.q_start);
    g.kv_start = fa_uniform(t.kv_start);
    g.sq = fa_uniform(t.sq);
    g.skv = fa_uniform(t.skv);
    g.a = fa_uniform(t.a);
    g.c = fa_uniform(t.c);
    g.f = fa_uniform(t.f);
    g.pad = 0;
    return g;
}

// Query rows [lo, hi] (batch-local) that can see a key in [j0, j1]: lo(i) <= j1 and hi(i) >= j0,
// a superset of the rows with a visible key there (masking removes the rest).
__device__ __forceinline__ void bw_row_range(const fa_geom& g, int j0, int j1, int& lo, int& hi) {
    lo = g.f >= j0 ? 0 : max(0, j0 - g.c);
    hi = min(g.sq - 1, j1 - g.a);
}

// Block w of a launch of pairs x nblk workgroups -> (pair, block). Workgroups go round-robin
// over the 8 XCDs; when the pair count is a multiple of 8, XCD x takes whole pairs x, x + 8, ...
// so every XCD gets the same mix of light and heavy blocks (block b otherwise lands on XCD
// b % 8 for every pair, and under causal masks the work grows with b) and a pair's K / V stay in
// one L2. reverse: hand out the blocks last first (dQ, whose last blocks see the most keys).
__device__ __forceinline__ void bw_block(int w, int pairs, int nblk, bool reverse, bool rank, bool rank_grouped,
                                         int& pair, int& blk) {
    if ((pairs & 7) == 0) {
        const int x = w & 7, s = w >> 3;
        if (rank) {
            // Rank-major: block r of every pair of the XCD, then block r + 1; in groups of four
            // pairs when the XCD's pairs split that way (rank == 2), as the forward does.
            const int ppx = pairs >> 3;
            if (rank_grouped && (ppx & 3) == 0 && ppx > 4) {
                const int gr = s / (4 * nblk), jj = s % (4 * nblk);
                pair = (gr * 4 + (jj & 3)) * 8 + x;
                blk = jj >> 2;
            } else {
                pair = (s % ppx) * 8 + x;
                blk = s / ppx;
            }
        } else {
            pair = (s / nblk) * 8 + x;
            blk = s % nblk;
        }
    } else {
        pair = w / nblk;
        blk = w % nblk;
    }
    if (reverse) blk = nblk - 1 - blk;
}

// Alibi bias in the log2 domain (AL: 1 linear, right- or left-aligned per aoff; 2 square root).
template <int AL>
__device__ __forceinline__ float bw_bias2(float slope2, int i, int j, int off, int aoff) {
    if (AL == 1) return slope2 * float(j - i - aoff);
    if (AL == 2) {
        const float dd = float(i + off - j);
        return -slope2 * copysignf(__builtin_amdgcn_sqrtf(fabsf(dd)), dd);
    }
    return 0.f;
}

template <typename T>
__device__ __forceinline__ float to_f(T x) {
    return float(x);
}

// ------------------------------------------------------------------------------------------
// Delta_i = sum_d dO_id O_id (fp32), one wave per query row.
// ------------------------------------------------------------------------------------------
constexpr int DL_ROWS = BW_THREADS / 64;   // rows per workgroup of fa_bwd_delta

template <typename T>
__global__ __launch_bounds__(BW_THREADS) void fa_bwd_delta(const fa_bwd_args a) {
    const int nrb = (a.n_qt * BW_T + DL_ROWS - 1) / DL_ROWS;
    const int bh = blockIdx.x / nrb;
    const int b = bh / a.N, h = bh % a.N;
    const fa_geom g = bw_geom(a, b);
    const int i = (blockIdx.x % nrb) * DL_ROWS + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (i >= g.sq) return;
    const int64_t ro = b * a.q_bs + h * a.q_hs + (int64_t(g.q_start) + i) * a.q_rs;
    const T* op = static_cast<const T*>(a.o) + ro;
    const T* dp = static_cast<const T*>(a.dout) + ro;
    float s = 0.f;
    for (int d = lane; d < a.D; d += 64) s = fmaf(to_f(op[d]), to_f(dp[d]), s);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (lane == 0) {
        const int64_t li = b * a.lse_bs + h * a.lse_hs + g.q_start + i;
        a.delta[li] = s;
        a.lse2[li] = a.lse[li] * kLog2e;
    }
}

// bf16 / fp16 with D % 8 == 0 and 16-byte aligned rows: 16 lanes per row, 16 bytes per lane and
// load, four rows per wave. O is read only here (non-temporal); dO stays cached for the two
// kernels after this one.
constexpr int DLV_ROWS = (BW_THREADS / 64) * 4;   // rows per workgroup of fa_bwd_delta_v

template <typename T>
__device__ __forceinline__ float half_f(uint32_t bits) {
    return to_f(__builtin_bit_cast(T, uint16_t(bits)));
}

template <typename T>
__global__ __launch_bounds__(BW_THREADS) void fa_bwd_delta_v(const fa_bwd_args a) {
    const int nrb = (a.n_qt * BW_T + DLV_ROWS - 1) / DLV_ROWS;
    const int bh = blockIdx.x / nrb;
    const int b = bh / a.N, h = bh % a.N;
    const fa_geom g = bw_geom(a, b);
    const int lane = threadIdx.x & 63, c = lane & 15;
    const int i = (blockIdx.x % nrb) * DLV_ROWS + (threadIdx.x >> 6) * 4 + (lane >> 4);
    float s = 0.f;
    if (i < g.sq) {
        const int64_t ro = b * a.q_bs + h * a.q_hs + (int64_t(g.q_start) + i) * a.q_rs;
        const u32x4* op = reinterpret_cast<const u32x4*>(static_cast<const T*>(a.o) + ro);
        const u32x4* dp = reinterpret_cast<const u32x4*>(static_cast<const T*>(a.dout) + ro);
        for (int k = c; k < a.D / 8; k += 16) {
            const u32x4 x = __builtin_nontemporal_load(op + k);
            const u32x4 y = dp[k];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                s = fmaf(half_f<T>(x[w] & 0xffffu), half_f<T>(y[w] & 0xffffu), s);
                s = fmaf(half_f<T>(x[w] >> 16), half_f<T>(y[w] >> 16), s);
            }
        }
    }
    // Every lane takes part in the reduction over its 16-lane row group.
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (c == 0 && i < g.sq) {
        const int64_t li = b * a.lse_bs + h * a.lse_hs + g.q_start + i;
        a.delta[li] = s;
        a.lse2[li] = a.lse[li] * kLog2e;
    }
}

// ------------------------------------------------------------------------------------------
// Generic kernels (fp32 arithmetic).
// ------------------------------------------------------------------------------------------
template <bool DENSE>
__device__ __forceinline__ bool bw_visible(const fa_bwd_args& a, const fa_geom& g, int b, int h, int i, int j) {
    if (i < 0 || i >= g.sq || j < 0 || j >= g.skv) return false;
    if (DENSE) return a.mask[b * a.m_bs + h * a.m_hs + int64_t(i) * a.m_rs + j] == 0;
    return j >= fa_row_lo(g, i) && j <= fa_row_hi(g, i);
}

// dQ: one thread per query row; K / V tiles of GB_T keys staged in LDS.
template <typename T, int DMAX, bool DENSE, int AL>
__global__ __launch_bounds__(GB_ROWS) void fa_bwd_dq_generic(const fa_bwd_args a) {
    __shared__ float qs[GB_ROWS][DMAX + 1], dos[GB_ROWS][DMAX + 1];
    __shared__ float ks[GB_T][DMAX], vs[GB_T][DMAX];
    const int nqt = (a.n_qt * BW_T + GB_ROWS - 1) / GB_ROWS;
    const int bh = blockIdx.x / nqt, qt = blockIdx.x % nqt;
    const int b = bh / a.N, h = bh % a.N;
    const fa_geom g = bw_geom(a, b);
    const int i0 = qt * GB_ROWS;
    if (i0 >= g.sq) return;
    const int D = a.D, tid = threadIdx.x, i = i0 + tid;
    const T* qp = static_cast<const T*>(a.q) + b * a.q_bs + h * a.q_hs + int64_t(g.q_start) * a.q_rs;
    const T* dop = static_cast<const T*>(a.dout) + b * a.q_bs + h * a.q_hs + int64_t(g.q_start) * a.q_rs;
    const T* kp = static_cast<const T*>(a.k) + b * a.kv_bs + h * a.kv_hs + int64_t(g.kv_start) * a.kv_rs;
    const T* vp = static_cast<const T*>(a.v) + b * a.kv_bs + h * a.kv_hs + int64_t(g.kv_start) * a.kv_rs;
    for (int e = tid; e < GB_ROWS * DMAX; e += GB_ROWS) {
        const int r = e / DMAX, d = e % DMAX;
        const bool ok = i0 + r < g.sq && d < D;
        qs[r][d] = ok ? to_f(qp[int64_t(i0 + r) * a.q_rs + d]) : 0.f;
        dos[r][d] = ok ? to_f(dop[int64_t(i0 + r) * a.q_rs + d]) : 0.f;
    }
    const bool row_ok = i < g.sq;
    const int64_t li = b * a.lse_bs + h * a.lse_hs + g.q_start + (row_ok ? i : 0);
    const float lse2 = row_ok ? a.lse[li] * kLog2e : 0.f;
    const float dlt = row_ok ? a.delta[li] : 0.f;
    const float slope2 = AL ? a.slopes[h] * kLog2e : 0.f;
    const int off = g.skv - g.sq, aoff = a.alibi_left ? 0 : off;
    float dq[DMAX];
#pragma unroll
    for (int d = 0; d < DMAX; ++d) dq[d] = 0.f;
    const int i1 = min(i0 + GB_ROWS, g.sq) - 1;
    const fa_kv_range kr = DENSE ? fa_kv_range{0, (g.skv + GB_T - 1) / GB_T} : fa_tile_kv_range(g, i0, i1, GB_T);
    for (int kt = kr.begin; kt < kr.end; ++kt) {
        const int j0 = kt * GB_T;
        __syncthreads();
        for (int e = tid; e < GB_T * DMAX; e += GB_ROWS) {
            const int r = e / DMAX, d = e % DMAX;
            const bool ok = j0 + r < g.skv && d < D;
            ks[r][d] = ok ? to_f(kp[int64_t(j0 + r) * a.kv_rs + d]) : 0.f;
            vs[r][d] = ok ? to_f(vp[int64_t(j0 + r) * a.kv_rs + d]) : 0.f;
        }
        __syncthreads();
#pragma unroll 1
        for (int jj = 0; jj < GB_T; ++jj) {
            const int j = j0 + jj;
            if (!bw_visible<DENSE>(a, g, b, h, i, j)) continue;
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int d = 0; d < DMAX; ++d) {
                s = fmaf(qs[tid][d], ks[jj][d], s);
                dp = fmaf(dos[tid][d], vs[jj][d], dp);
            }
            const float p = exp2f(fmaf(s, a.scale_log2, bw_bias2<AL>(slope2, i, j, off, aoff)) - lse2);
            const float ds = p * (dp - dlt);
#pragma unroll
            for (int d = 0; d < DMAX; ++d) dq[d] = fmaf(ds, ks[jj][d], dq[d]);
        }
    }
    if (row_ok) {
        T* out = static_cast<T*>(a.dq) + b * a.q_bs + h * a.q_hs + (int64_t(g.q_start) + i) * a.q_rs;
#pragma unroll
        for (int d = 0; d < DMAX; ++d)
            if (d < D) out[d] = T(dq[d] * a.scale);
    }
}

// dK (WHICH = 1) or dV (WHICH = 0): one thread per key; Q / dO tiles of GB_T rows in LDS.
template <typename T, int DMAX, bool DENSE, int AL, int WHICH>
__global__ __launch_bounds__(GB_ROWS) void fa_bwd_dkdv_generic(const fa_bwd_args a) {
    __shared__ float ks[GB_ROWS][DMAX + 1], vs[GB_ROWS][DMAX + 1];
    __shared__ float qs[GB_T][DMAX], dos[GB_T][DMAX];
    __shared__ float ls[GB_T], dls[GB_T];
    const int nkt = (a.n_kt * BW_T + GB_ROWS - 1) / GB_ROWS;
    const int bh = blockIdx.x / nkt, kt = blockIdx.x % nkt;
    const int b = bh / a.N, h = bh % a.N;
    const fa_geom g = bw_geom(a, b);
    const int j0 = kt * GB_ROWS;
    if (j0 >= g.skv) return;
    const int D = a.D, tid = threadIdx.x, j = j0 + tid;
    const T* qp = static_cast<const T*>(a.q) + b * a.q_bs + h * a.q_hs + int64_t(g.q_start) * a.q_rs;
    const T* dop = static_cast<const T*>(a.dout) + b * a.q_bs + h * a.q_hs + int64_t(g.q_start) * a.q_rs;
    const T* kp = static_cast<const T*>(a.k) + b * a.kv_bs + h * a.kv_hs + int64_t(g.kv_start) * a.kv_rs;
    const T* vp = static_cast<const T*>(a.v) + b * a.kv_bs + h * a.kv_hs + int64_t(g.kv_start) * a.kv_rs;
    for (int e = tid; e < GB_ROWS * DMAX; e += GB_ROWS) {
        const int r = e / DMAX, d = e % DMAX;
        const bool ok = j0 + r < g.skv && d < D;
        ks[r][d] = ok ? to_f(kp[int64_t(j0 + r) * a.kv_rs + d]) : 0.f;
        vs[r][d] = ok ? to_f(vp[int64_t(j0 + r) * a.kv_rs + d]) : 0.f;
    }
    const float slope2 = AL ? a.slopes[h] * kLog2e : 0.f;
    const int off = g.skv - g.sq, aoff = a.alibi_left ? 0 : off;
    float acc[DMAX];
#pragma unroll
    for (int d = 0; d < DMAX; ++d) acc[d] = 0.f;
    int r_lo = 0, r_hi = g.sq - 1;
    if (!DENSE) bw_row_range(g, j0, min(j0 + GB_ROWS, g.skv) - 1, r_lo, r_hi);
    for (int t0 = (r_lo / GB_T) * GB_T; t0 <= r_hi; t0 += GB_T) {
        __syncthreads();
        for (int e = tid; e < GB_T * DMAX; e += GB_ROWS) {
            const int r = e / DMAX, d = e % DMAX;
            const bool ok = t0 + r < g.sq && d < D;
            qs[r][d] = ok ? to_f(qp[int64_t(t0 + r) * a.q_rs + d]) : 0.f;
            dos[r][d] = ok ? to_f(dop[int64_t(t0 + r) * a.q_rs + d]) : 0.f;
        }
        if (tid < GB_T) {
            const bool ok = t0 + tid < g.sq;
            const int64_t li = b * a.lse_bs + h * a.lse_hs + g.q_start + (ok ? t0 + tid : 0);
            ls[tid] = ok ? a.lse[li] * kLog2e : 0.f;
            dls[tid] = ok ? a.delta[li] : 0.f;
        }
        __syncthreads();
#pragma unroll 1
        for (int ii = 0; ii < GB_T; ++ii) {
            const int i = t0 + ii;
            if (!bw_visible<DENSE>(a, g, b, h, i, j)) continue;
            float s = 0.f;
#pragma unroll
            for (int d = 0; d < DMAX; ++d) s = fmaf(qs[ii][d], ks[tid][d], s);
            const float p = exp2f(fmaf(s, a.scale_log2, bw_bias2<AL>(slope2, i, j, off, aoff)) - ls[ii]);
            if (WHICH == 0) {
#pragma unroll
                for (int d = 0; d < DMAX; ++d) acc[d] = fmaf(p, dos[ii][d], acc[d]);
            } else {
                float dp = 0.f;
#pragma unroll
                for (int d = 0; d < DMAX; ++d) dp = fmaf(dos[ii][d], vs[tid][d], dp);
                const float ds = p * (dp - dls[ii]);
#pragma unroll
                for (int d = 0; d < DMAX; ++d) acc[d] = fmaf(ds, qs[ii][d], acc[d]);
            }
        }
    }
    if (j < g.skv) {
        T* out = static_cast<T*>(WHICH == 0 ? a.dv : a.dk) + b * a.kv_bs + h * a.kv_hs +
                 (int64_t(g.kv_start) + j) * a.kv_rs;
        const float f = WHICH == 0 ? 1.f : a.scale;
#pragma unroll
        for (int d = 0; d < DMAX; ++d)
            if (d < D) out[d] = T(acc[d] * f);
    }
}

// ------------------------------------------------------------------------------------------
// MFMA kernels.
// ------------------------------------------------------------------------------------------

// LDS tiles are 64 rows x D, row-major in 16-byte chunks; chunk c of row r sits at c ^ swz(r).
// Two read patterns must both spread over the banks: A-operand reads (16 bytes per lane; the
// 16 lanes of a group read rows 8 (n / 4) + n % 4 (+ const) at one logical chunk) and transpose
// reads (8 bytes per lane; four consecutive rows at logical chunks 2 db and 2 db + 1 per group).
// D = 128: bits 0-1 of r XOR chunk bits 2-3 and bits 2-3 of r XOR chunk bits 0-1. With
// SQ_LDS_BANK_CONFLICT, a read loop of each pattern measured no conflict cycles this way; an
// XOR of chunk bits 0-1 with r bits 0-1 (and 2-3 with r bits 3-4) gave two-way conflicts on
// the transpose reads. D = 64 (two 128-byte rows per 256 bytes): the same on y = r / 2.
template <int KCH>
__device__ __forceinline__ int bw_swz(int r) {
    if constexpr (KCH == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else {
        const int y = r >> 1;
        return ((y & 1) << 2) | ((y >> 1) & 3);
    }
}

// Row (or key) held by value e of a lane in group gq for 16 x 16 block bb of a 64-row tile:
// 32 (bb / 2) + 8 gq + 4 (bb % 2) + e. The A operand of block bb in row slot n holds
// perm_row(bb, n) = 32 (bb / 2) + 8 (n / 4) + 4 (bb % 2) + n % 4.
__device__ __forceinline__ int bw_perm(int bb, int r) { return 32 * (bb >> 1) + 8 * (r >> 2) + 4 * (bb & 1) + (r & 3); }

// Cooperative HBM -> LDS load of a 64-row tile by NT threads (rows past `rows` read as zeros).
template <int D, int NT>
__device__ __forceinline__ void bw_tile_load(const uint16_t* base, int rs, int rows, u32x4* dst) {
    constexpr int KCH = D / 8;
    constexpr int NLD = BW_T * KCH / NT;
    static_assert(NLD >= 1 && BW_T * KCH % NT == 0, "tile shape");
    const __amdgpu_buffer_rsrc_t r = fa_rsrc(base, rows > 0 ? ((rows - 1) * rs + D) * 2 : 0);
    const int wave = fa_uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
#pragma unroll
    for (int p = 0; p < NLD; ++p) {
        const int c = p * NT + wave * 64 + lane;
        const int row = c / KCH, cc = c % KCH;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + p * NT + wave * 64), 16,
                                                 (row * rs + (cc ^ bw_swz<KCH>(row)) * 8) * 2, 0, 0, 0);
    }
}

// Two tiles of the same rows (K and V, or Q and dO) starting at row r0.
template <int D, int NT>
__device__ __forceinline__ void bw_load2(const uint16_t* x, const uint16_t* y, int r0, int rs, int rows, u32x4* dx,
                                         u32x4* dy) {
    bw_tile_load<D, NT>(x + int64_t(r0) * rs, rs, rows, dx);
    bw_tile_load<D, NT>(y + int64_t(r0) * rs, rs, rows, dy);
}

// The MFMA kernels: eight waves of 16 rows (dQ) or 16 keys (dK dV), so one staged tile feeds
// 128 rows or keys; tiles stream through a ring of four LDS buffers, loaded three tiles ahead,
// each wave waiting (vmcnt) only for the tile the next step reads. The ring buffers are
// separate arrays picked at compile time, so the compiler sees which buffer every access and
// load touches.
constexpr int BW2_THREADS = 512;
constexpr int BW2_BLOCK = 128;   // query rows (dQ) or keys (dK dV) per workgroup

// Workgroup barrier that waits for this wave's LDS operations (lgkmcnt 0) but not for its
// loads into LDS still in flight (vmcnt), which each step waits for explicitly.
__device__ __forceinline__ void bw_lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left alone
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Per-lane byte offsets, inside a tile, of the two swizzled read patterns, computed once per
// kernel (bw_swz uses row bits 0-3 only, so rows 32 apart share them):
//  a[p][kd]: A operand of block bb with bb % 2 = p, row slot n (row bw_perm(bb, n)), logical
//            chunk 4 kd + gq; block bb adds 32 (bb / 2) rows;
//  b[hf][db]: transpose read of row 8 gq + 4 hf + n / 4 (+ 32 kk), bytes 32 db + 8 (n % 4).
template <int D>
struct bw_offsets {
    static constexpr int KCH = D / 8, KD = D / 32, DB = D / 16;
    int a[2][KD];
    int b[2][DB];
    __device__ __forceinline__ bw_offsets(int n, int gq) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int row = bw_perm(p, n);
#pragma unroll
            for (int kd = 0; kd < KD; ++kd) a[p][kd] = (row * KCH + ((4 * kd + gq) ^ bw_swz<KCH>(row))) * 16;
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int row = 8 * gq + 4 * hf + (n >> 2);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int byte = 32 * db + 8 * (n & 3);   // within the logical row
                b[hf][db] = (row * KCH + ((byte >> 4) ^ bw_swz<KCH>(row))) * 16 + (byte & 15);
            }
        }
    }
};

// A operand (16 B) of block bb, k-step kd, from a swizzled LDS tile.
template <int D>
__device__ __forceinline__ u32x4 bw_arow(const u32x4* tile, const bw_offsets<D>& o, int bb, int kd) {
    constexpr int KCH = D / 8;
    const char* p = reinterpret_cast<const char*>(tile) + 32 * (bb >> 1) * KCH * 16 + o.a[bb & 1][kd];
    return *reinterpret_cast<const u32x4*>(p);
}

// B operand: rows 32 kk + 8 gq + 0..7 of column 16 db + n, through two transpose reads.
template <int D>
__device__ __forceinline__ u32x4 bw_bcol(const u32x4* tile, const bw_offsets<D>& o, int kk, int db) {
    constexpr int KCH = D / 8;
    const char* base = reinterpret_cast<const char*>(tile) + 32 * kk * KCH * 16;
    u32x4 out;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(base + o.b[hf][db]));
        out[2 * hf] = __builtin_bit_cast(u32x2, x)[0];
        out[2 * hf + 1] = __builtin_bit_cast(u32x2, x)[1];
    }
    return out;
}

// dQ: eight waves x 16 query rows; kv tiles of 64 keys through the LDS ring.
template <int D, bool IS_BF16, int AL>
__global__ __launch_bounds__(BW2_THREADS) void fa_bwd_dq_mfma(const fa_bwd_args a) {
    using io = mfma_io<IS_BF16>;
    using mm = mfma16_io<IS_BF16>;
    constexpr int KD = D / 32, DB = D / 16, TILE_U4 = BW_T * D / 8;
    constexpr int LPT = 2 * TILE_U4 / BW2_THREADS;   // direct loads per thread and kv tile (K and V)
    __shared__ u32x4 k0[TILE_U4], k1[TILE_U4], k2[TILE_U4], k3[TILE_U4];
    __shared__ u32x4 v0[TILE_U4], v1[TILE_U4], v2[TILE_U4], v3[TILE_U4];
    FA_POISON_LDS(k0, k1, k2, k3, v0, v1, v2, v3);
    auto kbuf = [&](auto s_tag) __attribute__((always_inline)) -> u32x4* {
        constexpr int S = decltype(s_tag)::value & 3;
        if constexpr (S == 0) return k0;
        else if constexpr (S == 1) return k1;
        else if constexpr (S == 2) return k2;
        else return k3;
    };
    auto vbuf = [&](auto s_tag) __attribute__((always_inline)) -> u32x4* {
        constexpr int S = decltype(s_tag)::value & 3;
        if constexpr (S == 0) return v0;
        else if constexpr (S == 1) return v1;
        else if constexpr (S == 2) return v2;
        else return v3;
    };
    const int lane = threadIdx.x & 63, wave = fa_uniform(threadIdx.x >> 6);
    const int n = lane & 15, gq = lane >> 4;
    const bw_offsets<D> lo(n, gq);
    const int nqb = (a.n_qt * BW_T + BW2_BLOCK - 1) / BW2_BLOCK;
    int bh, qb;
    bw_block(blockIdx.x, a.B * a.N, nqb, true, a.rank_order != 0, a.rank_order == 2, bh, qb);
    const int b = bh / a.N, h = bh % a.N;
    const fa_geom g = bw_geom(a, b);
    const int i0 = qb * BW2_BLOCK;
    if (i0 >= g.sq) return;
    const int q_rs = int(a.q_rs), kv_rs = int(a.kv_rs);
    const int64_t qo = b * a.q_bs + h * a.q_hs + int64_t(g.q_start) * a.q_rs;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qo;
    const uint16_t* dop = static_cast<const uint16_t*>(a.dout) + qo;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.kv_bs + h * a.kv_hs + int64_t(g.kv_start) * a.kv_rs;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + b * a.kv_bs + h * a.kv_hs + int64_t(g.kv_start) * a.kv_rs;

    // This lane's query row (the S^T column) and its operands.
    const int wrow0 = i0 + 16 * wave;
    const int i = wrow0 + n;
    const bool row_ok = i < g.sq;
    u32x4 qop[KD], dop_[KD];
    {
        const int bytes = ((g.sq - 1) * q_rs + D) * 2;
        const __amdgpu_buffer_rsrc_t rq = fa_rsrc(qp, bytes), rd = fa_rsrc(dop, bytes);
#pragma unroll
        for (int kd = 0; kd < KD; ++kd) {
            qop[kd] = fa_bload(rq, (i * q_rs + 32 * kd + 8 * gq) * 2);
            dop_[kd] = fa_bload(rd, (i * q_rs + 32 * kd + 8 * gq) * 2);
        }
    }
    const int64_t li = b * a.lse_bs + h * a.lse_hs + g.q_start + (row_ok ? i : 0);
    const float lse2 = row_ok ? a.lse[li] * kLog2e : INFINITY;
    const float dlt = row_ok ? a.delta[li] : 0.f;
    const int row_lo = fa_row_lo(g, i), row_hi = fa_row_hi(g, i);
    const float sl2 = a.scale_log2;
    const float slope2 = AL ? a.slopes[h] * kLog2e : 0.f;
    const int off = g.skv - g.sq, aoff = a.alibi_left ? 0 : off;

    const fa_kv_range kr = fa_tile_kv_range(g, i0, min(i0 + BW2_BLOCK, g.sq) - 1, BW_T);
    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{};
    // kv tile kt (none past the range: zeros, nothing read).
    auto load = [&](int kt, u32x4* dk, u32x4* dv) __attribute__((always_inline)) {
        bw_load2<D, BW2_THREADS>(kp, vp, kt * BW_T, kv_rs, kt < kr.end ? min(BW_T, g.skv - kt * BW_T) : 0, dk, dv);
    };
    // S and dP of this wave's 16 rows against the 64 keys of a staged tile.
    auto scores = [&](const u32x4* kt_, const u32x4* vt_, f32x4 (&s)[4], f32x4 (&dp)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            s[bb] = f32x4{};
            dp[bb] = f32x4{};
#pragma unroll
            for (int kd = 0; kd < KD; ++kd) {
                s[bb] = mm::mma(bw_arow<D>(kt_, lo, bb, kd), qop[kd], s[bb]);
                dp[bb] = mm::mma(bw_arow<D>(vt_, lo, bb, kd), dop_[kd], dp[bb]);
            }
        }
    };
    // The scores of tile kt + 1 are computed one step ahead: their MFMAs are issued in between
    // the elementwise work of tile kt, which does not depend on them, so the matrix cores run
    // while this wave computes P and dS. Tiles where all of this wave's entries are visible
    // (most of them) take a branch-free path with no per-entry mask test.
    f32x4 sc[4], dpc[4];
    auto ahead = [&](auto full_tag, auto s1_tag, int kt, u32x4 (&dsop)[2]) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_tag)::value;
        f32x4 sn[4], dpn[4];
        scores(kbuf(s1_tag), vbuf(s1_tag), sn, dpn);   // tile kt + 1 (past the range: zeros, unused)
        const int j0 = kt * BW_T;
        float ds[16];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + 32 * (bb >> 1) + 8 * gq + 4 * (bb & 1) + e;
                const float x = AL ? fmaf(sc[bb][e], sl2, bw_bias2<AL>(slope2, i, j, off, aoff)) - lse2
                                   : fmaf(sc[bb][e], sl2, -lse2);
                float p = __builtin_amdgcn_exp2f(x);
                if (!FULL) p = (row_ok & (j >= row_lo) & (j <= row_hi)) ? p : 0.f;
                ds[4 * bb + e] = p * (dpc[bb][e] - dlt);
            }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const float* lo = ds + 8 * kk;
            const float* hi = ds + 8 * kk + 4;
            dsop[kk] = u32x4{io::pack(lo[0], lo[1]), io::pack(lo[2], lo[3]), io::pack(hi[0], hi[1]),
                             io::pack(hi[2], hi[3])};
        }
        if (FULL) {
            // The next tile's 32 MFMAs, each with a share of the VALU work; their A operands
            // are read from LDS six MFMAs ahead.
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);   // DS read
#pragma unroll
            for (int m = 0; m < 32; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                if (m < 26) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
            }
        }
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            sc[bb] = sn[bb];
            dpc[bb] = dpn[bb];
        }
    };
    auto step = [&](auto s_tag, int kt) __attribute__((always_inline)) {
        constexpr int S = decltype(s_tag)::value;
        using s1 = std::integral_constant<int, (S + 1) & 3>;
        using s3 = std::integral_constant<int, (S + 3) & 3>;
        load(kt + 3, kbuf(s3{}), vbuf(s3{}));
        const u32x4* kt_ = kbuf(s_tag);
        const int j0 = kt * BW_T;
        // Every (row, key) of this wave's 16 rows x 64 keys visible: no per-entry test.
        const bool full = fa_tile_full(g, wrow0, min(wrow0 + 15, g.sq - 1), j0, BW_T) && wrow0 + 15 < g.sq;
        u32x4 dsop[2];
        if (full) ahead(std::true_type{}, s1{}, kt, dsop);
        else ahead(std::false_type{}, s1{}, kt, dsop);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) acc[db] = mm::mma(dsop[kk], bw_bcol<D>(kt_, lo, kk, db), acc[db]);
        __builtin_amdgcn_s_waitcnt(fa_vmcnt64(LPT));   // tile kt + 2 has landed
        bw_lds_barrier();
    };
    if (kr.begin < kr.end) {
        using c0 = std::integral_constant<int, 0>;
        using c1 = std::integral_constant<int, 1>;
        using c2 = std::integral_constant<int, 2>;
        using c3 = std::integral_constant<int, 3>;
        load(kr.begin, k0, v0);
        load(kr.begin + 1, k1, v1);
        load(kr.begin + 2, k2, v2);
        __builtin_amdgcn_s_waitcnt(fa_vmcnt64(LPT));   // Q, dO and tiles 0 and 1
        bw_lds_barrier();
        scores(k0, v0, sc, dpc);
        // Trips of four; every path into a step runs the earlier ones.
        for (int kt = kr.begin; kt < kr.end; kt += 4) {
            step(c0{}, kt);
            if (kt + 1 >= kr.end) break;
            step(c1{}, kt + 1);
            if (kt + 2 >= kr.end) break;
            step(c2{}, kt + 2);
            if (kt + 3 >= kr.end) break;
            step(c3{}, kt + 3);
        }
        __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the loop
    }
    // Rows 16 wave + 4 gq + e, columns 16 db + n. Non-temporal: the kernel never reads dQ back.
    uint16_t* out = static_cast<uint16_t*>(a.dq) + qo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = wrow0 + 4 * gq + e;
        if (r < g.sq) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
                __builtin_nontemporal_store(uint16_t(io::pack(acc[db][e] * a.scale, 0.f) & 0xffffu), &out[int64_t(r) * q_rs + 16 * db + n]);
        }
    }
}

// dK and dV: eight waves x 16 keys; q tiles of 64 rows (Q, dO, LSE, Delta) through the LDS
// ring. Wave 0 also loads each tile's LSE and Delta (one 4-byte load per lane each).
template <int D, bool IS_BF16, int AL>
__global__ __launch_bounds__(BW2_THREADS) void fa_bwd_dkdv_mfma(const fa_bwd_args a) {
    using io = mfma_io<IS_BF16>;
    using mm = mfma16_io<IS_BF16>;
    constexpr int KD = D / 32, DB = D / 16, TILE_U4 = BW_T * D / 8;
    constexpr int LPT = 2 * TILE_U4 / BW2_THREADS;   // direct loads per thread and q tile (Q and dO)
    __shared__ u32x4 q0[TILE_U4], q1[TILE_U4], q2[TILE_U4], q3[TILE_U4];
    __shared__ u32x4 o0[TILE_U4], o1[TILE_U4], o2[TILE_U4], o3[TILE_U4];
    __shared__ __attribute__((aligned(16))) float l0[BW_T], l1[BW_T], l2[BW_T], l3[BW_T];
    __shared__ __attribute__((aligned(16))) float d0[BW_T], d1[BW_T], d2[BW_T], d3[BW_T];
    FA_POISON_LDS(q0, q1, q2, q3, o0, o1, o2, o3, l0, l1, l2, l3, d0, d1, d2, d3);
    auto qbuf = [&](auto s_tag) __attribute__((always_inline)) -> u32x4* {
        constexpr int S = decltype(s_tag)::value & 3;
        if constexpr (S == 0) return q0;
        else if constexpr (S == 1) return q1;
        else if constexpr (S == 2) return q2;
        else return q3;
    };
    auto obuf = [&](auto s_tag) __attribute__((always_inline)) -> u32x4* {
        constexpr int S = decltype(s_tag)::value & 3;
        if constexpr (S == 0) return o0;
        else if constexpr (S == 1) return o1;
        else if constexpr (S == 2) return o2;
        else return o3;
    };
    auto lbuf = [&](auto s_tag) __attribute__((always_inline)) -> float* {
        constexpr int S = decltype(s_tag)::value & 3;
        if constexpr (S == 0) return l0;
        else if constexpr (S == 1) return l1;
        else if constexpr (S == 2) return l2;
        else return l3;
    };
    auto dbuf = [&](auto s_tag) __attribute__((always_inline)) -> float* {
        constexpr int S = decltype(s_tag)::value & 3;
        if constexpr (S == 0) return d0;
        else if constexpr (S == 1) return d1;
        else if constexpr (S == 2) return d2;
        else return d3;
    };
    const int lane = threadIdx.x & 63, wave = fa_uniform(threadIdx.x >> 6);
    const int n = lane & 15, gq = lane >> 4;
    const bw_offsets<D> lo(n, gq);
    const int nkb = (a.n_kt * BW_T + BW2_BLOCK - 1) / BW2_BLOCK;
    int bh, kb;
    bw_block(blockIdx.x, a.B * a.N, nkb, false, a.rank_order != 0, a.rank_order == 2, bh, kb);
    const int b = bh / a.N, h = bh % a.N;
    const fa_geom g = bw_geom(a, b);
    const int j0 = kb * BW2_BLOCK;
    if (j0 >= g.skv) return;
    const int q_rs = int(a.q_rs), kv_rs = int(a.kv_rs);
    const int64_t qo = b * a.q_bs + h * a.q_hs + int64_t(g.q_start) * a.q_rs;
    const int64_t ko = b * a.kv_bs + h * a.kv_hs + int64_t(g.kv_start) * a.kv_rs;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qo;
    const uint16_t* dop = static_cast<const uint16_t*>(a.dout) + qo;
    const float* lsep = a.lse2 + b * a.lse_bs + h * a.lse_hs + g.q_start;
    const float* dlp = a.delta + b * a.lse_bs + h * a.lse_hs + g.q_start;

    // This lane's key (the S column) and its operands.
    const int wkey0 = j0 + 16 * wave;
    const int j = wkey0 + n;
    u32x4 kop[KD], vop[KD];
    {
        const int bytes = ((g.skv - 1) * kv_rs + D) * 2;
        const __amdgpu_buffer_rsrc_t rk = fa_rsrc(static_cast<const uint16_t*>(a.k) + ko, bytes);
        const __amdgpu_buffer_rsrc_t rv = fa_rsrc(static_cast<const uint16_t*>(a.v) + ko, bytes);
#pragma unroll
        for (int kd = 0; kd < KD; ++kd) {
            kop[kd] = fa_bload(rk, (j * kv_rs + 32 * kd + 8 * gq) * 2);
            vop[kd] = fa_bload(rv, (j * kv_rs + 32 * kd + 8 * gq) * 2);
        }
    }
    const float sl2 = a.scale_log2;
    const float slope2 = AL ? a.slopes[h] * kLog2e : 0.f;
    const int off = g.skv - g.sq, aoff = a.alibi_left ? 0 : off;
    int r_lo, r_hi;
    bw_row_range(g, j0, min(j0 + BW2_BLOCK, g.skv) - 1, r_lo, r_hi);
    const int t_begin = r_lo / BW_T, t_end = r_lo <= r_hi ? r_hi / BW_T + 1 : t_begin;
    // The rows that see this lane's key form one interval (both ends of a row's visible range
    // grow with the row); for a single key bw_row_range is exact. None past the sequence's keys.
    int key_row_lo, key_row_hi;
    bw_row_range(g, j, j, key_row_lo, key_row_hi);
    if (j >= g.skv) key_row_hi = -1;

    f32x4 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dk[db] = f32x4{};
        dv[db] = f32x4{};
    }
    // q tile t (none past the range: zeros, nothing read): Q and dO by every wave; the LSE in
    // log2 units (as the Delta kernel wrote it) and Delta (rows past the sequence read as zeros)
    // by wave 0.
    auto load = [&](int t, u32x4* dq_, u32x4* ddo, float* dl, float* ddl) __attribute__((always_inline)) {
        const int rows = t < t_end ? min(BW_T, g.sq - t * BW_T) : 0;
        bw_load2<D, BW2_THREADS>(qp, dop, t * BW_T, q_rs, rows, dq_, ddo);
        if (wave == 0) {
            const __amdgpu_buffer_rsrc_t rl = fa_rsrc(lsep + t * BW_T, rows * 4);
            const __amdgpu_buffer_rsrc_t rd = fa_rsrc(dlp + t * BW_T, rows * 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void_t*)dl, 4, lane * 4, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void_t*)ddl, 4, lane * 4, 0, 0, 0);
        }
    };
    auto step = [&](auto s_tag, int t) __attribute__((always_inline)) {
        constexpr int S = decltype(s_tag)::value;
        using s3 = std::integral_constant<int, (S + 3) & 3>;
        load(t + 3, qbuf(s3{}), obuf(s3{}), lbuf(s3{}), dbuf(s3{}));
        const u32x4* qt_ = qbuf(s_tag);
        const u32x4* dt_ = obuf(s_tag);
        const float* lt_ = lbuf(s_tag);
        const float* dlt_ = dbuf(s_tag);
        const int i0 = t * BW_T;
        // Two halves of the tile's 64 rows (blocks 2 hf, 2 hf + 1). Within a half the k-step loop is
        // outer, so consecutive MFMAs go to different accumulators; across halves the VALU work of
        // one half can run under the MFMAs of the other.
        f32x4 s[4], dp[4];
        // Every (row, key) of the 64 rows x this wave's 16 keys visible: no per-element test.
        const bool full = i0 + BW_T <= g.sq && fa_tile_full(g, i0, i0 + BW_T - 1, wkey0, 16);
        u32x4 pop[2], dsop[2];
        auto sdp = [&](int hf) __attribute__((always_inline)) {
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                s[2 * hf + r2] = f32x4{};
                dp[2 * hf + r2] = f32x4{};
            }
#pragma unroll
            for (int kd = 0; kd < KD; ++kd) {
#pragma unroll
                for (int r2 = 0; r2 < 2; ++r2) {
                    const int rb = 2 * hf + r2;
                    s[rb] = mm::mma(bw_arow<D>(qt_, lo, rb, kd), kop[kd], s[rb]);
                    dp[rb] = mm::mma(bw_arow<D>(dt_, lo, rb, kd), vop[kd], dp[rb]);
                }
            }
        };
        // P and dS of the half's 32 rows x this lane's key, packed as the dV / dK left operands.
        // FULL (every entry of the tile visible for this wave, most tiles): no mask test at all.
        auto soft = [&](auto full_tag, int hf) __attribute__((always_inline)) {
            constexpr bool FULL = decltype(full_tag)::value;
            float p[8], ds[8];
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int rb = 2 * hf + r2;
                const int r0 = 32 * (rb >> 1) + 8 * gq + 4 * (rb & 1);   // tile rows r0 .. r0 + 3
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lt_[r0]);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dlt_[r0]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + r0 + e;
                    const float x = AL ? fmaf(s[rb][e], sl2, bw_bias2<AL>(slope2, i, j, off, aoff)) - l4[e]
                                       : fmaf(s[rb][e], sl2, -l4[e]);
                    float pv = __builtin_amdgcn_exp2f(x);
                    if (!FULL) pv = (i >= key_row_lo && i <= key_row_hi) ? pv : 0.f;
                    p[4 * r2 + e] = pv;
                    ds[4 * r2 + e] = pv * (dp[rb][e] - d4[e]);
                }
            }
            pop[hf] = u32x4{io::pack(p[0], p[1]), io::pack(p[2], p[3]), io::pack(p[4], p[5]), io::pack(p[6], p[7])};
            dsop[hf] = u32x4{io::pack(ds[0], ds[1]), io::pack(ds[2], ds[3]), io::pack(ds[4], ds[5]), io::pack(ds[6], ds[7])};
        };
        auto dvdk = [&](int kk) __attribute__((always_inline)) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                dv[db] = mm::mma(pop[kk], bw_bcol<D>(dt_, lo, kk, db), dv[db]);
                dk[db] = mm::mma(dsop[kk], bw_bcol<D>(qt_, lo, kk, db), dk[db]);
            }
        };
        sdp(0);
        if (full) soft(std::true_type{}, 0);
        else soft(std::false_type{}, 0);
        sdp(1);
        dvdk(0);
        if (full) soft(std::true_type{}, 1);
        else soft(std::false_type{}, 1);
        dvdk(1);
        // q tile t + 1 has landed (wave 0 issues two more loads per tile).
        if (wave == 0) __builtin_amdgcn_s_waitcnt(fa_vmcnt64(2 * (LPT + 2)));
        else __builtin_amdgcn_s_waitcnt(fa_vmcnt64(2 * LPT));
        bw_lds_barrier();
    };
    if (t_begin < t_end) {
        using c0 = std::integral_constant<int, 0>;
        using c1 = std::integral_constant<int, 1>;
        using c2 = std::integral_constant<int, 2>;
        using c3 = std::integral_constant<int, 3>;
        load(t_begin, q0, o0, l0, d0);
        load(t_begin + 1, q1, o1, l1, d1);
        load(t_begin + 2, q2, o2, l2, d2);
        if (wave == 0) __builtin_amdgcn_s_waitcnt(fa_vmcnt64(2 * (LPT + 2)));   // K, V and tile 0
        else __builtin_amdgcn_s_waitcnt(fa_vmcnt64(2 * LPT));
        bw_lds_barrier();
        // Trips of four; every path into a step runs the earlier ones.
        for (int t = t_begin; t < t_end; t += 4) {
            step(c0{}, t);
            if (t + 1 >= t_end) break;
            step(c1{}, t + 1);
            if (t + 2 >= t_end) break;
            step(c2{}, t + 2);
            if (t + 3 >= t_end) break;
            step(c3{}, t + 3);
        }
        __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the loop
    }
    // Keys 16 wave + 4 gq + e, columns 16 db + n. Non-temporal: the kernel never reads dK / dV back.
    uint16_t* dkp = static_cast<uint16_t*>(a.dk) + ko;
    uint16_t* dvp = static_cast<uint16_t*>(a.dv) + ko;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int key = wkey0 + 4 * gq + e;
        if (key < g.skv) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                __builtin_nontemporal_store(uint16_t(io::pack(dk[db][e] * a.scale, 0.f) & 0xffffu), &dkp[int64_t(key) * kv_rs + 16 * db + n]);
                __builtin_nontemporal_store(uint16_t(io::pack(dv[db][e], 0.f) & 0xffffu), &dvp[int64_t(key) * kv_rs + 16 * db + n]);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Host side.
// ------------------------------------------------------------------------------------------

struct bw_plan {
    fa_plan p;
    bool mfma = false;
    int32_t n_qt = 0, n_kt = 0;
    size_t ws_delta_offset = 0, ws_lse2_offset = 0, ws_bytes = 0;
    int64_t lse_elems = 0;
};

fa_status make_bw_plan(const fa_call& c, bool sizes_only, bw_plan* out) {
    bw_plan bp;
    const fa_status st = sizes_only ? fa_make_plan_sizes(c, &bp.p) : fa_make_plan(c, false, &bp.p);
    if (st != FA_OK) return st;
    const fa_dims& d = *c.dims;
    const fa_plan& p = bp.p;
    int64_t max_sq = 0, max_skv = 0;
    if (c.layout == FA_LAYOUT_TND) {
        int64_t pq = 0, pk = 0;
        for (int64_t b = 0; b < d.B; ++b) {
            max_sq = std::max(max_sq, c.actual_seq_qlen[b] - pq);
            max_skv = std::max(max_skv, c.actual_seq_kvlen[b] - pk);
            pq = c.actual_seq_qlen[b];
            pk = c.actual_seq_kvlen[b];
        }
        bp.lse_elems = d.N * d.T_q;
    } else {
        max_sq = d.Sq;
        max_skv = d.Skv;
        bp.lse_elems = d.B * d.N * d.Sq;
    }
    bp.n_qt = int32_t((max_sq + BW_T - 1) / BW_T);
    bp.n_kt = int32_t((max_skv + BW_T - 1) / BW_T);
    bp.mfma = (d.dtype == FA_DTYPE_F16 || d.dtype == FA_DTYPE_BF16) && (d.D == 64 || d.D == 128) &&
              c.sparse_mode != 1 && d.N * d.D * 2 * 256 < (int64_t(1) << 31);
    size_t off = 0;
    if (p.table) off = (size_t(d.B) * sizeof(fa_geom) + 255) & ~size_t(255);
    bp.ws_delta_offset = off;
    off = (off + size_t(bp.lse_elems) * sizeof(float) + 255) & ~size_t(255);
    bp.ws_lse2_offset = off;
    off += size_t(bp.lse_elems) * sizeof(float);
    bp.ws_bytes = (p.rows_total == 0 && p.kv_total == 0) ? 0 : ((off + 255) & ~size_t(255));
    *out = std::move(bp);
    return FA_OK;
}

template <typename T, int DMAX, bool DENSE, int AL>
void launch_generic(const fa_bwd_args& a, int64_t pairs, hipStream_t s) {
    const int nq = (a.n_qt * BW_T + GB_ROWS - 1) / GB_ROWS, nk = (a.n_kt * BW_T + GB_ROWS - 1) / GB_ROWS;
    if (nk > 0) {
        fa_bwd_dkdv_generic<T, DMAX, DENSE, AL, 0><<<dim3(unsigned(pairs * nk)), dim3(GB_ROWS), 0, s>>>(a);
        fa_bwd_dkdv_generic<T, DMAX, DENSE, AL, 1><<<dim3(unsigned(pairs * nk)), dim3(GB_ROWS), 0, s>>>(a);
    }
    if (nq > 0) fa_bwd_dq_generic<T, DMAX, DENSE, AL><<<dim3(unsigned(pairs * nq)), dim3(GB_ROWS), 0, s>>>(a);
}

template <typename T, int DMAX>
void launch_generic_d(const fa_bwd_args& a, int al, bool dense, int64_t pairs, hipStream_t s) {
    switch (al * 2 + (dense ? 1 : 0)) {
        case 0: launch_generic<T, DMAX, false, 0>(a, pairs, s); break;
        case 1: launch_generic<T, DMAX, true, 0>(a, pairs, s); break;
        case 2: launch_generic<T, DMAX, false, 1>(a, pairs, s); break;
        case 3: launch_generic<T, DMAX, true, 1>(a, pairs, s); break;
        case 4: launch_generic<T, DMAX, false, 2>(a, pairs, s); break;
        default: launch_generic<T, DMAX, true, 2>(a, pairs, s); break;
    }
}

template <typename T>
void launch_generic_t(const fa_bwd_args& a, int al, bool dense, int64_t pairs, hipStream_t s) {
    if (a.D <= 32) launch_generic_d<T, 32>(a, al, dense, pairs, s);
    else if (a.D <= 64) launch_generic_d<T, 64>(a, al, dense, pairs, s);
    else launch_generic_d<T, 128>(a, al, dense, pairs, s);
}

template <int D, bool BF, int AL>
void launch_mfma(const fa_bwd_args& a, int64_t pairs, hipStream_t s) {
    const int64_t nqb = (int64_t(a.n_qt) * BW_T + BW2_BLOCK - 1) / BW2_BLOCK;
    const int64_t nkb = (int64_t(a.n_kt) * BW_T + BW2_BLOCK - 1) / BW2_BLOCK;
    // Block order: host code 1 = the forward planner took rank-major (item costs spread widely),
    // 2 / 3 = forced rank / pair. Rank-major pays off only while a pair has few blocks: with
    // many, neighbouring blocks of a pair differ little in cost. Same box, rank-major against
    // pair-major: causal_2048 (16 blocks a pair) +9%, causal_8192 (64) -0.5%.
    const char* ge = std::getenv("FA_BWD_GROUPED");
    const bool grouped = !(ge && ge[0] == '0');
    auto order = [&](int64_t nblk) {
        fa_bwd_args c = a;
        c.rank_order = a.rank_order == 2 || (a.rank_order == 1 && nblk <= 32) ? (grouped ? 2 : 1) : 0;
        return c;
    };
    if (nkb > 0) fa_bwd_dkdv_mfma<D, BF, AL><<<dim3(unsigned(pairs * nkb)), dim3(BW2_THREADS), 0, s>>>(order(nkb));
    if (nqb > 0) fa_bwd_dq_mfma<D, BF, AL><<<dim3(unsigned(pairs * nqb)), dim3(BW2_THREADS), 0, s>>>(order(nqb));
}

template <int D, bool BF>
void launch_mfma_al(const fa_bwd_args& a, int al, int64_t pairs, hipStream_t s) {
    switch (al) {
        case 0: launch_mfma<D, BF, 0>(a, pairs, s); break;
        case 1: launch_mfma<D, BF, 1>(a, pairs, s); break;
        default: launch_mfma<D, BF, 2>(a, pairs, s); break;
    }
}

fa_call bw_call(const fa_dims* dims, int32_t layout, int32_t sparse_mode, int64_t pre, int64_t next,
                const int64_t* qlen, const int64_t* kvlen, const int64_t* prefix, bool alibi, int32_t alibi_mode,
                bool mask, const int64_t* mask_bcast, float scale) {
    fa_call c;
    c.dims = dims;
    c.layout = layout;
    c.sparse_mode = sparse_mode;
    c.pre_tokens = pre;
    c.next_tokens = next;
    c.actual_seq_qlen = qlen;
    c.actual_seq_kvlen = kvlen;
    c.prefix = prefix;
    c.has_alibi = alibi;
    c.alibi_mode = alibi_mode;
    c.has_mask = mask;
    c.mask_bcast = mask_bcast;
    c.scale = scale;
    return c;
}

}  // namespace

extern "C" fa_status fa_bwd_workspace_size(const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                                           const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                                           size_t* bytes) {
    if (!dims || !bytes) return FA_ERR_NULLPTR;
    const fa_call c = bw_call(dims, layout, sparse_mode, 0, 0, actual_seq_qlen, actual_seq_kvlen, nullptr, false,
                              FA_ALIBI_RIGHT, false, nullptr, 1.f);
    bw_plan bp;
    const fa_status st = make_bw_plan(c, true, &bp);
    if (st != FA_OK) return st;
    *bytes = bp.ws_bytes;
    return FA_OK;
}

extern "C" fa_status fa_bwd(const void* q, const void* k, const void* v, const void* out, const float* softmax_lse,
                            const void* dout, void* dq, void* dk, void* dv, const fa_dims* dims, int32_t layout,
                            int32_t sparse_mode, int64_t pre_tokens, int64_t next_tokens,
                            const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen, const int64_t* prefix,
                            const float* alibi_slopes, int32_t alibi_mode, const uint8_t* atten_mask,
                            const int64_t* mask_bcast, float scale, void* workspace, size_t workspace_bytes,
                            void* stream) {
    const fa_call c = bw_call(dims, layout, sparse_mode, pre_tokens, next_tokens, actual_seq_qlen, actual_seq_kvlen,
                              prefix, alibi_slopes != nullptr, alibi_mode, atten_mask != nullptr, mask_bcast, scale);
    bw_plan bp;
    fa_status st = make_bw_plan(c, false, &bp);
    if (st != FA_OK) return st;
    const fa_plan& p = bp.p;
    if (p.rows_total > 0 && (!q || !out || !softmax_lse || !dout || !dq)) return FA_ERR_NULLPTR;
    if (p.kv_total > 0 && (!k || !v || !dk || !dv)) return FA_ERR_NULLPTR;
    if (bp.ws_bytes > 0) {
        if (!workspace) return FA_ERR_NULLPTR;
        if (workspace_bytes < bp.ws_bytes) return FA_ERR_WORKSPACE;
    }
    const int64_t pairs = int64_t(p.B) * p.N;
    if (pairs * std::max<int64_t>(int64_t(std::max(bp.n_qt, bp.n_kt)) * (BW_T / DL_ROWS), 1) >= (int64_t(1) << 31))
        return FA_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    // Every dK / dV row of a sequence with keys is written (zeros where no query sees the key),
    // also when there are no query rows at all.
    if (p.kv_total == 0 && p.rows_total == 0) return FA_OK;
    if (p.table) {
        if (hipMemcpyAsync(workspace, p.geoms.data(), p.geoms.size() * sizeof(fa_geom), hipMemcpyHostToDevice, s) !=
            hipSuccess)
            return FA_ERR_HIP;
    }
    fa_bwd_args a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = out;
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.lse = softmax_lse;
    a.delta = reinterpret_cast<float*>(static_cast<char*>(workspace) + bp.ws_delta_offset);
    a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + bp.ws_lse2_offset);
    a.slopes = alibi_slopes;
    a.mask = atten_mask;
    a.geoms = p.table ? static_cast<const fa_geom*>(workspace) : nullptr;
    a.geom0 = p.geom0;
    a.q_bs = p.q_bs; a.q_hs = p.q_hs; a.q_rs = p.q_rs;
    a.kv_bs = p.kv_bs; a.kv_hs = p.kv_hs; a.kv_rs = p.kv_rs;
    a.lse_bs = p.lse_bs; a.lse_hs = p.lse_hs;
    a.m_bs = p.m_bs; a.m_hs = p.m_hs; a.m_rs = p.m_rs;
    a.B = p.B;
    a.N = p.N;
    a.D = p.D;
    a.n_qt = bp.n_qt;
    a.n_kt = bp.n_kt;
    a.alibi_left = alibi_mode == FA_ALIBI_LEFT ? 1 : 0;
    {
        // FA_BWD_ORDER=rank|pair forces the MFMA kernels' block order (comparisons).
        const char* e = std::getenv("FA_BWD_ORDER");
        a.rank_order = e && std::strcmp(e, "rank") == 0 ? 2 : (e && std::strcmp(e, "pair") == 0 ? 3 : (p.xcd_major >= 2 ? 1 : 0));
    }
    a.scale_log2 = scale * kLog2e;
    a.scale = scale;
    const int al = alibi_slopes == nullptr ? 0 : (alibi_mode == FA_ALIBI_SQRT ? 2 : 1);
    const bool dense = sparse_mode == 1;
    const int32_t dtype = dims->dtype;
    // The vector Delta kernel reads rows as 16-byte chunks: every row offset and both bases must be
    // 16-byte aligned.
    const bool delta_v = dtype != FA_DTYPE_F32 && p.D % 8 == 0 && p.q_bs % 8 == 0 && p.q_hs % 8 == 0 &&
                         p.q_rs % 8 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(dout) & 15) == 0;
    if (bp.n_qt > 0 && delta_v) {
        const dim3 grid(unsigned(pairs * ((bp.n_qt * BW_T + DLV_ROWS - 1) / DLV_ROWS)));
        if (dtype == FA_DTYPE_F16) fa_bwd_delta_v<_Float16><<<grid, dim3(BW_THREADS), 0, s>>>(a);
        else fa_bwd_delta_v<__bf16><<<grid, dim3(BW_THREADS), 0, s>>>(a);
    } else if (bp.n_qt > 0) {
        const dim3 grid(unsigned(pairs * ((bp.n_qt * BW_T + DL_ROWS - 1) / DL_ROWS)));
        switch (dtype) {
            case FA_DTYPE_F32: fa_bwd_delta<float><<<grid, dim3(BW_THREADS), 0, s>>>(a); break;
            case FA_DTYPE_F16: fa_bwd_delta<_Float16><<<grid, dim3(BW_THREADS), 0, s>>>(a); break;
            default: fa_bwd_delta<__bf16><<<grid, dim3(BW_THREADS), 0, s>>>(a); break;
        }
    }
    if (bp.mfma) {
        const bool bf = dtype == FA_DTYPE_BF16;
        if (p.D == 128) {
            if (bf) launch_mfma_al<128, true>(a, al, pairs, s);
            else launch_mfma_al<128, false>(a, al, pairs, s);
        } else {
            if (bf) launch_mfma_al<64, true>(a, al, pairs, s);
            else launch_mfma_al<64, false>(a, al, pairs, s);
        }
    } else {
        switch (dtype) {
            case FA_DTYPE_F32: launch_generic_t<float>(a, al, dense, pairs, s); break;
            case FA_DTYPE_F16: launch_generic_t<_Float16>(a, al, dense, pairs, s); break;
            default: launch_generic_t<__bf16>(a, al, dense, pairs, s); break;
        }
    }
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    return FA_OK;
}
