// fa_fwd_common.h - what the forward kernels' translation units share: the kernel argument
// block, the work-item decode, and the device helpers of the ping-pong phase machinery (lane-pair
// reductions, the LDS tile swizzle, phase barriers).
#ifndef FA_FWD_COMMON_H_
#define FA_FWD_COMMON_H_

#include <hip/hip_runtime.h>

#include "fa_device.h"
#include "fa_mask.h"
#include "fa_plan.h"

struct fa_kargs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const float* slopes;
    const uint8_t* mask;
    const fa_geom* geoms;   // per-batch table (workspace) or nullptr
    const int32_t* items;   // (b, q tile) launch list (workspace) or nullptr
    fa_geom geom0;          // shared geometry when there is no table
    int64_t q_bs, q_hs, q_rs;
    int64_t kv_bs, kv_hs, kv_rs;
    int64_t lse_bs, lse_hs;
    int64_t m_bs, m_hs, m_rs;
    int32_t B, N, D;
    int32_t n_qtiles_fixed;
    int32_t reverse_qt;
    int32_t xcd_major;      // fixed-length launch order, see fa_decode_item
    int32_t alibi_left;     // linear alibi measured from the top-left diagonal (else bottom-right)
    float scale_log2;       // scale * log2(e)
    // Paged K / V (k and v are the caches; kv_bs = 0, sequences start at key 0 of their pages).
    const int32_t* block_table;   // [B, bt_stride] page ids, or nullptr
    int64_t page_stride;          // elements from one page to the next
    int64_t bt_stride;
    int32_t block_size;
    int32_t log2_block_size;      // ping-pong kernel: block_size = 2^log2_block_size >= 64
    int32_t num_pages;            // valid page ids are [0, num_pages)
    // Dense mask (sparse mode 1) on the ping-pong kernel: the pre-pass's tables (workspace).
    const uint32_t* tile_list;    // [slices, nqt, 1 + nkt]: count, then kt | full-wave bits << 24
    const uint32_t* tile_bits;    // [slices, nqt, nkt, 512]: hidden-key bits, one dword per lane
    const int32_t* tile_perm;     // [slices, nqt]: q tiles of a slice in launch order
    int32_t dense_nqt, dense_nkt;
    int32_t m_heads, m_bcast_b, m_bcast_h;
};


// Persistent schedule of fa_fwd_ps: which items each workgroup works through. Items form one
// list per XCD (xcd = 1: XCD x = blockIdx % 8 takes the (batch, head) pairs congruent to x, each
// pair's q tiles heaviest first) or one list for all (xcd = 0; in table mode the planner's
// heaviest-first (batch, q tile) list times the heads, heads fastest). Round r of the W
// workgroups sharing a list takes items r W .. r W + W - 1, the j-th of them going to workgroup
// j in even rounds and to workgroup W - 1 - j in odd rounds, which evens out the work of
// heaviest-first lists.
struct fa_ps_args {
    int32_t W;        // workgroups sharing one list
    int32_t xcd;      // lists per XCD
    int32_t n_list;   // items in one list
    int32_t nq;       // fixed-length mode: q tiles per (batch, head)
    // Divisions of list positions (< 2^31) by nq and by N: n / d = mulhi(n, mul) >> shr, or
    // n >> shr when mul is 0 (d a power of two); see fa_magic_divisor.
    uint32_t nq_mul, nq_shr;
    uint32_t n_mul, n_shr;
    int32_t N;
    int32_t reverse_qt;   // fixed-length mode: rank r is q tile nq - 1 - r
    int32_t table;        // items come from fa_kargs::items (varlen / prefix modes)
    int32_t pad;
};

// Multiplier and shift that divide any n < 2^31 by d >= 1 (Granlund-Montgomery with a rounded-up
// multiplier): s = floor(log2 d); for d = 2^s the quotient is n >> s (mul = 0), else
// mul = ceil(2^(32+s) / d) < 2^32, and mulhi(n, mul) >> s is exact because the rounding error of
// mul, below d, times n < 2^31 stays below 2^(32+s).
inline void fa_magic_divisor(uint32_t d, uint32_t* mul, uint32_t* shr) {
    uint32_t s = 0;
    while ((uint64_t(1) << (s + 1)) <= d) ++s;
    *shr = s;
    *mul = (d & (d - 1)) == 0 ? 0u : uint32_t(((uint64_t(1) << (32 + s)) + d - 1) / d);
}

// Launches fa_fwd_ps (fa_fwd_ps.hip) for fp16 / bf16 with D = 64 or 128; alibi: 0 none, 1
// linear, 2 square root.
void launch_fwd_ps(const fa_kargs& a, const fa_ps_args& ps, int D, bool bf16, int alibi, unsigned grid,
                   hipStream_t s);

namespace {

// Work item of this workgroup. Workgroups are dispatched round-robin over the 8 XCDs, each
// with its own L2. Table mode (varlen / prefix): heads are the fastest index, so the blocks
// of one (batch, head) share an XCD when N is a multiple of 8, and items run in the order of
// the planner's table (sequence-major for varlen, longest first for prefix). Fixed-length mode with xcd_major: XCD x = blockIdx % 8
// works through the (batch, head) pairs congruent to x one pair at a time, heaviest q tile
// first, so each XCD streams the K/V of about one pair through its L2 at a time.

__device__ __forceinline__ fa_geom fa_geom_of(const fa_kargs& a, int b) {
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

__device__ __forceinline__ void fa_decode_item(const fa_kargs& a, int& b, int& h, int& qt,
                                               fa_geom& g) {
    const int w = blockIdx.x;
    h = w % a.N;
    const int item = w / a.N;
    if (a.items) {
        b = fa_uniform(a.items[2 * item]);
        qt = fa_uniform(a.items[2 * item + 1]);
    } else if (a.xcd_major) {
        // Pair-major (1): the pairs of XCD x one after another, each heaviest q tile first.
        // Rank-major (2): the heaviest q tile of every pair of XCD x, then the next rank.
        // Grouped rank-major (3): rank-major over four pairs of XCD x at a time.
        const int x = w & 7, slot = w >> 3;
        const int ppx = a.B * a.N / 8;
        int pair, r;
        if (a.xcd_major == 3) {
            // Rank-major within groups of four pairs (the planner keeps (B N / 8) % 4 == 0).
            const int nq = a.n_qtiles_fixed, gr = slot / (4 * nq), jj = slot % (4 * nq);
            pair = (gr * 4 + (jj & 3)) * 8 + x;
            r = jj >> 2;
        } else {
            pair = (a.xcd_major == 2 ? slot % ppx : slot / a.n_qtiles_fixed) * 8 + x;
            r = a.xcd_major == 2 ? slot / ppx : slot % a.n_qtiles_fixed;
        }
        b = pair / a.N;
        h = pair % a.N;
        qt = a.reverse_qt ? a.n_qtiles_fixed - 1 - r : r;
    } else {
        const int r = item / a.B;
        b = item % a.B;
        qt = a.reverse_qt ? a.n_qtiles_fixed - 1 - r : r;
    }
    g = fa_geom_of(a, b);
}

// max / sum of x over the lane pair (l, l ^ 32); both lanes get the same bits.
__device__ __forceinline__ float pair_max(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}


// K and V tiles live in LDS row-major (a row is D/8 chunks of 16 bytes); chunk c of row j
// sits at c ^ swz(j). D = 128 (256-byte rows): swz swaps the two 2-bit fields of j & 15, a
// bijection, so the 16 rows one 16-lane group reads with ds_read_b128 (K) land on 16
// distinct bank groups; and 4 consecutive rows (j & 3 = 0..3) XOR chunk bits 2-3 with
// distinct values, so the 4 rows x 4 chunks that lanes 0-31 touch with a V transpose read
// cover all 16 bank groups once. D = 64 (two 128-byte rows per 256-byte line): the same
// idea on y = j >> 1.
template <int KCH>
__device__ __forceinline__ int fa_swz(int j, int c) {
    if constexpr (KCH == 16) return c ^ (((j & 3) << 2) | ((j >> 2) & 3));
    else {
        const int y = j >> 1;
        return c ^ (((y & 1) << 2) | ((y >> 1) & 3));
    }
}

// Dense-mask tile entries: the kv tile index in the low 24 bits; FA_DENSE_END (past the list)
// names a tile past every key, whose loads read nothing.
constexpr uint32_t FA_DENSE_KT = 0xFFFFFFu;
constexpr uint32_t FA_DENSE_END = 0xFFFFFFFFu;

constexpr int PP_BM = FA_PP_BM;   // 256 query rows per workgroup (8 waves x 32 rows)
constexpr int PP_BN = FA_PP_BN;   // 64 keys per kv tile
constexpr int PP_THREADS = 512;

// Phase barrier: waits for this wave's LDS reads (lgkmcnt 0) but not for its direct-to-LDS
// loads (vmcnt), which are waited for explicitly in the phase before their data is read; a
// memory fence here would wait for those loads too. The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void fa_lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left alone
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Phase barrier that lets this wave's last N LDS reads stay in flight (LDS operations complete
// in order, so everything issued before them has completed). For reads of data that no other
// wave overwrites before the next barrier.
template <int N>
__device__ __forceinline__ void fa_lds_barrier_pending() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));   // lgkmcnt(N); vmcnt and expcnt left alone
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt immediate for vmcnt(n) alone (n < 16).
constexpr int fa_vmcnt(int n) { return 0x0F70 | n; }

}  // namespace

#endif  // FA_FWD_COMMON_H_
