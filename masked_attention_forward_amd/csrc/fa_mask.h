// fa_mask.h - mask geometry shared by the host planner and the device kernels.
//
// Every sparseMode except 1 makes the visible columns of query row i (batch-local) one
// contiguous interval. With per-batch integers a, c, f:
//
//     lo(i) = i + a,   hi(i) = max(i + c, f),   visible iff lo(i) <= j <= hi(i), 0 <= j < Skv_b.
//
// This is the rule set of "sparseMode介绍" (sections sparseMode=0..8) restated as interval
// bounds; off = Skv_b - Sq_b is the bottom-right alignment of "压缩mask" (the operator derives
// the alignment from kvSeqLen and qSeqLen):
//   mode 0:    a = -pre,        c = next,        f = -BIG  (offsets from the top-left)
//   mode 2:    a = -BIG,        c = 0,           f = -BIG
//   mode 3:    a = -BIG,        c = off,         f = -BIG
//   mode 4:    a = off - pre,   c = off + next,  f = -BIG  (offsets from the bottom-right)
//   mode 5/6:  a = -BIG,        c = off,         f = prefix_b - 1
//   mode 7/8:  the band batch as mode 4, the others as mode 3 / mode 2
//   mode 1:    a = -BIG,        c = +BIG,        f = -BIG  (every column; the dense mask decides)
// pre and next are clamped to +-FA_LIM by the planner, which also guarantees a <= c
// (pre + next >= 0), so the union of the intervals of consecutive non-empty rows has no gap.
// That makes the kv-tile range of a q tile exact: every tile in it holds a visible entry.
#ifndef FA_MASK_H_
#define FA_MASK_H_

#include <stdint.h>

#if defined(__HIPCC__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

#define FA_BIG (1 << 30)
#define FA_LIM (1 << 29)        // |pre|, |next| clamp; sequence lengths stay below 2^28
#define FA_MAX_SEQ (1 << 28)

// Per-batch geometry. Token offsets are used by the packed TND layout (0 otherwise).
struct fa_geom {
    int32_t q_start, kv_start;
    int32_t sq, skv;
    int32_t a, c, f;
    int32_t pad;
};

FA_HD int32_t fa_imin(int32_t x, int32_t y) { return x < y ? x : y; }
FA_HD int32_t fa_imax(int32_t x, int32_t y) { return x > y ? x : y; }

// First visible column of row i, clipped at 0 (may exceed hi when the row is empty).
FA_HD int32_t fa_row_lo(const fa_geom& g, int32_t i) { return fa_imax(i + g.a, 0); }
// Last visible column of row i, clipped at Skv - 1.
FA_HD int32_t fa_row_hi(const fa_geom& g, int32_t i) {
    return fa_imin(fa_imax(i + g.c, g.f), g.skv - 1);
}

// kv tiles [begin, end) a q tile with rows i0..i1 (inclusive, i1 < sq) has to visit.
struct fa_kv_range {
    int32_t begin, end;
};

FA_HD fa_kv_range fa_tile_kv_range(const fa_geom& g, int32_t i0, int32_t i1, int32_t bn) {
    fa_kv_range r = {0, 0};
    if (g.skv <= 0 || i1 < i0) return r;
    // Rows with a visible column: hi(i) >= 0 and lo(i) <= Skv - 1 (a <= c does the rest).
    const int32_t r_lo = (g.f >= 0) ? 0 : fa_imax(-g.c, 0);
    const int32_t r_hi = fa_imin(g.sq - 1, g.skv - 1 - g.a);
    const int32_t p = fa_imax(i0, r_lo);
    const int32_t q = fa_imin(i1, r_hi);
    if (p > q) return r;
    r.begin = fa_row_lo(g, p) / bn;
    r.end = fa_row_hi(g, q) / bn + 1;
    return r;
}

// True when every (row, column) of the tile rows i0..i1 x columns j0..j0+bn-1 is visible
// and inside the sequence, so the kernel can skip per-element masking.
FA_HD bool fa_tile_full(const fa_geom& g, int32_t i0, int32_t i1, int32_t j0, int32_t bn) {
    const int32_t j1 = j0 + bn;
    return j1 <= g.skv && i1 + g.a <= j0 && fa_imax(i0 + g.c, g.f) >= j1 - 1;
}

#endif  // FA_MASK_H_
