// fa_kv_cache.hip - paged KV cache scatter for gfx950 and its C ABI entry point.
//
// "aclnnScatterPaKvCache" (ops-transformer doc), sections "功能说明" (scenarios two, six and
// seven) and "约束说明": token t of key [num_tokens, N, Dk] (and value [num_tokens, N, Dv])
// goes to cache slot slot_mapping[t] = block * block_size + offset, for every head, in a
// "Norm" cache [num_blocks, block_size, N, D] or an "NHSD" cache [num_blocks, N, block_size, D].
// Element types are copied as raw bytes (1, 2 or 4 bytes per element).
//
// A Norm slot row (N * D elements) is contiguous in the cache, an NHSD slot is N rows of D
// elements block_size * D apart; either way the source token row is contiguous. Threads move
// the widest chunk (16, 8, 4, 2 or 1 bytes) that every size and base address allows. The copy
// is HBM-bound: it reads and writes each byte once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>

#include "../../include/fa.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int C>
struct chunk_t;
template <>
struct chunk_t<16> { typedef u32x4 type; };
template <>
struct chunk_t<8> { typedef u32x2 type; };
template <>
struct chunk_t<4> { typedef uint32_t type; };
template <>
struct chunk_t<2> { typedef uint16_t type; };
template <>
struct chunk_t<1> { typedef uint8_t type; };

struct kv_scatter_args {
    const char* key;
    const char* value;
    char* key_cache;
    char* value_cache;
    const void* slots;
    int64_t num_heads, block_size, n_slots;
    int64_t k_row, v_row;   // bytes of one head's row (D * elem)
    int32_t slot64;         // slot_mapping holds int64 (else int32)
    int32_t nhsd;
};

// Slot-row destination offset (bytes) of head h. Norm: ((block * block_size + offset) * N + h) * row;
// NHSD: ((block * N + h) * block_size + offset) * row.
__device__ __forceinline__ int64_t slot_offset(int64_t row, int64_t heads, int64_t block_size, int64_t block,
                                               int64_t offset, int h, bool nhsd) {
    return nhsd ? ((block * heads + h) * block_size + offset) * row
                : ((block * block_size + offset) * heads + h) * row;
}

// A work unit is one segment of 256 chunks of one token's K row or V row (all heads): each
// thread moves one chunk. Units are ordered tensor-major (every K unit, then every V unit; in
// each, token-major), and a workgroup walks them with the grid's stride (one unit per
// workgroup unless the grid is capped). Tensor-major keeps each phase on one source stream
// and one cache, which measured a few percent faster than alternating K and V per token. Small units keep many workgroups in flight: on gfx950 a copy that gives each
// thread one 16-byte chunk sustains more HBM bandwidth than one that gives it several. The
// chunk load does not depend on the slot, so both loads are in flight together. Source and
// cache bytes are each touched once, so both sides are streamed past the caches.
template <int C>
__global__ __launch_bounds__(256) void fa_kv_scatter(const kv_scatter_args a, int64_t units, int32_t ksegs,
                                                     int32_t vsegs, int64_t kunits) {
    typedef typename chunk_t<C>::type T;
    const bool nhsd = a.nhsd != 0;
    const int heads = int(a.num_heads);
    // The host keeps heads * row below 2^31.
    const int kper = int(a.k_row / C), vper = int(a.v_row / C);
    const int ktot = kper * heads, vtot = a.value_cache ? vper * heads : 0;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const bool isv = u >= kunits;
        const int64_t r = isv ? u - kunits : u;
        const int32_t nseg = isv ? vsegs : ksegs;
        const int64_t t = r / nseg;
        const int c = int(r - t * nseg) * 256 + int(threadIdx.x);
        const int tot = isv ? vtot : ktot;
        const char* src = isv ? a.value + t * a.num_heads * a.v_row : a.key + t * a.num_heads * a.k_row;
        T x{};
        if (c < tot) x = __builtin_nontemporal_load(reinterpret_cast<const T*>(src) + c);
        const int64_t slot = a.slot64 ? static_cast<const int64_t*>(a.slots)[t]
                                      : int64_t(static_cast<const int32_t*>(a.slots)[t]);
        // A slot outside the cache (e.g. -1 for padding) writes nothing.
        if (slot < 0 || slot >= a.n_slots || c >= tot) continue;
        const int64_t block = slot / a.block_size, offset = slot % a.block_size;
        const int per = isv ? vper : kper;
        const int h = c / per, w = c % per;
        const int64_t row = isv ? a.v_row : a.k_row;
        char* cache = isv ? a.value_cache : a.key_cache;
        T* dst = reinterpret_cast<T*>(cache + slot_offset(row, heads, a.block_size, block, offset, h, nhsd)) + w;
        __builtin_nontemporal_store(x, dst);
    }
}

// Grid cap: FA_SCATTER_GRID (tests use it to drive the grid-stride loop), else 2^30.
int64_t scatter_grid_cap() {
    const char* e = std::getenv("FA_SCATTER_GRID");
    if (e) {
        const long long v = std::atoll(e);
        if (v >= 1 && v <= (1ll << 30)) return v;
    }
    return int64_t(1) << 30;
}

int chunk_bytes(const kv_scatter_args& a) {
    uintptr_t m = uintptr_t(a.k_row) | uintptr_t(a.key) | uintptr_t(a.key_cache);
    if (a.value_cache) m |= uintptr_t(a.v_row) | uintptr_t(a.value) | uintptr_t(a.value_cache);
    for (int c = 16; c > 1; c >>= 1)
        if ((m & uintptr_t(c - 1)) == 0) return c;
    return 1;
}

}  // namespace

extern "C" fa_status fa_scatter_kv_cache(const void* key, const void* value, void* key_cache,
                                         void* value_cache, const void* slot_mapping,
                                         const fa_kv_cache_dims* dims, int32_t cache_layout,
                                         void* stream) {
    if (!dims) return FA_ERR_NULLPTR;
    const fa_kv_cache_dims& d = *dims;
    if (cache_layout != FA_CACHE_NORM && cache_layout != FA_CACHE_NHSD) return FA_ERR_PARAM_INVALID;
    if (d.num_tokens < 0 || d.num_heads < 1 || d.k_head_size < 1 || d.num_blocks < 1 || d.block_size < 1)
        return FA_ERR_PARAM_INVALID;
    if (d.elem_bytes != 1 && d.elem_bytes != 2 && d.elem_bytes != 4) return FA_ERR_PARAM_INVALID;
    if (d.slot_bytes != 4 && d.slot_bytes != 8) return FA_ERR_PARAM_INVALID;
    const bool has_v = value != nullptr || value_cache != nullptr;
    if (has_v && d.v_head_size < 1) return FA_ERR_PARAM_INVALID;
    // Sizes: every byte offset must fit in int64 with room to spare.
    const int64_t lim = int64_t(1) << 40;
    if (d.num_tokens > lim || d.num_heads > (1 << 16) || d.k_head_size > (1 << 20) || d.v_head_size > (1 << 20) ||
        d.num_blocks > lim || d.block_size > (1 << 24) || d.num_blocks * d.block_size > lim)
        return FA_ERR_UNSUPPORTED;
    if (d.num_tokens == 0) return FA_OK;
    if (!key || !key_cache || !slot_mapping) return FA_ERR_NULLPTR;
    if (has_v && (!value || !value_cache)) return FA_ERR_NULLPTR;
    if (d.num_tokens >= (int64_t(1) << 31)) return FA_ERR_UNSUPPORTED;
    if (d.num_heads * d.k_head_size * d.elem_bytes >= (int64_t(1) << 31) ||
        (has_v && d.num_heads * d.v_head_size * d.elem_bytes >= (int64_t(1) << 31)))
        return FA_ERR_UNSUPPORTED;

    kv_scatter_args a{};
    a.key = static_cast<const char*>(key);
    a.value = static_cast<const char*>(value);
    a.key_cache = static_cast<char*>(key_cache);
    a.value_cache = has_v ? static_cast<char*>(value_cache) : nullptr;
    a.slots = slot_mapping;
    a.num_heads = d.num_heads;
    a.block_size = d.block_size;
    a.n_slots = d.num_blocks * d.block_size;
    a.k_row = d.k_head_size * d.elem_bytes;
    a.v_row = has_v ? d.v_head_size * d.elem_bytes : 0;
    a.slot64 = d.slot_bytes == 8;
    a.nhsd = cache_layout == FA_CACHE_NHSD;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int cb = chunk_bytes(a);
    const int64_t kchunks = d.num_heads * a.k_row / cb, vchunks = has_v ? d.num_heads * a.v_row / cb : 0;
    const int32_t ksegs = int32_t((kchunks + 255) / 256), vsegs = int32_t((vchunks + 255) / 256);
    const int64_t kunits = d.num_tokens * ksegs, units = kunits + d.num_tokens * vsegs;
    const dim3 grid(unsigned(std::min<int64_t>(units, scatter_grid_cap()))), block(256);
    (void)hipGetLastError();
    switch (cb) {
        case 16: fa_kv_scatter<16><<<grid, block, 0, s>>>(a, units, ksegs, vsegs, kunits); break;
        case 8: fa_kv_scatter<8><<<grid, block, 0, s>>>(a, units, ksegs, vsegs, kunits); break;
        case 4: fa_kv_scatter<4><<<grid, block, 0, s>>>(a, units, ksegs, vsegs, kunits); break;
        case 2: fa_kv_scatter<2><<<grid, block, 0, s>>>(a, units, ksegs, vsegs, kunits); break;
        default: fa_kv_scatter<1><<<grid, block, 0, s>>>(a, units, ksegs, vsegs, kunits); break;
    }
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
