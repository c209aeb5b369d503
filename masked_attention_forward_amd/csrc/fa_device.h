// fa_device.h - small device-side helpers shared by the forward and backward kernels:
// vector types, buffer-resource loads, and the bf16 / fp16 MFMA wrappers.
#ifndef FA_DEVICE_H_
#define FA_DEVICE_H_

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Debug builds (FA_LDS_POISON defined) fill a kernel's LDS tiles with all-ones words before its
// first load: 0xFFFF is a NaN in bf16 and fp16 and 0xFFFFFFFF one in fp32, so a read of any
// byte that no load or store of the kernel wrote (a tile row past a sequence that was not
// zero-filled, say) turns outputs into NaN, even where the value is multiplied by a zero
// probability. The library built this way is a separate file; the tests compare its outputs
// with the normal library's bit for bit. Without the flag FA_POISON_LDS expands to nothing.
#ifdef FA_LDS_POISON
template <typename T, int N>
__device__ __forceinline__ void fa_poison_one(T (&a)[N]) {
    static_assert(sizeof(a) % 4 == 0, "LDS arrays are whole words");
    uint32_t* w = reinterpret_cast<uint32_t*>(a);
    for (int i = int(threadIdx.x); i < int(sizeof(a) / 4); i += int(blockDim.x)) w[i] = 0xFFFFFFFFu;
}
template <typename... A>
__device__ __forceinline__ void fa_poison_lds(A&... a) {
    (fa_poison_one(a), ...);
    __syncthreads();
}
#define FA_POISON_LDS(...) fa_poison_lds(__VA_ARGS__)
#else
#define FA_POISON_LDS(...) \
    do {                   \
    } while (0)
#endif

// Values read from the workspace tables are the same for every lane; readfirstlane keeps them
// in scalar registers (buffer descriptors built from them must be wave-uniform).
__device__ __forceinline__ int fa_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// 32x32x16 MFMA (forward kernels) and rounding of two floats into a packed pair.
template <bool IS_BF16>
struct mfma_io;

template <>
struct mfma_io<true> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        bf16x2 r;
        r.x = (__bf16)x;
        r.y = (__bf16)y;
        return __builtin_bit_cast(uint32_t, r);
    }
};

template <>
struct mfma_io<false> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        f16x2 r;
        r.x = (_Float16)x;
        r.y = (_Float16)y;
        return __builtin_bit_cast(uint32_t, r);
    }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t fa_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 fa_bload(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// s_waitcnt immediate for vmcnt(n), n < 64 (vmcnt bits 3:0 and 15:14; the other counters
// left at their maxima).
constexpr int fa_vmcnt64(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// 16x16x32 MFMA (decode and backward kernels).
template <bool IS_BF16>
struct mfma16_io;

template <>
struct mfma16_io<true> {
    static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <>
struct mfma16_io<false> {
    static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

}  // namespace

#endif  // FA_DEVICE_H_
