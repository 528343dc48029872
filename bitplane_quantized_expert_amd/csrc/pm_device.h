// Device helpers shared by the kernel sources of libpm (gfx950, 64-wide
// wavefronts): DPP reductions, wave-uniform values, vector and address-space
// types.  Internal linkage: every source gets its own copy.
#pragma once

#include <hip/hip_runtime.h>

namespace pm {
namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kRowsPerBlock = kBlock / kWave;

template <int CTRL, int ROW_MASK>
__device__ inline float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                           false));
}

// Sum over each 16-lane row; every lane of the row gets the row's sum.
__device__ inline float row16_sum(float v) {
    v += dpp<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141, 0xF>(v);   // row_half_mirror
    v += dpp<0x140, 0xF>(v);   // row_mirror
    return v;
}

// Sum over each 32-lane half of the wave; the total lands in lanes 16..31
// (first half) and 48..63 (second half).
__device__ inline float half_sum(float v) {
    v = row16_sum(v);
    v += dpp<0x142, 0xA>(v);   // row_bcast15 into rows 1 and 3
    return v;
}

// Sum over the wave; the total lands in lane 63.
__device__ inline float wave_sum(float v) {
    v = half_sum(v);
    v += dpp<0x143, 0xC>(v);   // row_bcast31 into rows 2 and 3
    return v;
}

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Values the whole wave shares, made explicit so that they live in scalar
// registers: arguments of out-of-line functions and values read from LDS
// arrive in vector registers.
__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline float uni_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ inline uint64_t uni64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    return (uint64_t(hi) << 32) | lo;
}
template <class T>
__device__ inline T* uni_ptr(T* p) {
    return reinterpret_cast<T*>(uni64(reinterpret_cast<uint64_t>(p)));
}

typedef __attribute__((address_space(3))) float lds_float;
// Global-memory views: in out-of-line functions a plain pointer would be
// generic and its loads flat_load, which also count against the LDS wait
// counter and would serialise the prefetch with the table lookups.
typedef __attribute__((address_space(1))) const float g_f32;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const f32x4 g_f32x4;
typedef __attribute__((address_space(1))) float g_f32_out;

inline unsigned grid_for(size_t n, int per) { return unsigned((n + per - 1) / per); }

}  // namespace
}  // namespace pm
