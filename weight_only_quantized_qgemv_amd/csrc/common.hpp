// common.hpp — device-side helpers shared by the qpack kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qp {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Element types, same numbering as qp_dtype.
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int DT> struct Elem;
template <> struct Elem<DT_F32> {
    using storage = float;
    static __device__ __forceinline__ float to_f32(float v) { return v; }
    static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<DT_F16> {
    using storage = uint16_t;
    static __device__ __forceinline__ float to_f32(uint16_t h)
    {
        return (float)__builtin_bit_cast(_Float16, h);
    }
    // Round to nearest even (the hardware conversion in the default mode).
    static __device__ __forceinline__ uint16_t from_f32(float v)
    {
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    }
};
template <> struct Elem<DT_BF16> {
    using storage = uint16_t;
    static __device__ __forceinline__ float to_f32(uint16_t h)
    {
        return __uint_as_float((uint32_t)h << 16);
    }
    static __device__ __forceinline__ uint16_t from_f32(float v)
    {
        return __builtin_bit_cast(uint16_t, (__bf16)v);
    }
};

// Sum over aligned segments of SEG lanes (SEG a power of two <= 64); every
// lane of a segment ends with the segment's total.
template <int SEG>
__device__ __forceinline__ float segment_sum(float v)
{
#pragma unroll
    for (int off = 1; off < SEG; off <<= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// Read-once streaming load of NW consecutive u32 words (weights are touched
// exactly once per launch, so they bypass reuse in the caches).
template <int NW>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t (&w)[NW])
{
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW; i += 4) {
            u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + i));
            w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
        }
    } else if constexpr (NW % 2 == 0) {
#pragma unroll
        for (int i = 0; i < NW; i += 2) {
            u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p + i));
            w[i] = v.x; w[i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i)
            w[i] = __builtin_nontemporal_load(p + i);
    }
}

// Code `c` (0..31) of a 32-code unit held in BITS consecutive words.
template <int BITS>
__device__ __forceinline__ uint32_t unit_code(const uint32_t* w, int c)
{
    const int bit = c * BITS, wi = bit / 32, sh = bit % 32;
    const uint32_t mask = (1u << BITS) - 1u;
    if (sh + BITS <= 32)
        return (w[wi] >> sh) & mask;
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & mask;
}

} // namespace qp
