// common.hpp — device-side helpers shared by the qpack kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace qp {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
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

// Work description of one tile: `count` pairs (at most the tile height) of one expert, taken
// from positions [start, start + count) of the pair list.
struct TileDesc {
    int expert;
    int start;
    int count;
};

// SiLU(z) = z * sigmoid(z), in fp32 (the activation of the fused gate / up
// form; ferrum-kernels `gemv_moe_id_gate_up_silu` docs).
__device__ __forceinline__ float silu_f32(float z)
{
    return z / (1.0f + expf(-z));
}

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1, so the body sees
// I as a compile-time constant (table lookups fold, register arrays are
// indexed statically).
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>)
{
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One DPP-moved copy of v (gfx9 data-parallel primitives); lanes whose row is
// masked off, or whose source is out of range, read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, ROW_MASK, 0xF, true));
}

// Sum over aligned segments of `seg` lanes (1, 2, 4, ..., 64) with DPP adds.
// The total is valid in every lane of the segment for seg <= 16, and in the
// segment's last lane for seg = 32 or 64 (see segment_writer).
__device__ __forceinline__ float segment_reduce(float v, int seg)
{
    if (seg >= 2) v += dpp_f32<0xB1>(v);         // quad_perm [1,0,3,2]: lane ^ 1
    if (seg >= 4) v += dpp_f32<0x4E>(v);         // quad_perm [2,3,0,1]: lane ^ 2
    if (seg >= 8) v += dpp_f32<0x141>(v);        // row_half_mirror: i <-> 7 - i
    if (seg >= 16) v += dpp_f32<0x140>(v);       // row_mirror: i <-> 15 - i
    if (seg >= 32) v += dpp_f32<0x142, 0xA>(v);  // row_bcast15 into rows 1, 3
    if (seg >= 64) v += dpp_f32<0x143, 0xC>(v);  // row_bcast31 into rows 2, 3
    return v;
}
__device__ __forceinline__ bool segment_writer(int lane_in_seg, int seg)
{
    return seg <= 16 ? lane_in_seg == 0 : lane_in_seg == seg - 1;
}

// segment_reduce for N independent values at once and a compile-time segment
// width: the steps are interleaved across the values, so consecutive DPP reads
// never depend on the instruction just before them.
template <int N, int SEG>
__device__ __forceinline__ void reduce_slots(float* v)
{
    if constexpr (SEG >= 2) { for (int i = 0; i < N; ++i) v[i] += dpp_f32<0xB1>(v[i]); }
    if constexpr (SEG >= 4) { for (int i = 0; i < N; ++i) v[i] += dpp_f32<0x4E>(v[i]); }
    if constexpr (SEG >= 8) { for (int i = 0; i < N; ++i) v[i] += dpp_f32<0x141>(v[i]); }
    if constexpr (SEG >= 16) { for (int i = 0; i < N; ++i) v[i] += dpp_f32<0x140>(v[i]); }
    if constexpr (SEG >= 32) { for (int i = 0; i < N; ++i) v[i] += dpp_f32<0x142, 0xA>(v[i]); }
    if constexpr (SEG >= 64) { for (int i = 0; i < N; ++i) v[i] += dpp_f32<0x143, 0xC>(v[i]); }
}

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

// Code C (0..31) of a 32-code unit held in BITS consecutive words.
template <int BITS, int C>
__device__ __forceinline__ uint32_t unit_code(const uint32_t* w)
{
    constexpr int bit = C * BITS, wi = bit / 32, sh = bit % 32;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    if constexpr (sh + BITS <= 32)
        return (w[wi] >> sh) & mask;
    else
        return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & mask;
}

// x & mask, opaque to the optimizer: the byte reads below must stay byte
// conversions (v_cvt_f32_ubyteN) instead of being folded into bit-field
// extracts of the unmasked word.
__device__ __forceinline__ uint32_t and_opaque(uint32_t x, uint32_t mask)
{
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(mask));
    return r;
}

// A unit's 32 codes as bytes, so that each converts with one v_cvt_f32_ubyteN:
// 8-bit codes already are bytes; 4-bit (2-bit) words are split into 2 (4)
// words of one code per byte. 3- and 6-bit codes keep the word form and are
// extracted with a bit-field read.
template <int BITS> struct CodeBytes {
    static constexpr bool BYTEWISE = BITS == 2 || BITS == 4 || BITS == 8;
    static constexpr int NBW = BYTEWISE ? 8 : BITS;   // words after splitting
    static __device__ __forceinline__ void split(const uint32_t (&w)[BITS], uint32_t (&bw)[NBW])
    {
        if constexpr (BITS == 8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) bw[i] = w[i];
        } else if constexpr (BITS == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bw[2 * i] = and_opaque(w[i], 0x0F0F0F0Fu);
                bw[2 * i + 1] = and_opaque(w[i] >> 4, 0x0F0F0F0Fu);
            }
        } else if constexpr (BITS == 2) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int h = 0; h < 4; ++h) bw[4 * i + h] = and_opaque(w[i] >> (2 * h), 0x03030303u);
        } else {
#pragma unroll
            for (int i = 0; i < BITS; ++i) bw[i] = w[i];
        }
    }
    // Code C of the unit as fp32.
    template <int C> static __device__ __forceinline__ float code(const uint32_t (&bw)[NBW])
    {
        if constexpr (BITS == 8) {
            return (float)((bw[C / 4] >> (8 * (C % 4))) & 0xFFu);
        } else if constexpr (BITS == 4) {   // code 8 wi + 2 i + h: byte i of word 2 wi + h
            return (float)((bw[2 * (C / 8) + (C % 2)] >> (8 * ((C % 8) / 2))) & 0xFFu);
        } else if constexpr (BITS == 2) {   // code 16 wi + 4 i + h: byte i of word 4 wi + h
            return (float)((bw[4 * (C / 16) + (C % 4)] >> (8 * ((C % 16) / 4))) & 0xFFu);
        } else {
            return (float)unit_code<BITS, C>(bw);
        }
    }
};

} // namespace qp
