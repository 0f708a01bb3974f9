// mx.hpp — lane and scale formats of the microscaled modes (emily
// lib/emily/quantization.ex, "Defn-native dequantize": the mxfp4, mxfp8 and
// nvfp4 implementations and their lookup tables). No biases; one scale byte
// per group of lanes; w = lane_value * scale_value.
//   mxfp4: 4-bit FP4-E2M1 lanes, groups of 32, FP8-E8M0 scales;
//   mxfp8: 8-bit FP8-E4M3 lanes, groups of 32, FP8-E8M0 scales;
//   nvfp4: 4-bit FP4-E2M1 lanes, groups of 16, FP8-E4M3 scales.
// The pages' E4M3 is MLX's: no code is NaN, 0x7F / 0xFF are +-480.
#pragma once

#include "common.hpp"

namespace qp {

enum : int { MODE_MXFP4 = 1, MODE_MXFP8 = 2, MODE_NVFP4 = 3 };

template <int MODE> struct MxFmt {
    static constexpr int BITS = MODE == MODE_MXFP8 ? 8 : 4;
    static constexpr int GS = MODE == MODE_NVFP4 ? 16 : 32;
    static constexpr bool FP8_LANES = MODE == MODE_MXFP8;
    static constexpr bool E4M3_SCALES = MODE == MODE_NVFP4;
};

// FP8-E4M3 byte (sign, 4 exponent bits of bias 7, 3 mantissa bits, exponent
// field 0 subnormal) as fp32, exactly. Its magnitude bits shifted left by 7
// form the binary16 number of the same mantissa and an exponent 8 lower
// (bias 15 against 7), subnormals included; scaling by 2^8 restores it.
__device__ __forceinline__ float mx_e4m3(uint32_t b)
{
    const float mag =
        (float)__builtin_bit_cast(_Float16, (uint16_t)((b & 0x7Fu) << 7)) * 256.0f;
    return (b & 0x80u) ? -mag : mag;
}

// FP4-E2M1 code (sign bit 3, 2 exponent bits of bias 1, 1 mantissa bit) as
// fp32, exactly: the three magnitude bits shifted left by 9 form the binary16
// number of the same mantissa and an exponent 14 lower (subnormal code 1
// included); scaling by 2^14 restores it.
__device__ __forceinline__ float mx_e2m1(uint32_t c)
{
    const float mag =
        (float)__builtin_bit_cast(_Float16, (uint16_t)((c & 7u) << 9)) * 16384.0f;
    return (c & 8u) ? -mag : mag;
}

template <int MODE>
__device__ __forceinline__ float mx_lane(uint32_t code)
{
    if constexpr (MxFmt<MODE>::FP8_LANES)
        return mx_e4m3(code);
    else
        return mx_e2m1(code);
}

// v times the value of scale byte `byte`. FP8-E8M0 is 2^(byte - 127), applied
// as an exponent shift (v_ldexp_f32): exact, with zero staying zero and
// overflow going to infinity, even for byte 255 (2^128, not an fp32 value).
template <int MODE>
__device__ __forceinline__ float mx_scaled(float v, uint32_t byte)
{
    if constexpr (MxFmt<MODE>::E4M3_SCALES)
        return v * mx_e4m3(byte);
    else
        return __builtin_amdgcn_ldexpf(v, (int)byte - 127);
}

} // namespace qp
