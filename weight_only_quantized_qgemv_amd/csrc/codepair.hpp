// codepair.hpp — exact 16-bit operands from packed codes, and the per-group
// choice of which end of the quantization grid the folded bias sits at.
//
// The affine weight of code q in group g is w' = q * s'_g + b'_g (emily
// lib/emily/quantization.ex, `dequantize_defn/1`). The product kernels fold it
// out of their inner loops,
//     sum_k x_k w'_k = s' * sum_k q_k x_k + b' * sum_k x_k       (per group),
// so the codes must reach the dot products as exact values and the two folded
// sums must not carry an error that is large next to sum_k |x_k| |w'_k|.
//
// Exact codes. gfx950 converts FP8-E4M3 and FP4-E2M1 pairs to bf16 / fp16 in
// one instruction, with an fp32 scale. E4M3 bytes 0..15 are the subnormals
// m * 2^-9 and the first normal binade (8 + m) * 2^-9, so a byte holding a code
// q < 16 converts to exactly q * 2^-9, and to q with the scale 2^9. E2M1
// nibbles 0..3 are 0, 0.5, 1, 1.5: a 2-bit code converts to q with the scale 2.
// 8-bit codes go through fp32 (v_cvt_f32_ubyteN, exact) and one pack.
//
// Unit layout. A unit is 32 consecutive codes of a row (BITS words). Its 16
// pairs come out in the order below; the activation pairs a kernel dots them
// with must be built in the same order (lo_code / hi_code):
//   4-bit: word i, pair 4i + t: lo = w & 0x0F0F0F0F holds codes 8i + 2b in its
//          bytes, hi = (w >> 4) & 0x0F0F0F0F codes 8i + 2b + 1; t = 0, 1 take
//          bytes (0,1), (2,3) of lo, t = 2, 3 those of hi.
//   2-bit: word i, pair 8i + t: lo = w & 0x33333333 holds code 16i + 2n in
//          nibble n, hi = (w >> 2) & 0x33333333 code 16i + 2n + 1; t = 0..3
//          take byte t of lo, t = 4..7 byte t - 4 of hi (low nibble first).
//   8-bit: word i, pair 2i + t: bytes 2t, 2t + 1 of word i.
//
// Orientation. With b'' = fl(fl(qmax * s') + b') the weight of the top code
// (computed as the dequantization computes it), the same group is also
//     w' = -s' * (qmax - q) + b''   (to one rounding of b''),
// and complementing every code (q -> qmax - q, an xor of the code bits) is
// free in the split above. The kernels take the end whose bias is smaller in
// magnitude. For a group whose weights all have one sign (zeros included:
// pruned rows, one spike among zeros, groups entirely below zero) that makes
// the bias and the scaled codes agree in sign, so the folded sum has no
// cancellation and its error is a few fp32 roundings of sum |x| |w'|. A group
// of constant zeros has s' = FLT_EPSILON, b' = +0 and codes 0: its dot
// products are exactly +0 and so is its contribution.
#pragma once

#include "common.hpp"

namespace qp {

template <int BITS> struct CodeOrder;
template <> struct CodeOrder<4> {
    static constexpr int lo_code(int p)
    {
        return 8 * (p / 4) + (p % 4 == 0 ? 0 : p % 4 == 1 ? 4 : p % 4 == 2 ? 1 : 5);
    }
    static constexpr int hi_code(int p) { return lo_code(p) + 2; }
};
template <> struct CodeOrder<2> {
    static constexpr int lo_code(int p) { return 16 * (p / 8) + 4 * (p % 4) + (p % 8) / 4; }
    static constexpr int hi_code(int p) { return lo_code(p) + 2; }
};
template <> struct CodeOrder<8> {
    static constexpr int lo_code(int p) { return 4 * (p / 2) + 2 * (p % 2); }
    static constexpr int hi_code(int p) { return lo_code(p) + 1; }
};

template <int DT> struct ExactCvt;
template <> struct ExactCvt<DT_BF16> {
    template <bool HI> static __device__ __forceinline__ uint32_t fp8(uint32_t w)
    {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, HI));
    }
    template <int B> static __device__ __forceinline__ uint32_t fp4(uint32_t w)
    {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 2.0f, B));
    }
    static __device__ __forceinline__ uint32_t pack(float lo, float hi)
    {
        return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
    }
};
template <> struct ExactCvt<DT_F16> {
    template <bool HI> static __device__ __forceinline__ uint32_t fp8(uint32_t w)
    {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 512.0f, HI));
    }
    template <int B> static __device__ __forceinline__ uint32_t fp4(uint32_t w)
    {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, B));
    }
    static __device__ __forceinline__ uint32_t pack(float lo, float hi)
    {
        return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)lo, (_Float16)hi});
    }
};

// The 16 exact code pairs of one unit (BITS words), every code first
// complemented when `flip` is all ones (flip is 0 or ~0).
template <int BITS, int DT>
__device__ __forceinline__ void code_pairs(const uint32_t* w, uint32_t flip, uint32_t (&p)[16])
{
    using C = ExactCvt<DT>;
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = (w[i] ^ flip) & 0x0F0F0F0Fu;
            const uint32_t hi = ((w[i] >> 4) ^ flip) & 0x0F0F0F0Fu;
            p[4 * i + 0] = C::template fp8<false>(lo);
            p[4 * i + 1] = C::template fp8<true>(lo);
            p[4 * i + 2] = C::template fp8<false>(hi);
            p[4 * i + 3] = C::template fp8<true>(hi);
        }
    } else if constexpr (BITS == 2) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t lo = (w[i] ^ flip) & 0x33333333u;
            const uint32_t hi = ((w[i] >> 2) ^ flip) & 0x33333333u;
            p[8 * i + 0] = C::template fp4<0>(lo);
            p[8 * i + 1] = C::template fp4<1>(lo);
            p[8 * i + 2] = C::template fp4<2>(lo);
            p[8 * i + 3] = C::template fp4<3>(lo);
            p[8 * i + 4] = C::template fp4<0>(hi);
            p[8 * i + 5] = C::template fp4<1>(hi);
            p[8 * i + 6] = C::template fp4<2>(hi);
            p[8 * i + 7] = C::template fp4<3>(hi);
        }
    } else {
        static_assert(BITS == 8, "2-, 4- and 8-bit codes");
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t v = w[i] ^ flip;
            p[2 * i + 0] = C::pack((float)(v & 0xFFu), (float)((v >> 8) & 0xFFu));
            p[2 * i + 1] = C::pack((float)((v >> 16) & 0xFFu), (float)(v >> 24));
        }
    }
}

// fl(fl(q * s) + b): the weight of code q as the dequantization forms it, a
// rounded product and then a rounded sum (no fused multiply-add).
__device__ __forceinline__ float affine_weight(float q, float s, float b)
{
#pragma clang fp contract(off)
    return q * s + b;
}

// Folded scale and bias of one group, oriented as above: the group's unit
// sums are then  s_eff * sum (q or qmax - q) x + b_eff * sum x, with the codes
// complemented when `flip` is ~0.
struct Orient {
    float s, b;
    uint32_t flip;
};
template <int BITS>
__device__ __forceinline__ Orient orient(float s, float b)
{
    constexpr float QMAX = (float)((1 << BITS) - 1);
    const float top = affine_weight(QMAX, s, b);
    const bool f = __builtin_fabsf(top) < __builtin_fabsf(b);
    return Orient{f ? -s : s, f ? top : b, f ? ~0u : 0u};
}

} // namespace qp
