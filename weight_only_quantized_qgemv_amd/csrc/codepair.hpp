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
// 6- and 8-bit codes go through fp32 (v_cvt_f32_ubyteN, exact) and one pack
// for bf16; for fp16 each code byte goes under the exponent byte of 1024 and
// one packed subtraction of 1024 leaves it.
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
//   3-bit: slice j = bytes 3j .. 3j+2 of the unit (codes 8j .. 8j+7, LSB
//          first across the word boundaries); its even codes spread to the
//          bytes of one word and its odd codes to those of another, so the
//          pairs are those of the 4-bit order.
//   6-bit: slice j = bytes 6j .. 6j+5, its two 3-byte halves spread to bytes:
//          pair p holds codes 2p, 2p + 1, the 8-bit order.
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
template <> struct CodeOrder<3> : CodeOrder<4> {};
template <> struct CodeOrder<6> : CodeOrder<8> {};

// Bytes of 3- and 6-bit codes. A 24-bit piece s holds codes at bits 0, w, 2w,
// ... (w = 3 or 6; bits above 24 are ignored). First the upper 12 bits move
// up by 4 (one shift and one bit-field insert), so that the fields at 0, 6,
// 16 and 22 (of this word or of it shifted right by 3) are the ones that go
// to bytes 0..3: bytes 0 and 2 are already in place, and bytes 1 and 3 are
// those of the word shifted left by 2, so one byte permute gathers them. A
// last mask, with the codes complemented by `flip` in the same operation,
// clears the neighbouring fields.
__device__ __forceinline__ uint32_t code_stage(uint32_t s)
{
    return (s & 0xFFFu) | ((s << 4) & ~0xFFFu);
}
__device__ __forceinline__ uint32_t code_gather(uint32_t y, uint32_t flip, uint32_t mask)
{
    return (__builtin_amdgcn_perm(y << 2, y, 0x07020500u) ^ flip) & mask;
}
// The eight 3-bit codes of s: codes 0, 2, 4, 6 to bytes 0..3 of `even`, codes
// 1, 3, 5, 7 to those of `odd`.
__device__ __forceinline__ void code_bytes3(uint32_t s, uint32_t flip, uint32_t& even, uint32_t& odd)
{
    const uint32_t y = code_stage(s);
    even = code_gather(y, flip, 0x07070707u);
    odd = code_gather(y >> 3, flip, 0x07070707u);
}
// The four 6-bit codes of s to bytes 0..3. The empty asm hides that each
// byte is below 64, which otherwise turns the byte conversions that follow
// (v_cvt_f32_ubyteN) into a bit-field extract and a conversion each.
__device__ __forceinline__ uint32_t code_bytes6(uint32_t s, uint32_t flip)
{
    uint32_t v = code_gather(code_stage(s), flip, 0x3F3F3F3Fu);
    asm("" : "+v"(v));
    return v;
}

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
    // Bytes 0, 1 (HI: 2, 3) of v, each a code, as an exact pair: through fp32.
    template <bool HI> static __device__ __forceinline__ uint32_t bytes(uint32_t v)
    {
        return HI ? pack((float)((v >> 16) & 0xFFu), (float)(v >> 24))
                  : pack((float)(v & 0xFFu), (float)((v >> 8) & 0xFFu));
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
    // Bytes 0, 1 (HI: 2, 3) of v, each a code, as an exact pair: the byte
    // permute puts each code c under the exponent byte 0x64, which makes the
    // half 1024 + c exactly (c < 1024), and one packed subtraction of 1024
    // leaves c.
    template <bool HI> static __device__ __forceinline__ uint32_t bytes(uint32_t v)
    {
        const uint32_t h = __builtin_amdgcn_perm(0x64646464u, v, HI ? 0x04030402u : 0x04010400u);
        return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, h) - f16x2_t{1024.0f16, 1024.0f16});
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
    } else if constexpr (BITS == 3) {
        // Slice j (24 bits, codes 8j .. 8j+7) in the low bits of s[j].
        const uint32_t s[4] = {w[0], __builtin_amdgcn_alignbyte(w[1], w[0], 3),
                               __builtin_amdgcn_alignbyte(w[2], w[1], 2), w[2] >> 8};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t even, odd;
            code_bytes3(s[j], flip, even, odd);
            p[4 * j + 0] = C::template fp8<false>(even);
            p[4 * j + 1] = C::template fp8<true>(even);
            p[4 * j + 2] = C::template fp8<false>(odd);
            p[4 * j + 3] = C::template fp8<true>(odd);
        }
    } else if constexpr (BITS == 6) {
        // Codes 4h .. 4h+3 (24 bits) in the low bits of s[h].
        uint32_t s[8];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            s[4 * j + 0] = w[3 * j];
            s[4 * j + 1] = __builtin_amdgcn_alignbyte(w[3 * j + 1], w[3 * j], 3);
            s[4 * j + 2] = __builtin_amdgcn_alignbyte(w[3 * j + 2], w[3 * j + 1], 2);
            s[4 * j + 3] = w[3 * j + 2] >> 8;
        }
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const uint32_t v = code_bytes6(s[h], flip);
            p[2 * h + 0] = C::template bytes<false>(v);
            p[2 * h + 1] = C::template bytes<true>(v);
        }
    } else {
        static_assert(BITS == 8, "2-, 3-, 4-, 6- and 8-bit codes");
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t v = w[i] ^ flip;
            p[2 * i + 0] = C::template bytes<false>(v);
            p[2 * i + 1] = C::template bytes<true>(v);
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
