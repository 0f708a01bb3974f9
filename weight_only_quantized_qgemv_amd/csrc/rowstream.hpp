// rowstream.hpp — the decode GEMV for 2-, 4- and 8-bit codes with one weight
// row per wave (emily lib/emily/quantization.ex, `quantized_matmul/2`;
// affine codes of `dequantize_defn/1`):
//   y[m, n] = sum_g s'[n,g] * sum_{k in g} x q + b'[n,g] * sum_{k in g} x.
//
// Lane l of a wave takes the 32-code units l, l + 64, ... of the row, so its
// slice of the activation rows is fixed for the whole launch and sits in
// registers. A unit is BITS code words; pair t of a word holds codes t and
// t + 16 / BITS, cut out by one shift and mask-and-or: the code lands in the
// mantissa of OFFSET (bf16 128, fp16 1024, both with a mantissa step of 1),
// giving OFFSET + q exactly. (8-bit codes with bf16 activations exceed the
// bf16 mantissa, so those bytes are converted instead, with no offset.) The
// activation pairs are stored permuted to match. v_dot2 forms
// sum x (OFFSET + q) per unit, the unit's activation sum removes the offset,
// and the group's scale and bias are applied once per unit. D rows are
// loaded before any is reduced.
#pragma once

#include "common.hpp"
#include "gemv_core.hpp"

namespace qp {

struct RowStreamArgs {
    const void* x;              // [M, K] (the rows of this launch)
    const uint32_t* wq;         // [N, K*bits/32]
    const void* scales;         // [N, K/gs]
    const void* biases;
    void* y;                    // [M, N]
    int M, N, K, gs;
    uint32_t units_row;         // K / 32
};

template <int DT> struct RowStreamPair;
template <> struct RowStreamPair<DT_BF16> {
    static constexpr uint32_t MAGIC = 0x43004300u;   // bf16 pair (128, 128)
    static constexpr float OFFSET = 128.0f;
    static __device__ __forceinline__ float dot(uint32_t a, uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, x), acc, false);
    }
};
template <> struct RowStreamPair<DT_F16> {
    static constexpr uint32_t MAGIC = 0x64006400u;   // fp16 pair (1024, 1024)
    static constexpr float OFFSET = 1024.0f;
    static __device__ __forceinline__ float dot(uint32_t a, uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, x),
                                      acc, false);
    }
};

// Rows in flight: about 32 VGPRs of codes.
template <int BITS, int UPL> constexpr int rowstream_depth()
{
    return 32 / (BITS * UPL) < 1 ? 1 : (32 / (BITS * UPL) > 4 ? 4 : 32 / (BITS * UPL));
}

template <int BITS, int DT, int MT, int UPL>
__global__ __launch_bounds__(256) void qgemv_rowstream_kernel(RowStreamArgs a)
{
    using PX = RowStreamPair<DT>;
    using E = Elem<DT>;
    using St = typename E::storage;
    static_assert(BITS == 2 || BITS == 4 || BITS == 8, "codes in whole 16-bit halves");
    constexpr int D = rowstream_depth<BITS, UPL>();
    constexpr int CPW = 32 / BITS;                   // codes per word
    constexpr int HALF = CPW / 2;                    // pairs per word
    constexpr bool CONVERT = BITS == 8 && DT == DT_BF16;
    constexpr float OFFSET = CONVERT ? 0.0f : PX::OFFSET;
    constexpr uint32_t M1 = (1u << BITS) - 1u;
    constexpr uint32_t MASK = M1 | (M1 << 16);
    const int lane = threadIdx.x & 63;
    const int gw = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    const int GW = (int)gridDim.x * 4;

    // Activation pairs of the lane's units, permuted: pair HALF i + t of a
    // unit holds x[CPW i + t] (low) and x[CPW i + t + HALF] (high); and each
    // unit's sum.
    uint32_t xr[MT][UPL][16];
    float xs[MT][UPL];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
            const int u = lane + 64 * j;
            xs[m][j] = 0.0f;
            if (u < (int)a.units_row && m < a.M) {
                const St* p = static_cast<const St*>(a.x) + (int64_t)m * a.K + 32 * u;
                uint32_t raw[16];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const u32x4_t q = reinterpret_cast<const u32x4_t*>(p)[v];
                    raw[4 * v] = q.x; raw[4 * v + 1] = q.y; raw[4 * v + 2] = q.z; raw[4 * v + 3] = q.w;
                }
                // raw[k / 2] holds x[k] (low) and x[k + 1] (high).
#pragma unroll
                for (int i = 0; i < BITS; ++i)
#pragma unroll
                    for (int t = 0; t < HALF; ++t) {
                        const int k0 = CPW * i + t, k1 = k0 + HALF;
                        const uint32_t lo = (raw[k0 / 2] >> (16 * (k0 & 1))) & 0xFFFFu;
                        const uint32_t hi = (raw[k1 / 2] >> (16 * (k1 & 1))) & 0xFFFFu;
                        xr[m][j][HALF * i + t] = lo | (hi << 16);
                    }
#pragma unroll
                for (int k = 0; k < 32; ++k)
                    xs[m][j] += E::to_f32((uint16_t)(raw[k / 2] >> (16 * (k & 1))));
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) xr[m][j][i] = 0u;
            }
        }

    const uint32_t row_bytes = (uint32_t)a.K * BITS / 8;
    const uint32_t groups_row = (uint32_t)(a.K / a.gs);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.wq, (uint32_t)a.N * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales, (uint32_t)a.N * groups_row * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.biases, (uint32_t)a.N * groups_row * 2);
    St* y = static_cast<St*>(a.y);
    uint32_t gofs[UPL];
#pragma unroll
    for (int j = 0; j < UPL; ++j)
        gofs[j] = (uint32_t)((32 * (lane + 64 * j)) / a.gs) * 2;

    for (int r0 = gw * D; r0 < a.N; r0 += GW * D) {
        uint32_t w[D][UPL][BITS];
        St sv[D][UPL], bv[D][UPL];
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int j = 0; j < UPL; ++j) {
                const int u = lane + 64 * j, r = r0 + d;
                const bool live = u < (int)a.units_row && r < a.N;
                buffer_words<BITS, BITS == 8 ? 0 : kStreamPolicy>(
                    rw, live ? (uint32_t)r * row_bytes + (uint32_t)u * (4 * BITS) : OOB, w[d][j]);
                const uint32_t so = live ? (uint32_t)r * groups_row * 2 + gofs[j] : OOB;
                sv[d][j] = buffer_elem<DT>(rs, so);
                bv[d][j] = buffer_elem<DT>(rb, so);
            }
        float acc[D * MT];
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float total = 0.0f;
#pragma unroll
                for (int j = 0; j < UPL; ++j) {
                    float part = 0.0f;
#pragma unroll
                    for (int i = 0; i < BITS; ++i)
#pragma unroll
                        for (int t = 0; t < HALF; ++t) {
                            const uint32_t codes = (w[d][j][i] >> (BITS * t)) & MASK;
                            uint32_t pair;
                            if constexpr (CONVERT)
                                pair = __builtin_bit_cast(
                                    uint32_t, bf16x2_t{(__bf16)(float)(codes & 0xFFu),
                                                       (__bf16)(float)(codes >> 16)});
                            else
                                pair = codes | PX::MAGIC;
                            part = PX::dot(pair, xr[m][j][HALF * i + t], part);
                        }
                    const float s = E::to_f32(sv[d][j]), b = E::to_f32(bv[d][j]);
                    const float qx = part - OFFSET * xs[m][j];
                    total = __builtin_fmaf(s, qx, __builtin_fmaf(b, xs[m][j], total));
                }
                acc[d * MT + m] = total;
            }
        reduce_slots<D * MT, 64>(acc);
        if (lane == 63) {
#pragma unroll
            for (int d = 0; d < D; ++d)
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (r0 + d < a.N && m < a.M)
                        y[(int64_t)m * a.N + r0 + d] = E::from_f32(acc[d * MT + m]);
        }
    }
}

} // namespace qp
