// dequantize.hip — the dense weight from packed codes, scales and biases
// (emily lib/emily/quantization.ex, "Defn-native dequantize":
// `dequantize_defn/1`, its affine `dequantize_impl`, and
// `QuantizedWeight.to_dense/1`, whose math it shares). Lane i of a row sits
// at bits [i*bits, i*bits + bits) of the row's little-endian u32 stream,
// g = i / gs, and w = lane * scales[g] + biases[g].
//
// Two output forms:
//  - fp32: fp32(q) * s + b, a multiply and then an add in fp32 (the weight
//    the quantized product is defined on);
//  - the scales' own 16-bit type T (the pages cast the codes to the scales'
//    type before the affine step): the product and then the sum, each
//    rounded to nearest-even in T. Both are taken in fp32 and rounded to T,
//    which gives the correctly rounded result of T: q * s is exact in fp32
//    (at most 8 + 11 significant bits), and an fp32 sum of two values of T
//    rounds to the same value of T as the exact sum (24 >= 2 * 11 + 2).
//
// The kernel is bound by HBM: each thread turns 8 consecutive codes of a row
// into one 16-byte (16-bit output) or 32-byte (fp32) run of the output, and
// the lanes of a wave take consecutive runs, so the code loads and the output
// stores are both contiguous across the wave.
#include "common.hpp"
#include "launch.hpp"
#include "mx.hpp"

namespace qp {

#pragma clang fp contract(off)

namespace {

constexpr int kThreads = 256;
constexpr int kRunsPerThread = 4;   // independent 8-code runs in flight per thread

template <int BITS, int SDT, int ODT, bool VEC>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    const uint32_t* __restrict__ wq, const typename Elem<SDT>::storage* __restrict__ scales,
    const typename Elem<SDT>::storage* __restrict__ biases, uint32_t runs, uint32_t runs_row,
    uint32_t words_row, uint32_t groups_row, int run_group_shift,
    typename Elem<ODT>::storage* __restrict__ out)
{
    using SE = Elem<SDT>;
    using OE = Elem<ODT>;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    constexpr int U = kRunsPerThread;
    const uint32_t first = blockIdx.x * (uint32_t)(kThreads * U) + threadIdx.x;

    // All loads first, each thread's U runs in flight together: a run past
    // the end reads the last run instead (in bounds) and stores nothing.
    uint32_t lo[U], hi[U], sh[U];
    typename SE::storage s_raw[U], b_raw[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        uint32_t r = first + (uint32_t)(j * kThreads);
        r = r < runs ? r : runs - 1u;
        const uint32_t row = r / runs_row, rc = r - row * runs_row;
        // The run's 8 * BITS bits start at bit 8 * BITS * rc of the row.
        const uint32_t bit = rc * (8u * BITS);
        const uint32_t* p = wq + (size_t)row * words_row + (bit >> 5);
        sh[j] = bit & 31u;
        lo[j] = __builtin_nontemporal_load(p);
        hi[j] = 0u;
        if (sh[j] + 8u * BITS > 32u)   // the run crosses into the next word of the row
            hi[j] = __builtin_nontemporal_load(p + 1);
        const size_t g = (size_t)row * groups_row + (rc >> run_group_shift);
        s_raw[j] = scales[g];
        b_raw[j] = biases[g];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const uint32_t r = first + (uint32_t)(j * kThreads);
        if (r >= runs)
            continue;
        const float s = SE::to_f32(s_raw[j]), b = SE::to_f32(b_raw[j]);
        const uint64_t window = ((((uint64_t)hi[j]) << 32) | lo[j]) >> sh[j];
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q = (float)((uint32_t)(window >> (i * BITS)) & mask);
            if constexpr (ODT == DT_F32) {
                const float prod = q * s;
                v[i] = prod + b;
            } else {
                const float prod = OE::to_f32(OE::from_f32(q * s));
                v[i] = prod + b;
            }
        }
        typename OE::storage* o = out + (size_t)r * 8;
        if constexpr (ODT == DT_F32) {
            if constexpr (VEC) {
                reinterpret_cast<float4*>(o)[0] = make_float4(v[0], v[1], v[2], v[3]);
                reinterpret_cast<float4*>(o)[1] = make_float4(v[4], v[5], v[6], v[7]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = v[i];
            }
        } else {
            uint16_t h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                h[i] = OE::from_f32(v[i]);
            if constexpr (VEC) {
                u32x4_t w;
                w.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                w.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
                w.z = (uint32_t)h[4] | ((uint32_t)h[5] << 16);
                w.w = (uint32_t)h[6] | ((uint32_t)h[7] << 16);
                *reinterpret_cast<u32x4_t*>(o) = w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = h[i];
            }
        }
    }
}

template <int BITS, int SDT, int ODT>
hipError_t run_dequantize(const DequantArgs& a, hipStream_t st)
{
    using S = typename Elem<SDT>::storage;
    using O = typename Elem<ODT>::storage;
    const int64_t runs_row = a.K / 8, words_row = a.K * BITS / 32, groups_row = a.K / a.gs;
    const int run_group_shift = __builtin_ctz((unsigned)a.gs) - 3;
    const bool vec = reinterpret_cast<uintptr_t>(a.out) % 16 == 0;
    // 32-bit run indices: launch at most 2^30 runs (whole rows) at a time.
    const int64_t rows_per_launch = ((int64_t)1 << 30) / runs_row;
    for (int64_t r0 = 0; r0 < a.N; r0 += rows_per_launch) {
        const int64_t rows = a.N - r0 < rows_per_launch ? a.N - r0 : rows_per_launch;
        const uint32_t runs = (uint32_t)(rows * runs_row);
        const uint32_t blocks = (runs + kThreads * kRunsPerThread - 1) / (kThreads * kRunsPerThread);
        const uint32_t* wq = a.wq + r0 * words_row;
        const S* sc = static_cast<const S*>(a.scales) + r0 * groups_row;
        const S* bi = static_cast<const S*>(a.biases) + r0 * groups_row;
        O* out = static_cast<O*>(a.out) + r0 * a.K;
        if (vec)
            hipLaunchKernelGGL((dequantize_kernel<BITS, SDT, ODT, true>), dim3(blocks),
                               dim3(kThreads), 0, st, wq, sc, bi, runs, (uint32_t)runs_row,
                               (uint32_t)words_row, (uint32_t)groups_row, run_group_shift, out);
        else
            hipLaunchKernelGGL((dequantize_kernel<BITS, SDT, ODT, false>), dim3(blocks),
                               dim3(kThreads), 0, st, wq, sc, bi, runs, (uint32_t)runs_row,
                               (uint32_t)words_row, (uint32_t)groups_row, run_group_shift, out);
        if (hipError_t e = hipGetLastError(); e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <int BITS>
hipError_t run_dequantize_bits(const DequantArgs& a, hipStream_t st)
{
    if (a.odt == DT_F32) {
        switch (a.sdt) {
        case DT_F32: return run_dequantize<BITS, DT_F32, DT_F32>(a, st);
        case DT_F16: return run_dequantize<BITS, DT_F16, DT_F32>(a, st);
        case DT_BF16: return run_dequantize<BITS, DT_BF16, DT_F32>(a, st);
        }
    } else if (a.odt == a.sdt) {
        switch (a.sdt) {
        case DT_F16: return run_dequantize<BITS, DT_F16, DT_F16>(a, st);
        case DT_BF16: return run_dequantize<BITS, DT_BF16, DT_BF16>(a, st);
        }
    }
    return hipErrorInvalidValue;
}

// Microscaled modes: w = lane * scale, exact in fp32 (at most 4 significant
// bits from the lane and a power of two or 4 bits from the scale, down to
// 2^-136), then rounded once to the output type. A run is 8 lanes: one word
// of 4-bit lanes, two of 8-bit lanes, all inside one group.
template <int MODE, int ODT, bool VEC>
__global__ __launch_bounds__(kThreads) void dequantize_mx_kernel(
    const uint32_t* __restrict__ wq, const uint8_t* __restrict__ scales, uint32_t runs,
    uint32_t runs_row, uint32_t words_row, uint32_t groups_row,
    typename Elem<ODT>::storage* __restrict__ out)
{
    using F = MxFmt<MODE>;
    using OE = Elem<ODT>;
    constexpr int U = kRunsPerThread;
    constexpr int WPR = F::BITS / 4;          // words per run
    constexpr int RPG = F::GS / 8;            // runs per group
    const uint32_t first = blockIdx.x * (uint32_t)(kThreads * U) + threadIdx.x;

    uint32_t w[U][WPR], sb[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        uint32_t r = first + (uint32_t)(j * kThreads);
        r = r < runs ? r : runs - 1u;       // in bounds; past-the-end runs store nothing
        const uint32_t row = r / runs_row, rc = r - row * runs_row;
        const uint32_t* p = wq + (size_t)row * words_row + (size_t)rc * WPR;
#pragma unroll
        for (int i = 0; i < WPR; ++i)
            w[j][i] = __builtin_nontemporal_load(p + i);
        sb[j] = scales[(size_t)row * groups_row + rc / RPG];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const uint32_t r = first + (uint32_t)(j * kThreads);
        if (r >= runs)
            continue;
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t code = (w[j][(i * F::BITS) / 32] >> ((i * F::BITS) % 32)) &
                                  ((1u << F::BITS) - 1u);
            v[i] = mx_scaled<MODE>(mx_lane<MODE>(code), sb[j]);
        }
        typename OE::storage* o = out + (size_t)r * 8;
        if constexpr (ODT == DT_F32) {
            if constexpr (VEC) {
                reinterpret_cast<float4*>(o)[0] = make_float4(v[0], v[1], v[2], v[3]);
                reinterpret_cast<float4*>(o)[1] = make_float4(v[4], v[5], v[6], v[7]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = v[i];
            }
        } else {
            uint16_t h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                h[i] = OE::from_f32(v[i]);
            if constexpr (VEC) {
                u32x4_t q;
                q.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                q.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
                q.z = (uint32_t)h[4] | ((uint32_t)h[5] << 16);
                q.w = (uint32_t)h[6] | ((uint32_t)h[7] << 16);
                *reinterpret_cast<u32x4_t*>(o) = q;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = h[i];
            }
        }
    }
}

template <int MODE, int ODT>
hipError_t run_dequantize_mx(const DequantMxArgs& a, hipStream_t st)
{
    using F = MxFmt<MODE>;
    using O = typename Elem<ODT>::storage;
    const int64_t runs_row = a.K / 8, words_row = a.K * F::BITS / 32, groups_row = a.K / F::GS;
    const bool vec = reinterpret_cast<uintptr_t>(a.out) % 16 == 0;
    const int64_t rows_per_launch = ((int64_t)1 << 30) / runs_row;
    for (int64_t r0 = 0; r0 < a.N; r0 += rows_per_launch) {
        const int64_t rows = a.N - r0 < rows_per_launch ? a.N - r0 : rows_per_launch;
        const uint32_t runs = (uint32_t)(rows * runs_row);
        const uint32_t blocks = (runs + kThreads * kRunsPerThread - 1) / (kThreads * kRunsPerThread);
        const uint32_t* wq = a.wq + r0 * words_row;
        const uint8_t* sc = a.scales + r0 * groups_row;
        O* out = static_cast<O*>(a.out) + r0 * a.K;
        if (vec)
            hipLaunchKernelGGL((dequantize_mx_kernel<MODE, ODT, true>), dim3(blocks),
                               dim3(kThreads), 0, st, wq, sc, runs, (uint32_t)runs_row,
                               (uint32_t)words_row, (uint32_t)groups_row, out);
        else
            hipLaunchKernelGGL((dequantize_mx_kernel<MODE, ODT, false>), dim3(blocks),
                               dim3(kThreads), 0, st, wq, sc, runs, (uint32_t)runs_row,
                               (uint32_t)words_row, (uint32_t)groups_row, out);
        if (hipError_t e = hipGetLastError(); e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <int MODE>
hipError_t run_dequantize_mx_mode(const DequantMxArgs& a, hipStream_t st)
{
    switch (a.odt) {
    case DT_F32: return run_dequantize_mx<MODE, DT_F32>(a, st);
    case DT_F16: return run_dequantize_mx<MODE, DT_F16>(a, st);
    case DT_BF16: return run_dequantize_mx<MODE, DT_BF16>(a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_dequantize_mx(const DequantMxArgs& a, hipStream_t st)
{
    switch (a.mode) {
    case MODE_MXFP4: return run_dequantize_mx_mode<MODE_MXFP4>(a, st);
    case MODE_MXFP8: return run_dequantize_mx_mode<MODE_MXFP8>(a, st);
    case MODE_NVFP4: return run_dequantize_mx_mode<MODE_NVFP4>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t st)
{
    switch (a.bits) {
    case 2: return run_dequantize_bits<2>(a, st);
    case 3: return run_dequantize_bits<3>(a, st);
    case 4: return run_dequantize_bits<4>(a, st);
    case 6: return run_dequantize_bits<6>(a, st);
    case 8: return run_dequantize_bits<8>(a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace qp
