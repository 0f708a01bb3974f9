// mx_gemv.hip — y = x @ dequant(W)^T for the microscaled modes (emily
// lib/emily/quantization.ex: `quantized_matmul/2` with mode mxfp4, mxfp8 or
// nvfp4, whose dense weight is the one of `dequantize_defn/1`'s microscaled
// implementations; formats in mx.hpp). Activations are fp32, fp16 or bf16
// (any float type, per the same page); y takes their type; fp32
// accumulation.
//
// Stream kernel (16-bit activations, K a multiple of 32, K <= 16384): a wave
// owns one weight row at a time; lane l takes the 32-lane units l, l + 64, ...
// of the row, so its slice of the activation rows is fixed and held in
// registers as 16-bit pairs for the whole launch. Per unit the gfx950
// conversion instructions turn the packed FP4 / FP8 codes into pairs of the
// activation type (every FP4-E2M1 and FP8-E4M3 value is exact in bf16 and
// fp16), v_dot2 forms the unit's partial sum in fp32, and the group scale is
// applied to that sum. The conversions read FP8 0x7F / 0xFF as NaN where the
// pages' E4M3 has +-480: in a unit holding such a code (found with integer
// ops on its code words) those halves of the converted pairs are replaced by
// +-480 before the products. D rows are loaded before any is reduced, and
// each wave's partial sums meet in a DPP reduction.
//
// Generic kernel (fp32 activations and every other shape): one wave per
// (activation row, weight row), lanes over the groups of the row, exact
// decode, fp32 FMAs.
#include "gemv_core.hpp"
#include "launch.hpp"
#include "mx.hpp"

namespace qp {

namespace {

struct MxKArgs {
    const void* x;              // [M, K] of DT (the rows of this launch)
    const uint32_t* wq;         // [N, K*bits/32] (the rows of this launch)
    const uint8_t* scales;      // [N, K/gs]
    void* y;                    // [M, y_ld] of DT
    int M, N, K;
    int64_t y_ld;               // elements between consecutive rows of y
    uint32_t row_bytes, groups_row, units_row;
};

// Pair `hi` (bytes 2, 3, else 0, 1) of FP8 word w converted to 16-bit `pair`,
// with the halves whose code is 0x7F / 0xFF (NaN to the conversion, +-480 on
// the pages) replaced by +-480 (`m480`: 480 in the 16-bit type). Bit 7 of a
// byte of f flags such a code; v_perm replicates a flag into the half's mask
// (selector 8 / 9: bit 15 / 31 of the low source, 10 / 11: of the high one),
// and the half's sign comes from its code's bit 7 the same way.
__device__ __forceinline__ uint32_t fp8_fix_nan(uint32_t pair, uint32_t w, bool hi, uint32_t m480)
{
    const uint32_t f = ((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
    const uint32_t sel = hi ? 0x0B0B0909u : 0x0A0A0808u;
    const uint32_t mask = __builtin_amdgcn_perm(f, f << 8, sel);
    const uint32_t sign = __builtin_amdgcn_perm(w, w << 8, sel) & 0x80008000u;
    const uint32_t repl = m480 | (m480 << 16) | sign;
    return (repl & mask) | (pair & ~mask);
}

template <int DT> struct MxPair;
template <> struct MxPair<DT_BF16> {
    using pair_t = bf16x2_t;
    static __device__ __forceinline__ pair_t fp4(uint32_t w, int byte)
    {
        switch (byte) {
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
        }
    }
    static __device__ __forceinline__ pair_t fp8(uint32_t w, bool hi)
    {
        return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                  : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    }
    static __device__ __forceinline__ pair_t fp8_fixed(uint32_t w, bool hi)
    {
        const uint32_t p = __builtin_bit_cast(uint32_t, fp8(w, hi));
        return __builtin_bit_cast(pair_t, fp8_fix_nan(p, w, hi, 0x43F0u));   // bf16 480
    }
    static __device__ __forceinline__ float dot(pair_t a, uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2_t, x), acc, false);
    }
};
template <> struct MxPair<DT_F16> {
    using pair_t = f16x2_t;
    static __device__ __forceinline__ pair_t fp4(uint32_t w, int byte)
    {
        switch (byte) {
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
        }
    }
    static __device__ __forceinline__ pair_t fp8(uint32_t w, bool hi)
    {
        return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                  : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    }
    static __device__ __forceinline__ pair_t fp8_fixed(uint32_t w, bool hi)
    {
        const uint32_t p = __builtin_bit_cast(uint32_t, fp8(w, hi));
        return __builtin_bit_cast(pair_t, fp8_fix_nan(p, w, hi, 0x5F80u));   // fp16 480
    }
    static __device__ __forceinline__ float dot(pair_t a, uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2(a, __builtin_bit_cast(f16x2_t, x), acc, false);
    }
};

// Activation k of a 16-bit pair table as fp32 (k even: low half).
template <int DT>
__device__ __forceinline__ float pair_elem(uint32_t pair, int k)
{
    const uint16_t h = (uint16_t)(k & 1 ? pair >> 16 : pair);
    return Elem<DT>::to_f32(h);
}

// Rows in flight per wave: about 64 VGPRs of codes.
template <int MODE, int UPL>
constexpr int mx_depth()
{
    constexpr int cw = MxFmt<MODE>::BITS;   // code words per 32-lane unit
    constexpr int d = 64 / (UPL * cw);
    return d < 1 ? 1 : (d > 4 ? 4 : d);
}

template <int MODE, int DT, int MT, int UPL>
__global__ __launch_bounds__(256) void qgemv_mx_stream_kernel(MxKArgs a)
{
    using F = MxFmt<MODE>;
    using PX = MxPair<DT>;
    using St = typename Elem<DT>::storage;
    constexpr int CW = F::BITS;             // code words per unit (16 or 32 bytes)
    constexpr int SPU = 32 / F::GS;         // scale bytes per unit
    constexpr int D = mx_depth<MODE, UPL>();
    const int lane = threadIdx.x & 63;
    const int gw = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    const int GW = (int)gridDim.x * 4;

    // The lane's activation slice: units u_j = lane + 64 j, 16 pairs each.
    uint32_t xr[MT][UPL][16];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
            const int u = lane + 64 * j;
            if (u < (int)a.units_row && m < a.M) {
                const u32x4_t* p = reinterpret_cast<const u32x4_t*>(
                    static_cast<const St*>(a.x) + (int64_t)m * a.K + 32 * u);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const u32x4_t q = p[v];
                    xr[m][j][4 * v] = q.x; xr[m][j][4 * v + 1] = q.y;
                    xr[m][j][4 * v + 2] = q.z; xr[m][j][4 * v + 3] = q.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) xr[m][j][i] = 0u;
            }
        }

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.wq, (uint32_t)a.N * a.row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales, (uint32_t)a.N * a.groups_row);
    St* y = static_cast<St*>(a.y);

    for (int r0 = gw * D; r0 < a.N; r0 += GW * D) {
        uint32_t w[D][UPL][CW];
        uint32_t sb[D][UPL];
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int j = 0; j < UPL; ++j) {
                const int u = lane + 64 * j, r = r0 + d;
                const bool live = u < (int)a.units_row && r < a.N;
                const uint32_t off = live ? (uint32_t)r * a.row_bytes + (uint32_t)u * CW * 4 : OOB;
                buffer_words<CW>(rw, off, w[d][j]);
                const uint32_t soff = live ? (uint32_t)r * a.groups_row + (uint32_t)u * SPU : OOB;
                if constexpr (SPU == 2)
                    sb[d][j] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, 0, 0);
                else
                    sb[d][j] = __builtin_amdgcn_raw_buffer_load_b8(rs, soff, 0, 0);
            }
        float acc[D * MT];
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float total = 0.0f;
#pragma unroll
                for (int j = 0; j < UPL; ++j) {
                    // Partial sums of the unit's groups (two for 16-lane groups).
                    float part[SPU];
#pragma unroll
                    for (int g = 0; g < SPU; ++g) part[g] = 0.0f;
                    if constexpr (F::BITS == 4) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                part[(i * SPU) / 4] = PX::dot(PX::fp4(w[d][j][i], b),
                                                              xr[m][j][4 * i + b],
                                                              part[(i * SPU) / 4]);
                    } else {
                        // Bit 7 of a byte of (w & 0x7F7F7F7F) + 0x01010101 is set
                        // exactly when the byte is 0x7F or 0xFF (no carry crosses
                        // bytes, since each sum stays below 0x100).
                        uint32_t nan_codes = 0u;
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            nan_codes |= (w[d][j][i] & 0x7F7F7F7Fu) + 0x01010101u;
                        if (__builtin_expect((nan_codes & 0x80808080u) == 0u, 1)) {
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                part[0] = PX::dot(PX::fp8(w[d][j][i], false), xr[m][j][2 * i],
                                                  part[0]);
                                part[0] = PX::dot(PX::fp8(w[d][j][i], true), xr[m][j][2 * i + 1],
                                                  part[0]);
                            }
                        } else {
                            // A 0x7F / 0xFF code: its half of the converted pair
                            // is replaced by +-480 before the product.
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                const uint32_t wi = w[d][j][i];
                                part[0] = PX::dot(PX::fp8_fixed(wi, false), xr[m][j][2 * i], part[0]);
                                part[0] = PX::dot(PX::fp8_fixed(wi, true), xr[m][j][2 * i + 1],
                                                  part[0]);
                            }
                        }
                    }
#pragma unroll
                    for (int g = 0; g < SPU; ++g)
                        total += mx_scaled<MODE>(part[g], (sb[d][j] >> (8 * g)) & 0xFFu);
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
                        y[(int64_t)m * a.y_ld + r0 + d] = Elem<DT>::from_f32(acc[d * MT + m]);
        }
    }
}

template <int MODE, int DT>
__global__ __launch_bounds__(256) void qgemv_mx_generic_kernel(MxKArgs a)
{
    using F = MxFmt<MODE>;
    using St = typename Elem<DT>::storage;
    constexpr int GW_WORDS = F::GS * F::BITS / 32;   // code words per group
    const int lane = threadIdx.x & 63;
    const int64_t total = (int64_t)a.M * a.N;
    const int64_t nw = (int64_t)gridDim.x * 4;
    const St* xs = static_cast<const St*>(a.x);
    St* y = static_cast<St*>(a.y);
    for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < total; t += nw) {
        const int m = (int)(t / a.N), r = (int)(t % a.N);
        const uint32_t* row = a.wq + (size_t)r * (a.row_bytes / 4);
        const St* xm = xs + (int64_t)m * a.K;
        float acc = 0.0f;
        for (uint32_t g = lane; g < a.groups_row; g += 64) {
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < GW_WORDS; ++i) {
                const uint32_t word = row[g * GW_WORDS + i];
#pragma unroll
                for (int c = 0; c < 32 / F::BITS; ++c) {
                    const uint32_t code = (word >> (c * F::BITS)) & ((1u << F::BITS) - 1u);
                    const int k = (int)g * F::GS + i * (32 / F::BITS) + c;
                    part = __builtin_fmaf(mx_lane<MODE>(code), Elem<DT>::to_f32(xm[k]), part);
                }
            }
            acc += mx_scaled<MODE>(part, a.scales[(size_t)r * a.groups_row + g]);
        }
        float v[1] = {acc};
        reduce_slots<1, 64>(v);
        if (lane == 63)
            y[(int64_t)m * a.y_ld + r] = Elem<DT>::from_f32(v[0]);
    }
}

constexpr int kMaxBlocks = 8192;

template <int MODE, int DT, int MT, int UPL>
hipError_t run_mx_stream(const MxKArgs& k, hipStream_t st)
{
    constexpr int D = mx_depth<MODE, UPL>();
    int64_t blocks = ((int64_t)k.N + 4 * D - 1) / (4 * D);
    blocks = blocks < kMaxBlocks ? blocks : kMaxBlocks;
    hipLaunchKernelGGL((qgemv_mx_stream_kernel<MODE, DT, MT, UPL>), dim3((int)blocks), dim3(256),
                       0, st, k);
    return hipGetLastError();
}

template <int MODE, int DT, int MT>
hipError_t run_mx_upl(const MxKArgs& k, hipStream_t st)
{
    const int upl = ((int)k.units_row + 63) / 64;
    if (upl <= 1) return run_mx_stream<MODE, DT, MT, 1>(k, st);
    if (upl <= 2) return run_mx_stream<MODE, DT, MT, 2>(k, st);
    if (upl <= 4) return run_mx_stream<MODE, DT, MT, 4>(k, st);
    if constexpr (MT == 1)
        return run_mx_stream<MODE, DT, MT, 8>(k, st);
    return hipErrorInvalidValue;   // two rows only up to four units per lane
}

template <int MODE, int DT>
hipError_t run_mx_dt(const GemvMxArgs& a, hipStream_t st)
{
    using F = MxFmt<MODE>;
    const int es = DT == DT_F32 ? 4 : 2;
    const int64_t row_bytes = a.K * F::BITS / 8, groups_row = a.K / F::GS;
    const bool stream = DT != DT_F32 && a.K % 32 == 0 && a.K <= 16384 &&
                        reinterpret_cast<uintptr_t>(a.x) % 16 == 0;
    // Weight rows per launch: 32-bit buffer offsets.
    const int64_t rows_cap = ((int64_t)1 << 31) / (row_bytes > groups_row ? row_bytes : groups_row);
    for (int64_t n0 = 0; n0 < a.N; n0 += rows_cap) {
        const int64_t nc = a.N - n0 < rows_cap ? a.N - n0 : rows_cap;
        // Activation rows: two at a time on the stream kernel (one when a lane
        // holds more than four units of them), all at once on the generic one.
        const int64_t mstep = stream ? (a.K / 32 > 256 ? 1 : 2) : a.M;
        for (int64_t m0 = 0; m0 < a.M; m0 += mstep) {
            const int64_t mc = a.M - m0 < mstep ? a.M - m0 : mstep;
            MxKArgs k{};
            k.x = static_cast<const char*>(a.x) + m0 * a.K * es;
            k.wq = a.wq + n0 * (row_bytes / 4);
            k.scales = a.scales + n0 * groups_row;
            k.y = static_cast<char*>(a.y) + (m0 * a.N + n0) * es;
            k.M = (int)mc;
            k.N = (int)nc;
            k.K = (int)a.K;
            k.y_ld = a.N;
            k.row_bytes = (uint32_t)row_bytes;
            k.groups_row = (uint32_t)groups_row;
            k.units_row = (uint32_t)(a.K / 32);
            hipError_t e;
            if (stream) {
                if constexpr (DT != DT_F32)
                    e = mc == 2 ? run_mx_upl<MODE, DT, 2>(k, st) : run_mx_upl<MODE, DT, 1>(k, st);
                else
                    e = hipErrorInvalidValue;
            } else {
                int64_t blocks = (mc * nc + 3) / 4;
                blocks = blocks < kMaxBlocks ? blocks : kMaxBlocks;
                hipLaunchKernelGGL((qgemv_mx_generic_kernel<MODE, DT>), dim3((int)blocks),
                                   dim3(256), 0, st, k);
                e = hipGetLastError();
            }
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

template <int MODE>
hipError_t run_mx_mode(const GemvMxArgs& a, hipStream_t st)
{
    switch (a.dt) {
    case DT_F32: return run_mx_dt<MODE, DT_F32>(a, st);
    case DT_F16: return run_mx_dt<MODE, DT_F16>(a, st);
    case DT_BF16: return run_mx_dt<MODE, DT_BF16>(a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_qmatmul_mx(const GemvMxArgs& a, hipStream_t st)
{
    switch (a.mode) {
    case MODE_MXFP4: return run_mx_mode<MODE_MXFP4>(a, st);
    case MODE_MXFP8: return run_mx_mode<MODE_MXFP8>(a, st);
    case MODE_NVFP4: return run_mx_mode<MODE_NVFP4>(a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace qp
