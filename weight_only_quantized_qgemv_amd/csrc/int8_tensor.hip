// int8_tensor.hip — per-tensor dynamic-range int8 weights (mlex src/quant.rs,
// `quantize_dynamic_int8` / `dequantize_dynamic_int8`): one output range
// [lo, hi] for the whole tensor, and w = (q + 128) * ((hi - lo) / 255) + lo
// for the signed code q, each step an fp32 operation.
//
//  - quantize: the tensor's min / max by order-preserving integer keys and
//    device atomics (min and max do not depend on the order, so the result is
//    deterministic), then q = clamp(round((w - lo) / step) - 128, -128, 127)
//    with the step floored at FLT_EPSILON, and the range written back;
//  - dequantize: the formula above, elementwise;
//  - product, y = x @ W^T: y[m, n] = step * sum_k x (q + 128) + lo * sum_k x.
//    The stream kernel keeps each lane's slice of the activation rows in
//    registers (16-bit pairs), turns code bytes (q + 128 = byte ^ 0x80, exact
//    in bf16 and fp16) into pairs for v_dot2, and applies step and lo once per
//    row. fp32 activations and other shapes take a generic kernel that forms
//    every weight with the fp32 steps above.
#include <float.h>

#include "common.hpp"
#include "gemv_core.hpp"
#include "launch.hpp"

namespace qp {

#pragma clang fp contract(off)

namespace {

// Unsigned key with the order of the fp32 values (finite inputs).
__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__global__ void range_init_kernel(uint32_t* keys)
{
    if (threadIdx.x == 0) {
        keys[0] = 0xFFFFFFFFu;   // min: above every key
        keys[1] = 0u;            // max: below every key
    }
}

__global__ __launch_bounds__(256) void range_minmax_kernel(const float* __restrict__ w,
                                                           int64_t count, uint32_t* keys)
{
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t k = order_key(w[i]);
        lo = k < lo ? k : lo;
        hi = k > hi ? k : hi;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t l2 = __shfl_xor(lo, off, 64), h2 = __shfl_xor(hi, off, 64);
        lo = l2 < lo ? l2 : lo;
        hi = h2 > hi ? h2 : hi;
    }
    if ((threadIdx.x & 63) == 0) {
        atomicMin(&keys[0], lo);
        atomicMax(&keys[1], hi);
    }
}

__global__ __launch_bounds__(256) void int8_quantize_kernel(const float* __restrict__ w,
                                                            int64_t count,
                                                            const uint32_t* __restrict__ keys,
                                                            int8_t* __restrict__ q)
{
    const float lo = key_value(keys[0]), hi = key_value(keys[1]);
    float step = (hi - lo) / 255.0f;
    if (!(step >= FLT_EPSILON))
        step = FLT_EPSILON;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x) {
        float t = roundf((w[i] - lo) / step) - 128.0f;
        t = t < -128.0f ? -128.0f : t;
        t = t > 127.0f ? 127.0f : t;
        q[i] = (int8_t)t;
    }
}

// Keys back to the range [lo, hi] in place.
__global__ void range_finalize_kernel(uint32_t* keys)
{
    if (threadIdx.x == 0) {
        const float lo = key_value(keys[0]), hi = key_value(keys[1]);
        keys[0] = __float_as_uint(lo);
        keys[1] = __float_as_uint(hi);
    }
}

__device__ __forceinline__ float int8_weight(int8_t q, float step, float lo)
{
    const float shifted = (float)q + 128.0f;
    const float scaled = shifted * step;
    return scaled + lo;
}

template <int ODT>
__global__ __launch_bounds__(256) void int8_dequantize_kernel(const int8_t* __restrict__ q,
                                                              int64_t count,
                                                              const float* __restrict__ range,
                                                              typename Elem<ODT>::storage* __restrict__ out)
{
    const float lo = range[0], step = (range[1] - range[0]) / 255.0f;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        out[i] = Elem<ODT>::from_f32(int8_weight(q[i], step, lo));
}

struct Int8KArgs {
    const void* x;              // [M, K] (the rows of this launch)
    const int8_t* q;            // [N, K]
    const float* range;         // [2]
    void* y;                    // [M, y_ld]
    int M, N, K;
    int64_t y_ld;
    uint32_t units_row;         // K / 32
};

template <int DT> struct Int8Pair;
template <> struct Int8Pair<DT_BF16> {
    // bytes b0, b1 as a bf16 pair (values 0..255 are exact in bf16)
    static __device__ __forceinline__ uint32_t pair(float a, float b)
    {
        return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)a, (__bf16)b});
    }
    static __device__ __forceinline__ float dot(uint32_t a, uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, x), acc, false);
    }
};
template <> struct Int8Pair<DT_F16> {
    static __device__ __forceinline__ uint32_t pair(float a, float b)
    {
        return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)a, (_Float16)b});
    }
    static __device__ __forceinline__ float dot(uint32_t a, uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, x),
                                      acc, false);
    }
};

template <int DT>
__device__ __forceinline__ float pair_value(uint32_t pair, int hi)
{
    return Elem<DT>::to_f32((uint16_t)(hi ? pair >> 16 : pair));
}

// Rows in flight: about 64 VGPRs of codes (8 per unit).
template <int UPL> constexpr int int8_depth() { return 8 / UPL < 1 ? 1 : (8 / UPL > 4 ? 4 : 8 / UPL); }

template <int DT, int MT, int UPL>
__global__ __launch_bounds__(256) void qgemv_int8t_stream_kernel(Int8KArgs a)
{
    using PX = Int8Pair<DT>;
    using St = typename Elem<DT>::storage;
    constexpr int D = int8_depth<UPL>();
    const int lane = threadIdx.x & 63;
    const int gw = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    const int GW = (int)gridDim.x * 4;
    const float lo = a.range[0], step = (a.range[1] - a.range[0]) / 255.0f;

    // The lane's activation slice (units u_j = lane + 64 j of 32 values) and
    // its plain sum per row.
    uint32_t xr[MT][UPL][16];
    float xsum[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        xsum[m] = 0.0f;
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
            const int u = lane + 64 * j;
            if (u < (int)a.units_row && m < a.M) {
                const u32x4_t* p = reinterpret_cast<const u32x4_t*>(
                    static_cast<const St*>(a.x) + (int64_t)m * a.K + 32 * u);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const u32x4_t qv = p[v];
                    xr[m][j][4 * v] = qv.x; xr[m][j][4 * v + 1] = qv.y;
                    xr[m][j][4 * v + 2] = qv.z; xr[m][j][4 * v + 3] = qv.w;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    xsum[m] += pair_value<DT>(xr[m][j][i], 0) + pair_value<DT>(xr[m][j][i], 1);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) xr[m][j][i] = 0u;
            }
        }
    }

    const uint32_t row_bytes = (uint32_t)a.K;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.q, (uint32_t)a.N * row_bytes);
    St* y = static_cast<St*>(a.y);
    for (int r0 = gw * D; r0 < a.N; r0 += GW * D) {
        uint32_t w[D][UPL][8];
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int j = 0; j < UPL; ++j) {
                const int u = lane + 64 * j, r = r0 + d;
                const bool live = u < (int)a.units_row && r < a.N;
                buffer_words<8>(rw, live ? (uint32_t)r * row_bytes + (uint32_t)u * 32 : OOB,
                                w[d][j]);
            }
        float acc[D * MT];
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < UPL; ++j)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        // q + 128 for the four codes of word i: flip each sign bit.
                        const uint32_t uw = w[d][j][i] ^ 0x80808080u;
                        const uint32_t p0 = PX::pair((float)(uw & 0xFFu), (float)((uw >> 8) & 0xFFu));
                        const uint32_t p1 = PX::pair((float)((uw >> 16) & 0xFFu), (float)(uw >> 24));
                        s = PX::dot(p0, xr[m][j][2 * i], s);
                        s = PX::dot(p1, xr[m][j][2 * i + 1], s);
                    }
                // Rows past N hold zero codes (u = 128) and are not stored.
                acc[d * MT + m] = step * s + lo * xsum[m];
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

template <int DT>
__global__ __launch_bounds__(256) void qgemv_int8t_generic_kernel(Int8KArgs a)
{
    using St = typename Elem<DT>::storage;
    const int lane = threadIdx.x & 63;
    const float lo = a.range[0], step = (a.range[1] - a.range[0]) / 255.0f;
    const int64_t total = (int64_t)a.M * a.N;
    const St* xs = static_cast<const St*>(a.x);
    St* y = static_cast<St*>(a.y);
    for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < total;
         t += (int64_t)gridDim.x * 4) {
        const int m = (int)(t / a.N), r = (int)(t % a.N);
        const int8_t* row = a.q + (size_t)r * a.K;
        const St* xm = xs + (int64_t)m * a.K;
        float acc = 0.0f;
        for (int k = lane; k < a.K; k += 64)
            acc = __builtin_fmaf(Elem<DT>::to_f32(xm[k]), int8_weight(row[k], step, lo), acc);
        float v[1] = {acc};
        reduce_slots<1, 64>(v);
        if (lane == 63)
            y[(int64_t)m * a.y_ld + r] = Elem<DT>::from_f32(v[0]);
    }
}

constexpr int kMaxBlocks = 8192;

template <int DT, int MT, int UPL>
hipError_t run_int8t_stream(const Int8KArgs& k, hipStream_t st)
{
    constexpr int D = int8_depth<UPL>();
    int64_t blocks = ((int64_t)k.N + 4 * D - 1) / (4 * D);
    blocks = blocks < kMaxBlocks ? blocks : kMaxBlocks;
    hipLaunchKernelGGL((qgemv_int8t_stream_kernel<DT, MT, UPL>), dim3((int)blocks), dim3(256), 0,
                       st, k);
    return hipGetLastError();
}

template <int DT, int MT>
hipError_t run_int8t_upl(const Int8KArgs& k, hipStream_t st)
{
    const int upl = ((int)k.units_row + 63) / 64;
    if (upl <= 1) return run_int8t_stream<DT, MT, 1>(k, st);
    if (upl <= 2) return run_int8t_stream<DT, MT, 2>(k, st);
    if (upl <= 4) return run_int8t_stream<DT, MT, 4>(k, st);
    if constexpr (MT == 1)
        return run_int8t_stream<DT, MT, 8>(k, st);
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t run_int8t_dt(const Int8TensorArgs& a, hipStream_t st)
{
    const int es = DT == DT_F32 ? 4 : 2;
    const bool stream = DT != DT_F32 && a.K % 32 == 0 && a.K <= 16384 &&
                        reinterpret_cast<uintptr_t>(a.x) % 16 == 0;
    const int64_t rows_cap = ((int64_t)1 << 31) / a.K;
    for (int64_t n0 = 0; n0 < a.N; n0 += rows_cap) {
        const int64_t nc = a.N - n0 < rows_cap ? a.N - n0 : rows_cap;
        const int64_t mstep = stream ? (a.K / 32 > 256 ? 1 : 2) : a.M;
        for (int64_t m0 = 0; m0 < a.M; m0 += mstep) {
            const int64_t mc = a.M - m0 < mstep ? a.M - m0 : mstep;
            Int8KArgs k{};
            k.x = static_cast<const char*>(a.x) + m0 * a.K * es;
            k.q = a.q + n0 * a.K;
            k.range = a.range;
            k.y = static_cast<char*>(a.y) + (m0 * a.N + n0) * es;
            k.M = (int)mc;
            k.N = (int)nc;
            k.K = (int)a.K;
            k.y_ld = a.N;
            k.units_row = (uint32_t)(a.K / 32);
            hipError_t e;
            if (stream) {
                if constexpr (DT != DT_F32)
                    e = mc == 2 ? run_int8t_upl<DT, 2>(k, st) : run_int8t_upl<DT, 1>(k, st);
                else
                    e = hipErrorInvalidValue;
            } else {
                int64_t blocks = (mc * nc + 3) / 4;
                blocks = blocks < kMaxBlocks ? blocks : kMaxBlocks;
                hipLaunchKernelGGL((qgemv_int8t_generic_kernel<DT>), dim3((int)blocks), dim3(256),
                                   0, st, k);
                e = hipGetLastError();
            }
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

int64_t grid_for(int64_t count)
{
    int64_t b = (count + 255) / 256;
    return b < 4096 ? b : 4096;
}

} // namespace

hipError_t launch_quantize_int8_tensor(const float* w, int64_t count, int8_t* q, float* range,
                                       hipStream_t st)
{
    uint32_t* keys = reinterpret_cast<uint32_t*>(range);
    hipLaunchKernelGGL(range_init_kernel, dim3(1), dim3(64), 0, st, keys);
    hipLaunchKernelGGL(range_minmax_kernel, dim3((int)grid_for(count)), dim3(256), 0, st, w, count,
                       keys);
    hipLaunchKernelGGL(int8_quantize_kernel, dim3((int)grid_for(count)), dim3(256), 0, st, w,
                       count, keys, q);
    hipLaunchKernelGGL(range_finalize_kernel, dim3(1), dim3(64), 0, st, keys);
    return hipGetLastError();
}

hipError_t launch_dequantize_int8_tensor(const int8_t* q, int64_t count, const float* range,
                                         int odt, void* out, hipStream_t st)
{
    const dim3 g((int)grid_for(count));
    switch (odt) {
    case DT_F32:
        hipLaunchKernelGGL((int8_dequantize_kernel<DT_F32>), g, dim3(256), 0, st, q, count, range,
                           static_cast<float*>(out));
        break;
    case DT_F16:
        hipLaunchKernelGGL((int8_dequantize_kernel<DT_F16>), g, dim3(256), 0, st, q, count, range,
                           static_cast<uint16_t*>(out));
        break;
    case DT_BF16:
        hipLaunchKernelGGL((int8_dequantize_kernel<DT_BF16>), g, dim3(256), 0, st, q, count,
                           range, static_cast<uint16_t*>(out));
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_qmatmul_int8_tensor(const Int8TensorArgs& a, hipStream_t st)
{
    switch (a.dt) {
    case DT_F32: return run_int8t_dt<DT_F32>(a, st);
    case DT_F16: return run_int8t_dt<DT_F16>(a, st);
    case DT_BF16: return run_int8t_dt<DT_BF16>(a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace qp
