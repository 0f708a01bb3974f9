// quantize.hip — affine group quantization and bit packing on the device.
//
// The pages call MLX's quantizer (ollama x/create/client/quantize.go,
// `loadAndQuantizeArray`; emily `QuantizedWeight.from_dense/2`) without
// printing it; this kernel computes the plain affine form, per row and group
// of gs consecutive elements along K:
//   s  = (max - min) / (2^bits - 1)  in fp32, floored at FLT_EPSILON
//        (the floor of mlex src/quant.rs `quantize_dynamic_int8`),
//   s' = RNE(s), b' = RNE(min) in the storage type, a zero bias stored as +0,
//   q  = clamp(round_half_away((w - b') / s'), 0, 2^bits - 1)
//        (round and clamp as in `quantize_dynamic_int8`),
// and packs lane i of the row at bits [i*bits, i*bits + bits) of the row's
// little-endian u32 stream (emily `dequantize_defn/1` docs).
//
// Every step is a single IEEE operation in a fixed order (fp32 subtract,
// correctly rounded divide, round, compare), contraction is off, so the result
// is reproducible bit for bit on any launch shape.
#include <float.h>

#include "common.hpp"
#include "launch.hpp"

namespace qp {

#pragma clang fp contract(off)

template <int BITS, int DT>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, int64_t N,
                                                       int64_t K, int gs, uint32_t* __restrict__ wq,
                                                       typename Elem<DT>::storage* __restrict__ scales,
                                                       typename Elem<DT>::storage* __restrict__ biases)
{
    using E = Elem<DT>;
    const int64_t groups_row = K / gs;
    const int64_t total = N * groups_row;
    const float qmax = (float)((1 << BITS) - 1);
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = t / groups_row, g = t % groups_row;
        const float* wg = w + row * K + g * gs;
        float mn = wg[0], mx = wg[0];
        for (int i = 1; i < gs; ++i) {
            const float v = wg[i];
            if (v < mn) mn = v;
            if (v > mx) mx = v;
        }
        float s = (mx - mn) / qmax;
        if (!(s >= FLT_EPSILON))
            s = FLT_EPSILON;
        const typename E::storage s_st = E::from_f32(s);
        typename E::storage b_st = E::from_f32(mn);
        const float sq = E::to_f32(s_st);
        float bq = E::to_f32(b_st);
        if (bq == 0.0f) {
            b_st = E::from_f32(0.0f);
            bq = 0.0f;
        }
        scales[t] = s_st;
        biases[t] = b_st;

        // Each group is gs/32 whole units of 32 codes = bits words each.
        uint32_t* out = wq + row * (K * BITS / 32) + g * (gs / 32) * BITS;
        for (int u = 0; u < gs / 32; ++u) {
            uint32_t words[BITS];
#pragma unroll
            for (int i = 0; i < BITS; ++i)
                words[i] = 0u;
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                float qf = roundf((wg[u * 32 + c] - bq) / sq);
                qf = qf < 0.0f ? 0.0f : qf;
                qf = qf > qmax ? qmax : qf;
                const uint32_t q = (uint32_t)qf;
                const int bit = c * BITS, wi = bit / 32, sh = bit % 32;
                words[wi] |= q << sh;
                if (sh + BITS > 32)
                    words[wi + 1] |= q >> (32 - sh);
            }
#pragma unroll
            for (int i = 0; i < BITS; ++i)
                out[u * BITS + i] = words[i];
        }
    }
}

namespace {

template <int BITS, int DT>
hipError_t run_quantize(const QuantizeArgs& a, hipStream_t st)
{
    using S = typename Elem<DT>::storage;
    int64_t total = a.N * (a.K / a.gs);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    hipLaunchKernelGGL((quantize_kernel<BITS, DT>), dim3((int)blocks), dim3(256), 0, st, a.w, a.N,
                       a.K, a.gs, a.wq, static_cast<S*>(a.scales), static_cast<S*>(a.biases));
    return hipGetLastError();
}

template <int BITS>
hipError_t run_quantize_bits(const QuantizeArgs& a, hipStream_t st)
{
    switch (a.dt) {
    case DT_F32: return run_quantize<BITS, DT_F32>(a, st);
    case DT_F16: return run_quantize<BITS, DT_F16>(a, st);
    case DT_BF16: return run_quantize<BITS, DT_BF16>(a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t st)
{
    switch (a.bits) {
    case 2: return run_quantize_bits<2>(a, st);
    case 3: return run_quantize_bits<3>(a, st);
    case 4: return run_quantize_bits<4>(a, st);
    case 6: return run_quantize_bits<6>(a, st);
    case 8: return run_quantize_bits<8>(a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace qp
