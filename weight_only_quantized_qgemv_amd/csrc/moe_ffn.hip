// moe_ffn.hip — the close of an MoE feed-forward block: each token's output
// is the weighted sum of its top_k slots' down-projection rows,
//   out[t, d] = sum_j rw[t*top_k + j] * o[t*top_k + j, d],
// with the router weights rw given by the caller (the ferrum-kernels MoE docs
// dispatch the per-role products and leave this step to the FFN). Slots
// whose expert id is outside [0, E) add nothing (their products were
// skipped). fp32 sum in slot order, rounded once to the activation type.
#include "common.hpp"
#include "launch.hpp"

namespace qp {

namespace {

template <int DT>
__global__ __launch_bounds__(256) void moe_combine_kernel(
    const typename Elem<DT>::storage* __restrict__ o, const int32_t* __restrict__ ids,
    const float* __restrict__ rw, int64_t n_tokens, int top_k, int64_t d_model, int num_experts,
    typename Elem<DT>::storage* __restrict__ out)
{
    using E = Elem<DT>;
    const int64_t total = n_tokens * d_model;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / d_model, d = i - t * d_model;
        float acc = 0.0f;
        for (int j = 0; j < top_k; ++j) {
            const int64_t p = t * top_k + j;
            const int32_t e = ids[p];
            if (e >= 0 && e < num_experts)
                acc = __builtin_fmaf(rw[p], E::to_f32(o[p * d_model + d]), acc);
        }
        out[i] = E::from_f32(acc);
    }
}

} // namespace

hipError_t launch_moe_combine(const MoeCombineArgs& a, hipStream_t st)
{
    const int64_t total = a.n_tokens * a.d_model;
    int64_t blocks = (total + 255) / 256;
    blocks = blocks < 4096 ? blocks : 4096;
    switch (a.dt) {
    case DT_F32:
        hipLaunchKernelGGL((moe_combine_kernel<DT_F32>), dim3((int)blocks), dim3(256), 0, st,
                           static_cast<const float*>(a.o), a.ids, a.rw, a.n_tokens, (int)a.top_k,
                           a.d_model, (int)a.E, static_cast<float*>(a.out));
        break;
    case DT_F16:
        hipLaunchKernelGGL((moe_combine_kernel<DT_F16>), dim3((int)blocks), dim3(256), 0, st,
                           static_cast<const uint16_t*>(a.o), a.ids, a.rw, a.n_tokens,
                           (int)a.top_k, a.d_model, (int)a.E, static_cast<uint16_t*>(a.out));
        break;
    case DT_BF16:
        hipLaunchKernelGGL((moe_combine_kernel<DT_BF16>), dim3((int)blocks), dim3(256), 0, st,
                           static_cast<const uint16_t*>(a.o), a.ids, a.rw, a.n_tokens,
                           (int)a.top_k, a.d_model, (int)a.E, static_cast<uint16_t*>(a.out));
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace qp
