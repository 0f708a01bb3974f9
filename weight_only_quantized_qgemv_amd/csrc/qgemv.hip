// qgemv.hip — dense decode GEMV (M <= 16): y[m, n] = x[m, :] @ dequant(W[n, :])
// (emily lib/emily/quantization.ex, `quantized_matmul/2` docs). The kernel is
// the streaming GEMV of gemv_core.hpp with a single tile holding the M
// activation rows; M above the register budget of one tile is split into
// chunks, each streaming the weights once.
#include "gemv_core.hpp"
#include "launch.hpp"

namespace qp {

template <int DT>
__global__ void fill_zero_kernel(typename Elem<DT>::storage* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = Elem<DT>::from_f32(0.f);
}

namespace {

template <int DT> using St = typename Elem<DT>::storage;

// Enough blocks to keep all 256 CUs busy several times over; each block
// strides over row passes beyond that.
constexpr int kMaxBlocks = 4096;

GemvKernelArgs dense_args(const GemvArgs& a, int64_t m0, int mc, int elem_size, int KL)
{
    GemvKernelArgs k{};
    k.x = static_cast<const char*>(a.x) + m0 * a.K * elem_size;
    k.top_k = 1;
    k.outer = a.K;
    k.inner = 0;
    k.perm = nullptr;
    k.tiles = nullptr;
    k.n_tiles = nullptr;
    k.M = mc;
    k.wq[0] = k.wq[1] = a.wq;
    k.scales[0] = k.scales[1] = a.scales;
    k.biases[0] = k.biases[1] = a.biases;
    k.R = a.N;
    k.K = a.K;
    k.gs = a.gs;
    k.KL = KL;
    k.out = static_cast<char*>(a.y) + m0 * a.N * elem_size;
    return k;
}

template <int BITS, int DT, int MT, int U>
hipError_t run_fast(const GemvArgs& a, int64_t m0, int mc, int KL, hipStream_t st)
{
    const int RP = GEMV_THREADS / KL;
    const int64_t passes = (a.N + RP - 1) / RP;
    const int blocks = (int)(passes < kMaxBlocks ? passes : kMaxBlocks);
    GemvKernelArgs k = dense_args(a, m0, mc, (int)sizeof(St<DT>), KL);
    hipLaunchKernelGGL((qgemv_stream_kernel<BITS, DT, MT, U, 1>), dim3(blocks),
                       dim3(GEMV_THREADS), 0, st, k);
    return hipGetLastError();
}

template <int BITS, int DT, int MT>
hipError_t run_chunk(const GemvArgs& a, int64_t m0, int mc, hipStream_t st, bool* done)
{
    *done = true;
    // Prefer slices that put 64 lanes (one wave) on a row; widest slice first.
    if constexpr (MT == 1) {
        if (int kl = gemv_lanes_per_row(a.K, 2); kl == 64) return run_fast<BITS, DT, MT, 2>(a, m0, mc, kl, st);
        if (int kl = gemv_lanes_per_row(a.K, 4); kl == 64) return run_fast<BITS, DT, MT, 4>(a, m0, mc, kl, st);
        if (int kl = gemv_lanes_per_row(a.K, 1); kl == 64) return run_fast<BITS, DT, MT, 1>(a, m0, mc, kl, st);
        if (int kl = gemv_lanes_per_row(a.K, 4)) return run_fast<BITS, DT, MT, 4>(a, m0, mc, kl, st);
        if (int kl = gemv_lanes_per_row(a.K, 2)) return run_fast<BITS, DT, MT, 2>(a, m0, mc, kl, st);
    } else if constexpr (MT == 2) {
        if (int kl = gemv_lanes_per_row(a.K, 2); kl == 64) return run_fast<BITS, DT, MT, 2>(a, m0, mc, kl, st);
        if (int kl = gemv_lanes_per_row(a.K, 2)) return run_fast<BITS, DT, MT, 2>(a, m0, mc, kl, st);
    }
    if (int kl = gemv_lanes_per_row(a.K, 1)) return run_fast<BITS, DT, MT, 1>(a, m0, mc, kl, st);
    *done = false;
    return hipSuccess;
}

template <int BITS, int DT>
hipError_t run_generic(const GemvArgs& a, hipStream_t st)
{
    int64_t blocks = (a.N + 3) / 4;
    if (blocks > kMaxBlocks)
        blocks = kMaxBlocks;
    GemvKernelArgs k = dense_args(a, 0, (int)a.M, (int)sizeof(St<DT>), 64);
    hipLaunchKernelGGL((qgemv_generic_kernel<BITS, DT, 1>), dim3((int)blocks), dim3(256), 0, st,
                       k);
    return hipGetLastError();
}

template <int BITS, int DT>
hipError_t run_gemv(const GemvArgs& a, hipStream_t st)
{
    constexpr int MTMAX = gemv_max_mt<BITS, DT>();
    if (gemv_lanes_per_row(a.K, 1) == 0)
        return run_generic<BITS, DT>(a, st);
    for (int64_t m0 = 0; m0 < a.M;) {
        const int mc = (int)((a.M - m0) < MTMAX ? (a.M - m0) : MTMAX);
        bool done = false;
        hipError_t e;
        if (mc == 1) {
            e = run_chunk<BITS, DT, 1>(a, m0, mc, st, &done);
        } else if (mc == 2) {
            e = run_chunk<BITS, DT, 2>(a, m0, mc, st, &done);
        } else if constexpr (MTMAX >= 8) {
            if (mc <= 4)
                e = run_chunk<BITS, DT, 4>(a, m0, mc, st, &done);
            else
                e = run_chunk<BITS, DT, 8>(a, m0, mc, st, &done);
        } else {
            e = hipErrorInvalidValue; // unreachable: mc <= MTMAX = 2
        }
        if (e != hipSuccess)
            return e;
        if (!done)
            return run_generic<BITS, DT>(a, st);
        m0 += mc;
    }
    return hipSuccess;
}

} // namespace

#ifdef QP_BITS
// This translation unit is compiled once per bit width (QP_BITS).
hipError_t QP_CAT(launch_qgemv_b, QP_BITS)(const GemvArgs& a, hipStream_t st)
{
    switch (a.dt) {
    case DT_F32: return run_gemv<QP_BITS, DT_F32>(a, st);
    case DT_F16: return run_gemv<QP_BITS, DT_F16>(a, st);
    case DT_BF16: return run_gemv<QP_BITS, DT_BF16>(a, st);
    }
    return hipErrorInvalidValue;
}
#endif

#if defined(QP_BITS) && QP_BITS == 4
hipError_t launch_fill_zero(void* p, int dt, int64_t n, hipStream_t st)
{
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024)
        blocks = 1024;
    if (blocks < 1)
        return hipSuccess;
    switch (dt) {
    case DT_F32:
        hipLaunchKernelGGL(fill_zero_kernel<DT_F32>, dim3((int)blocks), dim3(256), 0, st,
                           static_cast<float*>(p), n);
        break;
    case DT_F16:
        hipLaunchKernelGGL(fill_zero_kernel<DT_F16>, dim3((int)blocks), dim3(256), 0, st,
                           static_cast<uint16_t*>(p), n);
        break;
    default:
        hipLaunchKernelGGL(fill_zero_kernel<DT_BF16>, dim3((int)blocks), dim3(256), 0, st,
                           static_cast<uint16_t*>(p), n);
    }
    return hipGetLastError();
}

#endif

} // namespace qp
