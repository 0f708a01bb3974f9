// qgemm.hip — prefill path (M > 16): y = x @ dequant(W)^T on the matrix cores
// (emily lib/emily/quantization.ex, `quantized_matmul/2`). At M in the
// hundreds or thousands the product is a dense contraction (2048 x 14336 x
// 4096 is 240 GFLOP over 33 MB of weights), so it runs on bf16 / fp16 MFMA
// through the tile kernel of gemm_core.hpp, over a dense grid of BM x BN
// tiles mapped XCD by XCD in row-major tile order.
#include "gemm_core.hpp"
#include "launch.hpp"

namespace qp {

namespace {

// Pipeline depths: three activation stages and four code / scale stages.
template <int BITS, int DT, int BM, int BN, int NT>
hipError_t run_gemm(const GemvArgs& a, hipStream_t st)
{
    constexpr int NA = 3, NC = 4;
    constexpr int LDS = gemm::lds_bytes<BITS, BM, BN, NT, NA, NC>();
    static_assert(LDS <= 160 * 1024, "LDS budget");
    const void* kern = reinterpret_cast<const void*>(
        &gemm::qgemm_tile_kernel<BITS, DT, BM, BN, NT, 2, 1, false, NA, NC>);
    static bool attr_set = false; // per instantiation; set before its first launch
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    GemmArgs g{};
    g.x = a.x;
    g.wq[0] = g.wq[1] = a.wq;
    g.scales[0] = g.scales[1] = a.scales;
    g.biases[0] = g.biases[1] = a.biases;
    g.y = a.y;
    g.M = (int)a.M;
    g.N = (int)a.N;
    g.K = (int)a.K;
    g.gs = a.gs;
    g.x_bytes = (uint32_t)(a.M * a.K * 2);
    g.y_bytes = (uint32_t)(a.M * a.N * 2);
    g.sb_bytes = (uint32_t)((a.N * (a.K / a.gs) * 2 + 3) & ~int64_t(3));
    g.tiles_n = (int)((a.N + BN - 1) / BN);
    g.tiles = (int)((a.M + BM - 1) / BM) * g.tiles_n;
    g.per_xcd = (g.tiles + 7) / 8;
    hipLaunchKernelGGL((gemm::qgemm_tile_kernel<BITS, DT, BM, BN, NT, 2, 1, false, NA, NC>),
                       dim3(g.per_xcd * 8), dim3(NT), LDS, st, g);
    return hipGetLastError();
}

template <int DT>
hipError_t run_gemm_dt(const GemvArgs& a, hipStream_t st)
{
    // Wide tiles (eight waves, two per SIMD) when there are enough of them to
    // fill the 256 CUs and their stages fit the LDS (up to 4-bit codes);
    // otherwise 256 x 128 tiles with four waves.
    const bool wide = ((a.M + 255) / 256) * ((a.N + 255) / 256) >= 384;
    switch (a.bits) {
    case 2: return wide ? run_gemm<2, DT, 256, 256, 512>(a, st) : run_gemm<2, DT, 256, 128, 256>(a, st);
    case 3: return wide ? run_gemm<3, DT, 256, 256, 512>(a, st) : run_gemm<3, DT, 256, 128, 256>(a, st);
    case 4: return wide ? run_gemm<4, DT, 256, 256, 512>(a, st) : run_gemm<4, DT, 256, 128, 256>(a, st);
    case 6: return run_gemm<6, DT, 256, 128, 256>(a, st);
    case 8: return run_gemm<8, DT, 256, 128, 256>(a, st);
    }
    return hipErrorInvalidValue;
}

// Microscaled modes: the same tiles, codes converted by the gfx950 FP4 / FP8
// instructions and scaled exactly (mx.hpp); one-byte scales, no biases.
template <int MODE, int DT, int BM, int BN, int NT>
hipError_t run_gemm_mx(const GemvMxArgs& a, hipStream_t st)
{
    constexpr int BITS = MxFmt<MODE>::BITS, NA = 3, NC = 4;
    constexpr int LDS = gemm::lds_bytes<BITS, BM, BN, NT, NA, NC, MODE>();
    static_assert(LDS <= 160 * 1024, "LDS budget");
    const void* kern = reinterpret_cast<const void*>(
        &gemm::qgemm_tile_kernel<BITS, DT, BM, BN, NT, 2, 1, false, NA, NC, MODE>);
    static bool attr_set = false; // per instantiation; set before its first launch
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    GemmArgs g{};
    g.x = a.x;
    g.wq[0] = g.wq[1] = a.wq;
    g.scales[0] = g.scales[1] = a.scales;
    g.biases[0] = g.biases[1] = nullptr;   // never read in the microscaled modes
    g.y = a.y;
    g.M = (int)a.M;
    g.N = (int)a.N;
    g.K = (int)a.K;
    g.gs = MxFmt<MODE>::GS;
    g.x_bytes = (uint32_t)(a.M * a.K * 2);
    g.y_bytes = (uint32_t)(a.M * a.N * 2);
    g.sb_bytes = (uint32_t)((a.N * (a.K / MxFmt<MODE>::GS) + 3) & ~int64_t(3));
    g.tiles_n = (int)((a.N + BN - 1) / BN);
    g.tiles = (int)((a.M + BM - 1) / BM) * g.tiles_n;
    g.per_xcd = (g.tiles + 7) / 8;
    hipLaunchKernelGGL((gemm::qgemm_tile_kernel<BITS, DT, BM, BN, NT, 2, 1, false, NA, NC, MODE>),
                       dim3(g.per_xcd * 8), dim3(NT), LDS, st, g);
    return hipGetLastError();
}

template <int MODE, int DT>
hipError_t run_gemm_mx_dt(const GemvMxArgs& a, hipStream_t st)
{
    // As for the affine codes: wide tiles for 4-bit lanes when there are
    // enough of them, else 256 x 128.
    if constexpr (MxFmt<MODE>::BITS == 4) {
        if (((a.M + 255) / 256) * ((a.N + 255) / 256) >= 384)
            return run_gemm_mx<MODE, DT, 256, 256, 512>(a, st);
    }
    return run_gemm_mx<MODE, DT, 256, 128, 256>(a, st);
}

template <int MODE>
hipError_t run_gemm_mx_mode(const GemvMxArgs& a, hipStream_t st)
{
    if (a.dt == DT_BF16)
        return run_gemm_mx_dt<MODE, DT_BF16>(a, st);
    if (a.dt == DT_F16)
        return run_gemm_mx_dt<MODE, DT_F16>(a, st);
    return hipErrorInvalidValue;
}

} // namespace

bool qgemm_mx_fits(const GemvMxArgs& a)
{
    const int bits = a.mode == MODE_MXFP8 ? 8 : 4, gs = a.mode == MODE_NVFP4 ? 16 : 32;
    return (a.dt == DT_BF16 || a.dt == DT_F16) && a.K % gemm::BK == 0 &&
           reinterpret_cast<uintptr_t>(a.scales) % 4 == 0 &&
           a.M * a.K * 2 < (int64_t(1) << 31) && a.N * (a.K * bits / 8) < (int64_t(1) << 31) &&
           a.N * (a.K / gs) < (int64_t(1) << 31) - 4 && a.M * a.N * 2 < (int64_t(1) << 31) &&
           a.K < (int64_t(1) << 30);
}

hipError_t launch_qgemm_mx(const GemvMxArgs& a, hipStream_t stream)
{
    switch (a.mode) {
    case MODE_MXFP4: return run_gemm_mx_mode<MODE_MXFP4>(a, stream);
    case MODE_MXFP8: return run_gemm_mx_mode<MODE_MXFP8>(a, stream);
    case MODE_NVFP4: return run_gemm_mx_mode<MODE_NVFP4>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_qgemm(const GemvArgs& a, hipStream_t stream)
{
    // 32-bit buffer offsets (every operand below 2 GB), whole 64-wide k steps
    // and scales / biases readable as aligned dwords; otherwise the GEMV path
    // (in chunks of activation rows) covers the shape.
    const bool fits = a.K % gemm::BK == 0 && reinterpret_cast<uintptr_t>(a.scales) % 4 == 0 &&
                      reinterpret_cast<uintptr_t>(a.biases) % 4 == 0 &&
                      a.M * a.K * 2 < (int64_t(1) << 31) &&
                      a.N * (a.K * a.bits / 8) < (int64_t(1) << 31) &&
                      a.M * a.N * 2 < (int64_t(1) << 31) && a.K < (int64_t(1) << 30);
    if (!fits)
        return launch_qgemv(a, stream);
    if (a.dt == DT_BF16)
        return run_gemm_dt<DT_BF16>(a, stream);
    if (a.dt == DT_F16)
        return run_gemm_dt<DT_F16>(a, stream);
    return launch_qgemv(a, stream);
}

} // namespace qp
