// qgemv.hip — dense decode GEMV (M <= 16): y[m, n] = x[m, :] @ dequant(W[n, :])
// (emily lib/emily/quantization.ex, `quantized_matmul/2` docs). The kernel is
// the streaming GEMV of gemv_core.hpp with a single tile holding the M
// activation rows; M above the register budget of one tile is split into
// chunks, each streaming the weights once.
#include <stdlib.h>

#include "gemv_core.hpp"
#include "skinny.hpp"
#include "rowstream.hpp"
#include "skinny4.hpp"
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
    k.out_bytes = (uint32_t)(mc * a.N * elem_size);
    k.x_bytes = (uint32_t)(mc * a.K * elem_size);
    return k;
}


// Launch shape: at most one block per CU (256 blocks) holding W waves
// (4 <= W <= 10) so that all CUs get the same share; each wave keeps D rows
// (the ring depth the register budget allows) in flight and loops over the
// ring for the rest.
constexpr int kCUs = 256;

template <int BITS, int DT, int MT, int U, int G, int KL>
hipError_t run_fast(const GemvArgs& a, int64_t m0, int mc, hipStream_t st)
{
    // 512-thread blocks (256 VGPRs per lane): the fp32 activation slices take
    // 32 VGPRs per unit and activation row.
    constexpr int MAXT = (U == 3 || MT == 4) ? 256 : 512;
    // Waves per block: 10 measured best for the 14336 x 4096 decode shape.
    constexpr int WMAX = MAXT / 64 < 10 ? MAXT / 64 : 10;
    constexpr int D = ring_depth<BITS, DT, MT, U, G, 1, (131072 / MAXT < 512 ? 131072 / MAXT : 512)>();
    constexpr int RPW = 64 / KL;
    const int64_t passes = (a.N + RPW - 1) / RPW;
    const int64_t waves = (passes + D - 1) / D;
    int64_t W = (waves + kCUs - 1) / kCUs;
    W = W < 4 ? 4 : (W > WMAX ? WMAX : W);
    int64_t blocks = (waves + W - 1) / W;
    blocks = blocks < kCUs ? blocks : kCUs;
    GemvKernelArgs k = dense_args(a, m0, mc, (int)sizeof(St<DT>), KL);
    hipLaunchKernelGGL((qgemv_stream_kernel<BITS, DT, MT, U, G, KL, 1, MAXT>),
                       dim3((int)blocks), dim3((int)W * 64), 0, st, k);
    return hipGetLastError();
}

// The lane slice of U units lies in one quantization group when the group
// size is a multiple of the slice.
template <int BITS, int DT, int MT, int U, int KL>
hipError_t run_slice(const GemvArgs& a, int64_t m0, int mc, hipStream_t st)
{
    if constexpr (U > 1) {
        if (a.gs % (32 * U) == 0)
            return run_fast<BITS, DT, MT, U, 1, KL>(a, m0, mc, st);
        return run_fast<BITS, DT, MT, U, U, KL>(a, m0, mc, st);
    } else {
        return run_fast<BITS, DT, MT, 1, 1, KL>(a, m0, mc, st);
    }
}

// Shapes with a one-wave-per-row (or finer) register-resident kernel; others
// take the generic kernel.
template <int BITS, int DT, int MT>
hipError_t run_chunk(const GemvArgs& a, int64_t m0, int mc, hipStream_t st, bool* done)
{
    *done = true;
    const int64_t K = a.K;
    if (K == 2 * 32 * 64) return run_slice<BITS, DT, MT, 2, 64>(a, m0, mc, st);
    if (K == 1 * 32 * 64) return run_slice<BITS, DT, MT, 1, 64>(a, m0, mc, st);
    if (K == 3 * 32 * 8) {
        // One activation row per pass: two rows' fp32 slices of three units
        // would not fit the registers.
        for (int i = 0; i < mc; ++i)
            if (hipError_t e = run_fast<BITS, DT, 1, 3, 3, 8>(a, m0 + i, 1, st); e != hipSuccess)
                return e;
        return hipSuccess;
    }
    if constexpr (MT <= 2) {
        if (K == 32 * 32) return run_slice<BITS, DT, MT, 1, 32>(a, m0, mc, st);
    }
    *done = false;
    return hipSuccess;
}

// Any K and any activation alignment; up to 16 rows per launch.
template <int BITS, int DT>
hipError_t run_generic(const GemvArgs& a, hipStream_t st)
{
    int64_t blocks = (a.N + 3) / 4;
    if (blocks > kMaxBlocks)
        blocks = kMaxBlocks;
    for (int64_t m0 = 0; m0 < a.M; m0 += 16) {
        const int mc = (int)((a.M - m0) < 16 ? (a.M - m0) : 16);
        GemvKernelArgs k = dense_args(a, m0, mc, (int)sizeof(St<DT>), 64);
        hipLaunchKernelGGL((qgemv_generic_kernel<BITS, DT, 1>), dim3((int)blocks), dim3(256), 0,
                           st, k);
        if (hipError_t e = hipGetLastError(); e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// Three to sixteen activation rows (16-bit activations) on the 16x16x32
// matrix instruction with exact codes (skinny.hpp): about one block per CU
// over a contiguous range of weight rows, 16 activation rows per launch.
template <int BITS, int DT>
hipError_t run_skinny(const GemvArgs& a, hipStream_t st, bool* done)
{
    *done = false;
    // Activation rows are read in 16-byte pieces.
    if (a.K % 32 != 0 || reinterpret_cast<uintptr_t>(a.x) % 16 != 0)
        return hipSuccess;   // another kernel takes this shape
    SkinnyShape sh{};
    dim3 grid;
    skinny_dense_shape(a.N, a.K, &sh, &grid);
    for (int64_t m0 = 0; m0 < a.M; m0 += 16) {
        const int rows = (int)((a.M - m0) < 16 ? (a.M - m0) : 16);
        GemvKernelArgs k = dense_args(a, m0, rows, (int)sizeof(St<DT>), 0);
        if constexpr ((BITS == 2 || BITS == 3 || BITS == 4 || BITS == 6) && DT != DT_F32) {
            // 6-, 4-, 3- and 2-bit codes with rows of scales in whole 16-byte
            // pieces: the row-contiguous form (skinny4.hpp). Measured (graph-
            // replayed): 14336 x 4096 M = 16 13.2 us against 15.4, M = 8 12.2
            // against 14.6; 4096 x 14336 M = 16 18.3 against 25.5; 2-bit
            // 14336 x 4096 M = 16 11.9 against 12.5, 4096 x 14336 M = 16 18.3
            // against 21.7; 3-bit (queued launches) 14336 x 4096 M = 16 14.2
            // against 16.7, 4096 x 4096 M = 8 8.3 against 9.6 at gs 64; 6-bit
            // 4096 x 14336 M = 16 26.7 against 30.6, 14336 x 4096 M = 16 18.2
            // against 18.7, but 4096 x 4096 M = 8 10.7 against 10.2 and, at
            // gs 32 (whose scales and biases take 16 more registers, which
            // spills), 14.4 against 11.3: so 6-bit codes take it from gs 64 and
            // 2^25 codes. 8-bit codes measured no faster this way.
            const bool wide = BITS != 6 || (a.gs >= 64 && (int64_t)a.N * a.K >= (int64_t(1) << 25));
            const bool fit = wide && (2 * (a.K / a.gs)) % 16 == 0 && reinterpret_cast<uintptr_t>(a.scales) % 16 == 0 &&
                             reinterpret_cast<uintptr_t>(a.biases) % 16 == 0 &&
                             reinterpret_cast<uintptr_t>(a.wq) % 16 == 0 && sh.rows_per_block % 16 == 0;
            if (fit) {
                if (hipError_t e = skinny4_launch<BITS, DT>(k, sh, grid, st); e != hipSuccess)
                    return e;
                continue;
            }
        }
        if (hipError_t e = skinny_launch<BITS, DT, 1>(k, sh, grid, st); e != hipSuccess)
            return e;
    }
    *done = true;
    return hipSuccess;
}

// 2-, 4- and 8-bit codes, one or two 16-bit activation rows: the row-per-wave
// stream kernel (rowstream.hpp), for K a multiple of 32 up to 16384 (at most
// 8 units per lane).
template <int BITS, int DT, int MT, int UPL>
hipError_t run_rowstream(const GemvArgs& a, int64_t m0, int mc, hipStream_t st)
{
    constexpr int D = rowstream_depth<BITS, UPL, MT>();
    RowStreamArgs k{};
    k.x = static_cast<const char*>(a.x) + m0 * a.K * 2;
    k.wq = a.wq;
    k.scales = a.scales;
    k.biases = a.biases;
    k.y = static_cast<char*>(a.y) + m0 * a.N * 2;
    k.M = mc;
    k.N = (int)a.N;
    k.K = (int)a.K;
    k.gs = a.gs;
    k.units_row = (uint32_t)(a.K / 32);
    auto launch = [&](auto wpb) {
        constexpr int WPB = decltype(wpb)::value;
        auto go = [&](auto kl) {
            constexpr int KL = decltype(kl)::value;
            constexpr int ROWS = WPB * (64 / KL) * D;   // weight rows of a block
            int64_t blocks = (a.N + ROWS - 1) / ROWS;
            blocks = blocks < kMaxBlocks ? blocks : kMaxBlocks;
            // Scales and biases as whole dword-aligned rows when a row has an
            // even number of groups.
            if ((a.K / a.gs) % 2 == 0)
                hipLaunchKernelGGL((qgemv_rowstream_kernel<BITS, DT, MT, UPL, WPB, true, KL>),
                                   dim3((int)blocks), dim3(64 * WPB), 0, st, k);
            else
                hipLaunchKernelGGL((qgemv_rowstream_kernel<BITS, DT, MT, UPL, WPB, false, KL>),
                                   dim3((int)blocks), dim3(64 * WPB), 0, st, k);
            return hipGetLastError();
        };
        // Rows of at most 32 units: two rows side by side in a wave.
        if constexpr (UPL == 1) {
            if (a.K <= 32 * 32)
                return go(std::integral_constant<int, 32>{});
        }
        return go(std::integral_constant<int, 64>{});
    };
    return launch(std::integral_constant<int, 4>{});
}

template <int BITS, int DT, int MT>
hipError_t run_rowstream_upl(const GemvArgs& a, int64_t m0, int mc, hipStream_t st)
{
    const int64_t upl = (a.K / 32 + 63) / 64;
    constexpr bool exact = true;
    if (upl <= 1) return run_rowstream<BITS, DT, MT, 1>(a, m0, mc, st);
    if (upl <= 2) return run_rowstream<BITS, DT, MT, 2>(a, m0, mc, st);
    if constexpr (MT <= 2) {
        if (exact && upl <= 3) return run_rowstream<BITS, DT, MT, 3>(a, m0, mc, st);
        if (upl <= 4) return run_rowstream<BITS, DT, MT, 4>(a, m0, mc, st);
    }
    if constexpr (MT == 1) {
        // Units per lane as the row needs them (K = 14336: 7), so that no
        // lane carries a whole unit of zeros through the dot products.
        if (exact && upl <= 5) return run_rowstream<BITS, DT, MT, 5>(a, m0, mc, st);
        if (exact && upl <= 6) return run_rowstream<BITS, DT, MT, 6>(a, m0, mc, st);
        if (exact && upl <= 7) return run_rowstream<BITS, DT, MT, 7>(a, m0, mc, st);
        return run_rowstream<BITS, DT, MT, 8>(a, m0, mc, st);
    }
    // Two rows' activation slices fit in registers up to four units per
    // lane, four rows' up to two.
    return hipErrorInvalidValue;
}

// Three or four activation rows with the products on the 4x4x4 matrix
// instruction: a wave per four weight rows, R rounds of 16 units (up to
// K = 4096: the LDS of four rows' activation slices stays under 64 KB).
template <int BITS, int DT, int R>
hipError_t run_rowmfma_r(const GemvArgs& a, hipStream_t st)
{
    RowStreamArgs k{};
    k.x = a.x;
    k.wq = a.wq;
    k.scales = a.scales;
    k.biases = a.biases;
    k.y = a.y;
    k.M = (int)a.M;
    k.N = (int)a.N;
    k.K = (int)a.K;
    k.gs = a.gs;
    k.units_row = (uint32_t)(a.K / 32);
    int64_t blocks = (a.N + 15) / 16;
    blocks = blocks < kMaxBlocks ? blocks : kMaxBlocks;
    if ((a.K / a.gs) % 2 == 0)
        hipLaunchKernelGGL((qgemv_rowmfma_kernel<BITS, DT, R, true>), dim3((int)blocks), dim3(256), 0,
                           st, k);
    else
        hipLaunchKernelGGL((qgemv_rowmfma_kernel<BITS, DT, R, false>), dim3((int)blocks), dim3(256),
                           0, st, k);
    return hipGetLastError();
}

template <int BITS, int DT>
hipError_t run_rowmfma(const GemvArgs& a, hipStream_t st)
{
    const int64_t rounds = (a.K / 32 + 15) / 16;
    if (rounds <= 1) return run_rowmfma_r<BITS, DT, 1>(a, st);
    if (rounds <= 2) return run_rowmfma_r<BITS, DT, 2>(a, st);
    if (rounds <= 4) return run_rowmfma_r<BITS, DT, 4>(a, st);
    return run_rowmfma_r<BITS, DT, 8>(a, st);
}

template <int BITS, int DT>
hipError_t run_gemv(const GemvArgs& a, hipStream_t st)
{
    constexpr int MTMAX = gemv_max_mt<BITS, DT>();
    // The streaming kernel reads activations as 16-byte vectors.
    const bool x_vec = reinterpret_cast<uintptr_t>(a.x) % 16 == 0;
    // Raw buffer accesses address each matrix and the output with 32-bit
    // offsets.
    const int64_t es = (int64_t)sizeof(St<DT>);
    const bool small = a.N * (a.K * BITS / 8) < (int64_t(1) << 31) &&
                       a.N * (a.K / a.gs) * es < (int64_t(1) << 31) &&
                       a.M * a.N * es < (int64_t(1) << 31);
    if (!x_vec || !small)
        return run_generic<BITS, DT>(a, st);
    if constexpr (DT != DT_F32) {
        // Two rows stream faster with dot products (measured 15.0 vs 16.4 us
        // on the 14336 x 4096 decode shape); three and more go to the matrix cores.
        constexpr int min_m = 3;
        // Three and four rows: measured 12.0 us at 4 bits on 14336 x 4096
        // (15.5 on the tile path below, 14.6 with dot products on four
        // activation rows); one and two rows stay on the dot-product stream
        // (9.0 against 11.3 us at one row).
        if constexpr (BITS == 3 || BITS == 6) {
            // Three and four rows of 3- and 6-bit codes on the row kernel,
            // the four activation rows' slices in registers, where the matrix
            // is small enough that the skinny kernel's set-up dominates:
            // [4096, 4096] M = 4 measured 6.4 us at 3 bits against 8.6 on the
            // skinny kernel, 7.5 against 10.9 at 6 bits; at 14336 rows the
            // skinny kernel was faster (15.7 against 17.0 us at 3 bits).
            if ((a.M == 3 || a.M == 4) && a.K % 32 == 0 && a.K <= 2 * 64 * 32 && a.N <= 8192)
                return run_rowstream_upl<BITS, DT, 4>(a, 0, (int)a.M, st);
        }
        if constexpr (BITS == 2 || BITS == 4 || BITS == 8) {
            if ((a.M == 3 || a.M == 4) && a.K % 32 == 0 && a.K <= 2 * 64 * 32)
                return run_rowmfma<BITS, DT>(a, st);
        }
        if (a.M >= min_m) {
            bool done = false;
            hipError_t e = run_skinny<BITS, DT>(a, st, &done);
            if (e != hipSuccess || done)
                return e;
        }
    }
    if constexpr (DT != DT_F32) {
        // 8-bit codes as well: measured 12.4 against 14.4 us on the slice
        // kernel below at 14336 x 4096, 8.1 against 12.7 at 4096 x 8192.
        if (a.M <= 2 && a.K % 32 == 0 && a.K <= 8 * 64 * 32) {
            // Two activation rows per pass up to four units per lane, else one.
            const int rows = a.K <= 4 * 64 * 32 ? 2 : 1;
            for (int64_t m0 = 0; m0 < a.M; m0 += rows) {
                const int mc = (int)((a.M - m0) < rows ? (a.M - m0) : rows);
                hipError_t e = mc == 2 ? run_rowstream_upl<BITS, DT, 2>(a, m0, mc, st)
                                       : run_rowstream_upl<BITS, DT, 1>(a, m0, mc, st);
                if (e != hipSuccess)
                    return e;
            }
            return hipSuccess;
        }
    }
    for (int64_t m0 = 0; m0 < a.M;) {
        const int mc = (int)((a.M - m0) < MTMAX ? (a.M - m0) : MTMAX);
        bool done = false;
        hipError_t e;
        if (mc == 1) {
            e = run_chunk<BITS, DT, 1>(a, m0, mc, st, &done);
        } else if (mc == 2) {
            e = run_chunk<BITS, DT, 2>(a, m0, mc, st, &done);
        } else if constexpr (MTMAX >= 4) {
            e = run_chunk<BITS, DT, 4>(a, m0, mc, st, &done);
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
