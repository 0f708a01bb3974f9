// qgemv_t.hip — the transpose = false product (emily lib/emily/quantization.ex,
// `quantized_matmul/2`: with transpose = false the packed weight is read as
// already transposed, the AWQ convention): W is stored [K, N], each row of N
// lanes packed and grouped along N, and y = x @ dequant(W):
//   y[m, j] = sum_i x[m, i] * (q[i, j] * s[i, j/gs] + b[i, j/gs]).
//
// A row of W is contiguous along the output index, so a lane owns a fixed
// slice of 32 output columns (one 32-code unit, one group) and walks down
// every fourth row of its wave's share, folding the affine map into
// q * (x s) + x b; 16 lanes cover a row's 512 columns of the block's tile.
// A block's four waves take interleaved rows of its K range; row groups meet
// by shuffles and waves in LDS. Blocks split K further and write fp32
// partial sums to the caller's workspace, which a second kernel adds in split
// order (so results do not depend on scheduling) and rounds to the
// activation type.
#include "common.hpp"
#include "gemv_core.hpp"
#include "launch.hpp"

namespace qp {

namespace {

// A lane's chunk of a row: one 32-code unit (BITS words, one group). Lanes
// 16 r .. 16 r + 15 of a wave take row group r (rows i with i % 4 == r of
// the wave's rows), so one load instruction covers 4 rows x 16 units and a
// wave tile is 512 columns at every width.
template <int BITS> struct TChunk {
    static constexpr int WORDS = BITS;
    static constexpr int CODES = 32;
    static constexpr int MT_MAX = qgemv_t_rows(BITS);           // activation rows per pass
};

constexpr int kRowsInFlight = 4;
constexpr int kWaves = 4;                                       // waves per block
constexpr int kTileCols = 512;                                  // columns per block

template <int BITS, int DT, int MT, bool VEC>
__global__ __launch_bounds__(64 * kWaves) void qgemv_t_partial_kernel(QgemvTArgs a, int splits,
                                                                      int rows_per_split,
                                                                      float* __restrict__ partial)
{
    using C = TChunk<BITS>;
    using E = Elem<DT>;
    using St = typename E::storage;
    constexpr int U = kRowsInFlight;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    constexpr int RS = 4 * kWaves;                              // row streams per block
    __shared__ float red[kWaves - 1][MT][C::CODES][16];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = lane >> 4, cl = lane & 15;
    const int split = (int)blockIdx.x % splits, tile = (int)blockIdx.x / splits;
    const int64_t units_row = a.N / 32;
    const int64_t unit = (int64_t)tile * 16 + cl;
    const bool live = unit < units_row;
    const int64_t words_row = a.N * BITS / 32, groups_row = a.N / a.gs;
    const int64_t g = live ? (unit * 32) / a.gs : 0;
    const int k0 = split * rows_per_split;
    const int k1 = k0 + rows_per_split < a.K ? k0 + rows_per_split : a.K;

    const St* xs = static_cast<const St*>(a.x);
    const St* sc = static_cast<const St*>(a.scales);
    const St* bi = static_cast<const St*>(a.biases);
    float acc[MT][C::CODES], accb[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        accb[m] = 0.0f;
#pragma unroll
        for (int c = 0; c < C::CODES; ++c)
            acc[m][c] = 0.0f;
    }
    for (int i0 = k0 + wave * 4 + rg; i0 < k1; i0 += RS * U) {
        uint32_t w[U][C::WORDS];
        St s_raw[U], b_raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + RS * u;
            const bool ok = live && i < k1;
            const int ii = ok ? i : k0;   // an in-bounds row; its terms are not used
            const uint32_t* p = a.wq + (size_t)ii * words_row + (live ? unit : 0) * C::WORDS;
            if constexpr (VEC && C::WORDS % 4 == 0) {   // 16-byte aligned units
#pragma unroll
                for (int v = 0; v < C::WORDS; v += 4) {
                    const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + v));
                    w[u][v] = q.x; w[u][v + 1] = q.y; w[u][v + 2] = q.z; w[u][v + 3] = q.w;
                }
            } else {
#pragma unroll
                for (int v = 0; v < C::WORDS; ++v)
                    w[u][v] = __builtin_nontemporal_load(p + v);
            }
            s_raw[u] = sc[(size_t)ii * groups_row + g];
            b_raw[u] = bi[(size_t)ii * groups_row + g];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + RS * u;
            if (!(live && i < k1))
                continue;
            const float s = E::to_f32(s_raw[u]), b = E::to_f32(b_raw[u]);
            float xsv[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float xv = m < a.M ? E::to_f32(xs[(int64_t)m * a.K + i]) : 0.0f;
                xsv[m] = xv * s;
                accb[m] = __builtin_fmaf(xv, b, accb[m]);
            }
            if constexpr (BITS == 4) {
                // Codes 8v .. 8v + 7 of word v, exact in fp32 two at a time:
                // a mask per nibble parity puts them in bytes, and the FP8
                // (E4M3) pair conversion with scale 2^9 returns each byte
                // b <= 15 as b itself.
#pragma unroll
                for (int v = 0; v < C::WORDS; ++v) {
                    const uint32_t ev = w[u][v] & 0x0F0F0F0Fu, od = (w[u][v] >> 4) & 0x0F0F0F0Fu;
                    const f32x2_t e01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 512.0f, false);
                    const f32x2_t e23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 512.0f, true);
                    const f32x2_t o01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 512.0f, false);
                    const f32x2_t o23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 512.0f, true);
                    const float q[8] = {e01.x, o01.x, e01.y, o01.y, e23.x, o23.x, e23.y, o23.y};
#pragma unroll
                    for (int j = 0; j < 8; ++j)
#pragma unroll
                        for (int m = 0; m < MT; ++m)
                            acc[m][8 * v + j] = __builtin_fmaf(q[j], xsv[m], acc[m][8 * v + j]);
                }
            } else {
#pragma unroll
                for (int c = 0; c < C::CODES; ++c) {
                    const int bit = c * BITS, wi = bit / 32, sh = bit % 32;
                    uint32_t qc;
                    if (sh + BITS <= 32)
                        qc = (w[u][wi] >> sh) & mask;
                    else
                        qc = __builtin_amdgcn_alignbit(w[u][wi + 1], w[u][wi], sh) & mask;
                    const float q = (float)qc;
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        acc[m][c] = __builtin_fmaf(q, xsv[m], acc[m][c]);
                }
            }
        }
    }
    // Row groups of a wave, then the waves of the block, are added in a fixed
    // order: lanes cl, cl + 16, cl + 32, cl + 48 by two xor shuffles; waves
    // 1..3 through LDS into wave 0.
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < C::CODES; ++c) {
            float v = acc[m][c] + accb[m];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[m][c] = v;
        }
    if (wave > 0 && rg == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int c = 0; c < C::CODES; ++c)
                red[wave - 1][m][c][cl] = acc[m][c];
    }
    __syncthreads();
    if (wave == 0 && rg == 0 && live) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m >= a.M)
                continue;
            float* out = partial + ((size_t)split * a.M + m) * a.N + unit * 32;
#pragma unroll
            for (int c = 0; c < C::CODES; ++c) {
                float v = acc[m][c];
#pragma unroll
                for (int wv = 0; wv < kWaves - 1; ++wv)
                    v += red[wv][m][c][cl];
                out[c] = v;
            }
        }
    }
}

template <int DT>
__global__ __launch_bounds__(256) void qgemv_t_reduce_kernel(const float* __restrict__ partial,
                                                             int splits, int64_t mn,
                                                             typename Elem<DT>::storage* __restrict__ y)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn;
         i += (int64_t)gridDim.x * blockDim.x) {
        // Splits added in order; eight loads in flight at a time.
        float v = 0.0f;
        int s = 0;
        for (; s + 8 <= splits; s += 8) {
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                t[j] = partial[(size_t)(s + j) * mn + i];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v += t[j];
        }
        for (; s < splits; ++s)
            v += partial[(size_t)s * mn + i];
        y[i] = Elem<DT>::from_f32(v);
    }
}

constexpr int kTargetBlocks = 1024;

template <int BITS, int MT, bool VEC>
hipError_t run_t_mt(const QgemvTArgs& a, int64_t mc, const void* x, void* y, float* partial,
                    int splits, int rows_per_split, hipStream_t st)
{
    using C = TChunk<BITS>;
    QgemvTArgs k = a;
    k.x = x;
    k.M = mc;
    (void)sizeof(C);
    const int64_t tiles = (a.N + kTileCols - 1) / kTileCols;
    const dim3 grid((unsigned)(tiles * splits));
    switch (a.dt) {
    case DT_F32:
        hipLaunchKernelGGL((qgemv_t_partial_kernel<BITS, DT_F32, MT, VEC>), grid, dim3(64 * kWaves), 0, st, k,
                           splits, rows_per_split, partial);
        break;
    case DT_F16:
        hipLaunchKernelGGL((qgemv_t_partial_kernel<BITS, DT_F16, MT, VEC>), grid, dim3(64 * kWaves), 0, st, k,
                           splits, rows_per_split, partial);
        break;
    case DT_BF16:
        hipLaunchKernelGGL((qgemv_t_partial_kernel<BITS, DT_BF16, MT, VEC>), grid, dim3(64 * kWaves), 0, st, k,
                           splits, rows_per_split, partial);
        break;
    default:
        return hipErrorInvalidValue;
    }
    if (hipError_t e = hipGetLastError(); e != hipSuccess)
        return e;
    const int64_t mn = mc * a.N;
    int64_t blocks = (mn + 255) / 256;
    blocks = blocks < 4096 ? blocks : 4096;
    switch (a.dt) {
    case DT_F32:
        hipLaunchKernelGGL((qgemv_t_reduce_kernel<DT_F32>), dim3((int)blocks), dim3(256), 0, st,
                           partial, splits, mn, static_cast<float*>(y));
        break;
    case DT_F16:
        hipLaunchKernelGGL((qgemv_t_reduce_kernel<DT_F16>), dim3((int)blocks), dim3(256), 0, st,
                           partial, splits, mn, static_cast<uint16_t*>(y));
        break;
    default:
        hipLaunchKernelGGL((qgemv_t_reduce_kernel<DT_BF16>), dim3((int)blocks), dim3(256), 0, st,
                           partial, splits, mn, static_cast<uint16_t*>(y));
        break;
    }
    return hipGetLastError();
}

template <int BITS>
hipError_t run_t_bits(const QgemvTArgs& a, hipStream_t st)
{
    const QgemvTPlan p = qgemv_t_plan(a.M, a.K, a.N, a.bits);
    const int es = a.dt == DT_F32 ? 4 : 2;
    constexpr int MTX = TChunk<BITS>::MT_MAX;
    const bool vec = reinterpret_cast<uintptr_t>(a.wq) % 16 == 0;
    for (int64_t m0 = 0; m0 < a.M; m0 += MTX) {
        const int64_t mc = a.M - m0 < MTX ? a.M - m0 : MTX;
        const void* x = static_cast<const char*>(a.x) + m0 * a.K * es;
        void* y = static_cast<char*>(a.y) + m0 * a.N * es;
        hipError_t e;
        if (vec)
            e = mc == 1   ? run_t_mt<BITS, 1, true>(a, mc, x, y, a.workspace, p.splits, p.rows_per_split, st)
                : mc == 2 ? run_t_mt<BITS, 2, true>(a, mc, x, y, a.workspace, p.splits, p.rows_per_split, st)
                          : run_t_mt<BITS, MTX, true>(a, mc, x, y, a.workspace, p.splits, p.rows_per_split, st);
        else
            e = mc == 1   ? run_t_mt<BITS, 1, false>(a, mc, x, y, a.workspace, p.splits, p.rows_per_split, st)
                : mc == 2 ? run_t_mt<BITS, 2, false>(a, mc, x, y, a.workspace, p.splits, p.rows_per_split, st)
                          : run_t_mt<BITS, MTX, false>(a, mc, x, y, a.workspace, p.splits, p.rows_per_split, st);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

} // namespace

QgemvTPlan qgemv_t_plan(int64_t m, int64_t k, int64_t n, int bits)
{
    (void)bits;
    const int64_t tiles = (n + kTileCols - 1) / kTileCols;
    int64_t splits = tiles > 0 ? (kTargetBlocks + tiles - 1) / tiles : 1;
    const int64_t max_splits = k / 16 > 1 ? k / 16 : 1;   // at least 16 rows per block
    splits = splits < max_splits ? splits : max_splits;
    splits = splits > 0 ? splits : 1;
    QgemvTPlan p;
    p.rows_per_split = (int)((k + splits - 1) / splits);
    p.splits = (int)((k + p.rows_per_split - 1) / p.rows_per_split);
    const int64_t mrows = m < qgemv_t_rows(bits) ? m : qgemv_t_rows(bits);
    p.workspace_bytes = (size_t)p.splits * (size_t)mrows * (size_t)n * 4;
    return p;
}

hipError_t launch_qgemv_t(const QgemvTArgs& a, hipStream_t st)
{
    switch (a.bits) {
    case 2: return run_t_bits<2>(a, st);
    case 3: return run_t_bits<3>(a, st);
    case 4: return run_t_bits<4>(a, st);
    case 6: return run_t_bits<6>(a, st);
    case 8: return run_t_bits<8>(a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace qp
