// rowstream.hpp — the decode GEMV for 2-, 3-, 4-, 6- and 8-bit codes with a
// weight row per wave (or per 32-lane half of one, for rows of at most 32
// units), and its three- and four-row form on the 4x4x4 matrix instruction
// (emily lib/emily/quantization.ex, `quantized_matmul/2`; affine codes of
// `dequantize_defn/1`):
//   y[m, n] = sum_g s'[n,g] * sum_{k in g} x q + b'[n,g] * sum_{k in g} x.
//
// Lane l of a row's KL lanes takes the 32-code units l, l + KL, ... of the
// row, so its slice of the activation rows is fixed for the whole launch and
// sits in registers. A unit is BITS code words; its 32 codes become 16 exact
// 16-bit pairs (codepair.hpp: FP8 / FP4 conversion of split code bytes, the
// 3-bit fields spread to bytes first; bytes through fp32 at 6 and 8 bits),
// and the activation pairs are stored in the same order. v_dot2 forms
// sum x q per unit, and the group's scale and bias, oriented so that the
// folded bias does not cancel against the codes, are applied once per unit.
// D rows are loaded before any is reduced. One or two activation rows share
// a pass (and, for 3- and 6-bit codes on small matrices, up to four: their
// slices in registers up to two units per lane).
//
// Every wave of a block needs the same activation slices, so the block
// prepares them once: its threads load the raw activation units, permute
// them and form their sums into LDS, and each wave then copies its slices
// from there. The first row batch's loads are issued before that set-up (and
// after the raw activation loads, which are waited for first), so the set-up
// runs under the weight stream's latency.
#pragma once

#include "common.hpp"
#include "codepair.hpp"
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
    static __device__ __forceinline__ float dot(uint32_t a, uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, x), acc, false);
    }
};
template <> struct RowStreamPair<DT_F16> {
    static __device__ __forceinline__ float dot(uint32_t a, uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, x),
                                      acc, false);
    }
};

// Rows per wave: about 24 VGPRs of codes, from 1 to 4 rows. Each wave
// computes its rows after they arrive, so the rows of the last waves to be
// served are the kernel's tail; fewer rows per wave (and more waves) shorten
// it. Measured on the 14336 x 4096 decode (device time, events over
// back-to-back launches): 4-bit 3 rows 8.0 us against 4 rows 8.6 us and 2
// rows 8.2 us; 8-bit 1 row 11.8 us against 2 rows 12.2 us; 2-bit 4 rows 7.0
// us against 3 rows 7.2 us and 6 rows 8.0 us; at K = 14336 (seven units per
// lane) one row 10.3 us against two 11.1 us. Three-bit units cost the most
// VALU work per byte (the fields are spread to bytes first), so their waves
// take half as many rows: 14336 x 4096 3-bit 8.7 us with 2 rows against 9.6
// us with 4; at 6 bits one row (12.4 us) was slower than two (11.9 us).
// Two activation rows double the dot products per row, and two rows per wave
// measured best for them at up to two units per lane (14336 x 4096, M = 2:
// 4-bit 9.85 us against 10.5 with three rows, 8-bit 13.1 against 14.7 with
// one, 2-bit 8.9 against 9.5 with four). Two-bit rows of seven or eight units
// per lane take two rows rather than one (4096 x 14336: 8.3 us against 9.7).
template <int BITS, int UPL, int MT = 1> constexpr int rowstream_depth()
{
    constexpr int B = BITS == 3 ? 12 : 24;
    constexpr int d = B / (BITS * UPL) < 1 ? 1 : (B / (BITS * UPL) > 4 ? 4 : B / (BITS * UPL));
    if constexpr (MT == 2 && UPL <= 2 && (BITS == 2 || BITS == 4 || BITS == 8))
        return 2;
    else if constexpr (BITS == 2 && d < 2)
        return 2;
    else
        return d;
}

template <int BITS, int DT, int MT, int UPL, int WPB, bool WIDE, int KL>
__global__ __launch_bounds__(64 * WPB) void qgemv_rowstream_kernel(RowStreamArgs a)
{
    using PX = RowStreamPair<DT>;
    using E = Elem<DT>;
    using St = typename E::storage;
    static_assert(BITS == 2 || BITS == 3 || BITS == 4 || BITS == 6 || BITS == 8, "code widths");
    constexpr int D = rowstream_depth<BITS, UPL, MT>();
    using CO = CodeOrder<BITS>;
    const int lane = threadIdx.x & 63;
    // A wave is S slots of KL lanes (KL = 32 for rows of at most 32 units, so
    // that half the wave does not idle); slot s owns D rows.
    static_assert(KL == 32 || KL == 64, "32 or 64 lanes per row");
    constexpr int S = 64 / KL;
    const int kl = lane % KL, slot = lane / KL;
    const int gw = (int)blockIdx.x * WPB + (int)(threadIdx.x >> 6);
    const int GW = (int)gridDim.x * WPB;

    constexpr int UNITS = KL * UPL;                  // unit slots of one activation row
    constexpr int ENTRIES = MT * UNITS;              // (row, unit) slices set up per block
    constexpr int EPT = (ENTRIES + 64 * WPB - 1) / (64 * WPB);   // slices per thread
    // Permuted pairs of slice (m, u) as four 4-word vectors xl[m][q][u], and
    // its sum: consecutive lanes touch consecutive vectors.
    __shared__ u32x4_t xl[MT][4][UNITS];
    __shared__ float sl[MT][UNITS];

    const uint32_t row_bytes = (uint32_t)a.K * BITS / 8;
    const uint32_t groups_row = (uint32_t)(a.K / a.gs);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.wq, (uint32_t)a.N * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales, (uint32_t)a.N * groups_row * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.biases, (uint32_t)a.N * groups_row * 2);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)a.K * 2);
    St* y = static_cast<St*>(a.y);
    uint32_t gofs[UPL];
#pragma unroll
    for (int j = 0; j < UPL; ++j)
        gofs[j] = (uint32_t)((32 * (kl + KL * j)) / a.gs) * 2;

    // Raw activation slices of this thread: raw[e][k / 2] holds x[k] (low)
    // and x[k + 1] (high) of the 32 activations of its slice (zeros past the
    // row or the activation rows).
    uint32_t raw[EPT][16];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int idx = (int)threadIdx.x + 64 * WPB * e, m = idx / UNITS, u = idx % UNITS;
        const bool live = idx < ENTRIES && m < a.M && u < (int)a.units_row;
        buffer_words<16>(rx, live ? ((uint32_t)m * (uint32_t)a.K + 32u * (uint32_t)u) * 2 : OOB,
                         raw[e]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // WIDE (an even number of groups per row): a batch's scales and biases
    // are D whole rows, contiguous and dword-aligned, read as lane-contiguous
    // dwords (NV loads per array instead of D * UPL) and handed to the lanes
    // that need them through the wave's own LDS slots.
    constexpr int SBD = 32 * D * UPL;                // dwords of one batch's scales, gs >= 32
    constexpr int NV = (SBD + 63) / 64;
    __shared__ uint32_t sbl[WPB][2][WIDE ? SBD : 1];
    const int wv = (int)(threadIdx.x >> 6);
    const uint32_t nd = (uint32_t)(S * D) * groups_row / 2;   // the wave's S * D rows
    uint32_t sw[NV], bw[NV];
    uint32_t w[D][UPL][BITS];
    St sv[D][UPL], bv[D][UPL];
    auto load = [&](int r0) {
        if constexpr (WIDE) {
            const uint32_t base = (uint32_t)r0 * groups_row * 2;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const uint32_t i = (uint32_t)(lane + 64 * v);
                const uint32_t off = i < nd ? base + 4 * i : OOB;
                sw[v] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
                bw[v] = __builtin_amdgcn_raw_buffer_load_b32(rb, off, 0, 0);
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int j = 0; j < UPL; ++j) {
                const int u = kl + KL * j, r = r0 + slot * D + d;
                const bool live = u < (int)a.units_row && r < a.N;
                buffer_words<BITS, BITS == 8 ? 0 : kStreamPolicy>(
                    rw, live ? (uint32_t)r * row_bytes + (uint32_t)u * (4 * BITS) : OOB, w[d][j]);
                if constexpr (!WIDE) {
                    const uint32_t so = live ? (uint32_t)r * groups_row * 2 + gofs[j] : OOB;
                    sv[d][j] = buffer_elem<DT>(rs, so);
                    bv[d][j] = buffer_elem<DT>(rb, so);
                }
            }
    };
    // Units past the row take zero scale and bias, as the per-lane loads
    // give them (their codes and activations are zero as well).
    auto exchange = [&]() {
        if constexpr (WIDE) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const uint32_t i = (uint32_t)(lane + 64 * v);
                if (i < nd) {
                    sbl[wv][0][i] = sw[v];
                    sbl[wv][1][i] = bw[v];
                }
            }
#pragma unroll
            for (int d = 0; d < D; ++d)
#pragma unroll
                for (int j = 0; j < UPL; ++j) {
                    const bool live = kl + KL * j < (int)a.units_row;
                    // Element e = d * groups + g of the batch sits in half
                    // e % 2 of slot e / 2 (little-endian); e / 2 < SBD for
                    // every lane, live or not. Read as the slots' own type.
                    const uint32_t e = (uint32_t)(slot * D + d) * groups_row + gofs[j] / 2;
                    const uint32_t ds = sbl[wv][0][e >> 1], db = sbl[wv][1][e >> 1];
                    const uint32_t sh = 16 * (e & 1);
                    sv[d][j] = live ? St(ds >> sh) : St(0);
                    bv[d][j] = live ? St(db >> sh) : St(0);
                }
        }
    };
    int r0 = gw * S * D;
    load(r0);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int idx = (int)threadIdx.x + 64 * WPB * e, m = idx / UNITS, u = idx % UNITS;
        if (idx < ENTRIES) {
            // Pair q holds the activations of codes lo_code(q) (low half) and
            // hi_code(q) (high half) of the unit.
            uint32_t p[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int k0 = CO::lo_code(q), k1 = CO::hi_code(q);
                const uint32_t lo = (raw[e][k0 / 2] >> (16 * (k0 & 1))) & 0xFFFFu;
                const uint32_t hi = (raw[e][k1 / 2] >> (16 * (k1 & 1))) & 0xFFFFu;
                p[q] = lo | (hi << 16);
            }
            float sum = 0.0f;
#pragma unroll
            for (int k = 0; k < 32; ++k)
                sum += E::to_f32((uint16_t)(raw[e][k / 2] >> (16 * (k & 1))));
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xl[m][q][u] = u32x4_t{p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]};
            sl[m][u] = sum;
        }
    }
    __syncthreads();
    static_assert(MT <= 4, "at most four activation rows' slices in registers");
    uint32_t xr[MT][UPL][16];
    float xs[MT][UPL];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
            const int u = kl + KL * j;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4_t v = xl[m][q][u];
                xr[m][j][4 * q] = v.x; xr[m][j][4 * q + 1] = v.y;
                xr[m][j][4 * q + 2] = v.z; xr[m][j][4 * q + 3] = v.w;
            }
            xs[m][j] = sl[m][u];
        }

    for (bool first = true; r0 < a.N; r0 += GW * S * D, first = false) {
        if (!first)
            load(r0);
        exchange();
        float acc[D * MT];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            float total[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m)
                total[m] = 0.0f;
#pragma unroll
            for (int j = 0; j < UPL; ++j) {
                const Orient o = orient<BITS>(E::to_f32(sv[d][j]), E::to_f32(bv[d][j]));
                uint32_t cp[16];
                code_pairs<BITS, DT>(w[d][j], o.flip, cp);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    float part = 0.0f;
#pragma unroll
                    for (int p = 0; p < 16; ++p)
                        part = PX::dot(cp[p], xr[m][j][p], part);
                    total[m] = __builtin_fmaf(o.s, part, __builtin_fmaf(o.b, xs[m][j], total[m]));
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
                acc[d * MT + m] = total[m];
        }
        reduce_slots<D * MT, KL>(acc);
        if (kl == KL - 1) {
#pragma unroll
            for (int d = 0; d < D; ++d)
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (r0 + slot * D + d < a.N && m < a.M)
                        y[(int64_t)m * a.N + r0 + slot * D + d] = E::from_f32(acc[d * MT + m]);
        }
    }
}

// Three or four activation rows on the matrix cores: the 4x4x4 instruction
// holds sixteen independent 4 x 4 blocks per wave, and here block b of a wave
// is unit 16 rho + b of the wave's four weight rows at round rho. Lane 4 b + c
// holds, for its block, activation row c (operand A, four activations of the
// unit) and weight row r0 + c (operand B, the same four positions as exact
// code pairs), and ends with the sums for weight row r0 + c over activation rows
// 0..3 (one per accumulator register). A unit takes eight instructions; its
// group's scale and bias are then applied per lane, and the sixteen blocks are
// summed at the end. Per code this is the same extraction work as one
// activation row on the dot-product path, while the products of all four
// activation rows go to the matrix cores.
template <int DT> struct RowMfma;
template <> struct RowMfma<DT_BF16> {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ f32x4_t mma(u32x2_t a, u32x2_t b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                      __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
    }
};
template <> struct RowMfma<DT_F16> {
    typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ f32x4_t mma(u32x2_t a, u32x2_t b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4_t, a),
                                                  __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
    }
};

template <int BITS, int DT, int R, bool WIDE>
__global__ __launch_bounds__(256) void qgemv_rowmfma_kernel(RowStreamArgs a)
{
    using E = Elem<DT>;
    using St = typename E::storage;
    static_assert(BITS == 2 || BITS == 4 || BITS == 8, "codes in whole 16-bit halves");
    using CO = CodeOrder<BITS>;
    constexpr int UNITS = 16 * R;                    // unit slots of a row
    constexpr int ENTRIES = 4 * UNITS;               // (activation row, unit) slices
    constexpr int EPT = (ENTRIES + 255) / 256;
    // Permuted activation pairs of slice (m, u), four 4-word vectors, and the
    // slice sums of unit u for the four activation rows.
    __shared__ u32x4_t xl[4][4][UNITS];
    __shared__ float sl[UNITS][4];
    constexpr int SBD = 2 * UNITS;                   // dwords of four rows' scales at most
    constexpr int NV = (SBD + 63) / 64;
    __shared__ uint32_t sbl[4][2][WIDE ? SBD : 1];

    const int lane = threadIdx.x & 63, blk = lane >> 2, col = lane & 3;
    const int wv = (int)(threadIdx.x >> 6);
    const int gw = (int)blockIdx.x * 4 + wv;
    const int GW = (int)gridDim.x * 4;
    const uint32_t row_bytes = (uint32_t)a.K * BITS / 8;
    const uint32_t groups_row = (uint32_t)(a.K / a.gs);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.wq, (uint32_t)a.N * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales, (uint32_t)a.N * groups_row * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.biases, (uint32_t)a.N * groups_row * 2);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)a.K * 2);
    St* y = static_cast<St*>(a.y);
    uint32_t gofs[R];                                // byte offset of unit 16 rho + blk's group
#pragma unroll
    for (int rho = 0; rho < R; ++rho)
        gofs[rho] = (uint32_t)((32 * (16 * rho + blk)) / a.gs) * 2;

    uint32_t raw[EPT][16];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int idx = (int)threadIdx.x + 256 * e, m = idx / UNITS, u = idx % UNITS;
        const bool live = idx < ENTRIES && m < a.M && u < (int)a.units_row;
        buffer_words<16>(rx, live ? ((uint32_t)m * (uint32_t)a.K + 32u * (uint32_t)u) * 2 : OOB,
                         raw[e]);
    }
    __builtin_amdgcn_sched_barrier(0);

    const uint32_t nd = 2 * groups_row;              // dwords of four rows' scales
    uint32_t sw[NV], bw[NV];
    uint32_t w[R][BITS];
    St sv[R], bv[R];
    auto load = [&](int r0) {
        if constexpr (WIDE) {
            const uint32_t base = (uint32_t)r0 * groups_row * 2;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const uint32_t i = (uint32_t)(lane + 64 * v);
                const uint32_t off = i < nd ? base + 4 * i : OOB;
                sw[v] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
                bw[v] = __builtin_amdgcn_raw_buffer_load_b32(rb, off, 0, 0);
            }
        }
#pragma unroll
        for (int rho = 0; rho < R; ++rho) {
            const int u = 16 * rho + blk, r = r0 + col;
            const bool live = u < (int)a.units_row && r < a.N;
            buffer_words<BITS, BITS == 8 ? 0 : kStreamPolicy>(
                rw, live ? (uint32_t)r * row_bytes + (uint32_t)u * (4 * BITS) : OOB, w[rho]);
            if constexpr (!WIDE) {
                const uint32_t so = live ? (uint32_t)r * groups_row * 2 + gofs[rho] : OOB;
                sv[rho] = buffer_elem<DT>(rs, so);
                bv[rho] = buffer_elem<DT>(rb, so);
            }
        }
    };
    auto exchange = [&]() {
        if constexpr (WIDE) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const uint32_t i = (uint32_t)(lane + 64 * v);
                if (i < nd) {
                    sbl[wv][0][i] = sw[v];
                    sbl[wv][1][i] = bw[v];
                }
            }
#pragma unroll
            for (int rho = 0; rho < R; ++rho) {
                const bool live = 16 * rho + blk < (int)a.units_row;
                // Element e = c * groups + g sits in half e % 2 of slot e / 2;
                // e / 2 < SBD for every lane.
                const uint32_t e = (uint32_t)col * groups_row + gofs[rho] / 2;
                const uint32_t ds = sbl[wv][0][e >> 1], db = sbl[wv][1][e >> 1];
                const uint32_t sh = 16 * (e & 1);
                sv[rho] = live ? St(ds >> sh) : St(0);
                bv[rho] = live ? St(db >> sh) : St(0);
            }
        }
    };
    int r0 = gw * 4;
    load(r0);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int idx = (int)threadIdx.x + 256 * e, m = idx / UNITS, u = idx % UNITS;
        if (idx < ENTRIES) {
            // Pair q holds the activations of codes lo_code(q) (low half) and
            // hi_code(q) (high half) of the unit.
            uint32_t p[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int k0 = CO::lo_code(q), k1 = CO::hi_code(q);
                const uint32_t lo = (raw[e][k0 / 2] >> (16 * (k0 & 1))) & 0xFFFFu;
                const uint32_t hi = (raw[e][k1 / 2] >> (16 * (k1 & 1))) & 0xFFFFu;
                p[q] = lo | (hi << 16);
            }
            float sum = 0.0f;
#pragma unroll
            for (int k = 0; k < 32; ++k)
                sum += E::to_f32((uint16_t)(raw[e][k / 2] >> (16 * (k & 1))));
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xl[m][q][u] = u32x4_t{p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]};
            sl[u][m] = sum;
        }
    }
    __syncthreads();

    for (bool first = true; r0 < a.N; r0 += GW * 4, first = false) {
        if (!first)
            load(r0);
        exchange();
        // Two rounds at a time, their instruction chains interleaved.
        constexpr int RP = R >= 2 ? 2 : 1;
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int r2 = 0; r2 < R; r2 += RP) {
            f32x4_t c[RP];
            Orient o[RP];
            uint32_t cp[RP][16];
#pragma unroll
            for (int h = 0; h < RP; ++h) {
                c[h] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                o[h] = orient<BITS>(E::to_f32(sv[r2 + h]), E::to_f32(bv[r2 + h]));
                code_pairs<BITS, DT>(w[r2 + h], o[h].flip, cp[h]);
            }
            auto code_pair = [&](int h, int p) -> uint32_t { return cp[h][p]; };
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4_t xv[RP];
#pragma unroll
                for (int h = 0; h < RP; ++h)
                    xv[h] = xl[col][q][16 * (r2 + h) + blk];
#pragma unroll
                for (int h = 0; h < RP; ++h)
                    c[h] = RowMfma<DT>::mma(u32x2_t{xv[h].x, xv[h].y},
                                            u32x2_t{code_pair(h, 4 * q), code_pair(h, 4 * q + 1)},
                                            c[h]);
#pragma unroll
                for (int h = 0; h < RP; ++h)
                    c[h] = RowMfma<DT>::mma(u32x2_t{xv[h].z, xv[h].w},
                                            u32x2_t{code_pair(h, 4 * q + 2), code_pair(h, 4 * q + 3)},
                                            c[h]);
            }
#pragma unroll
            for (int h = 0; h < RP; ++h) {
                const int u = 16 * (r2 + h) + blk;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float xs = sl[u][i];
                    acc[i] = __builtin_fmaf(o[h].s, c[h][i], __builtin_fmaf(o[h].b, xs, acc[i]));
                }
            }
            // Two rounds' activation vectors live at a time.
            __builtin_amdgcn_sched_barrier(0);
        }
        // Sum over the sixteen blocks: rotations by 4 and 8 within each row of
        // 16 lanes, then across the rows.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = acc[i];
            v += dpp_f32<0x124>(v);
            v += dpp_f32<0x128>(v);
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[i] = v;
        }
        if (lane < 4 && r0 + lane < a.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < a.M)
                    y[(int64_t)i * a.N + r0 + lane] = E::from_f32(acc[i]);
        }
    }
}

} // namespace qp
