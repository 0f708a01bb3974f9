// moe_rows.hpp — routed MoE tiles on the row kernels (ferrum-kernels
// src/stacked_expert.rs, `gemv_moe_id_batched` and `gemv_moe_id_gate_up_silu`:
// every pair of a tile shares its expert's weights, which are read once per
// tile): tiles of up to 8 pairs on the 4x4x4 matrix instruction, and tiles of
// one pair on the dot-product row kernel.
//
// The dense four-row kernel (rowstream.hpp, `qgemv_rowmfma_kernel`) applied to
// a routed tile: the tile's pair rows are gathered into the block's LDS as the
// same permuted activation slices, and each wave owns four rows of the
// expert's matrix (or of both matrices of the fused form). Block b of a wave
// is unit 16 rho + b at round rho; lane 4 b + c holds activation row c of each
// 4-row chunk (A) and weight row r0 + c (B, exact code pairs). Per unit the
// group's scale and bias are applied per lane; the sixteen blocks are summed at
// the end, and lanes 0..3 store their row for every pair of the tile, through
// SiLU(gate) * up in the fused form.
//
// A block of 4 waves covers 64 weight rows, each wave 4 row quads in turn, so
// that the gather (up to 8 activation rows of K elements from L2) is shared by
// 64 rows while several blocks still share a CU and hide each other's
// latency.
#pragma once

#include "gemv_core.hpp"
#include "rowstream.hpp"

namespace qp {

#ifndef QP_MOE_ROW_WAVES
#define QP_MOE_ROW_WAVES 4
#endif
#ifndef QP_MOE_ROW_QUADS
#define QP_MOE_ROW_QUADS 4
#endif
constexpr int kMoeRowWaves = QP_MOE_ROW_WAVES;
constexpr int kMoeRowQuads = QP_MOE_ROW_QUADS;       // row quads per wave and tile

template <int BITS, int DT, int R, int NMAT, int MC>
__global__ __launch_bounds__(64 * kMoeRowWaves) void qgemv_moe_rowmfma_kernel(GemvKernelArgs a)
{
    using E = Elem<DT>;
    using St = typename E::storage;
    static_assert(BITS == 2 || BITS == 4 || BITS == 8, "codes in whole 16-bit halves");
    using CO = CodeOrder<BITS>;
    constexpr int MT = 4 * MC;                       // pairs per tile at most
    constexpr int UNITS = 16 * R;                    // unit slots of a row
    constexpr int ENTRIES = MT * UNITS;              // (pair, unit) slices
    constexpr int THREADS = 64 * kMoeRowWaves;
    constexpr int EPT = (ENTRIES + THREADS - 1) / THREADS;
    constexpr int SB = (int)sizeof(St);
    __shared__ u32x4_t xl[MT][4][UNITS];
    __shared__ float sl[UNITS][MT];

    const int lane = threadIdx.x & 63, blk = lane >> 2, col = lane & 3;
    const int wv = (int)(threadIdx.x >> 6);
    const int Rr = (int)a.R;
    const uint32_t units_row = (uint32_t)(a.K / 32);
    const uint32_t row_bytes = (uint32_t)a.K * BITS / 8;
    const uint32_t groups_row = (uint32_t)(a.K / a.gs);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out, a.out_bytes);
    uint32_t gofs[R];
#pragma unroll
    for (int rho = 0; rho < R; ++rho)
        gofs[rho] = (uint32_t)((32 * (16 * rho + blk)) / a.gs) * SB;

    const int ntiles = gemv_num_tiles(a);
    for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
        int expert, start, count;
        if (!gemv_tile(a, tile, expert, start, count))
            continue;
        // Gather: raw activation units of the tile's pairs (zeros past the
        // tile or the row).
        uint32_t raw[EPT][16];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int idx = (int)threadIdx.x + THREADS * e, m = idx / UNITS, u = idx % UNITS;
            uint32_t off = OOB;
            if (idx < ENTRIES && m < count && u < (int)units_row) {
                const uint32_t p = a.perm != nullptr ? (uint32_t)a.perm[start + m]
                                                     : (uint32_t)(start + m);
                const uint32_t tk = (uint32_t)a.top_k;
                off = ((p / tk) * (uint32_t)a.outer + (p % tk) * (uint32_t)a.inner +
                       32u * (uint32_t)u) * (uint32_t)SB;
            }
            buffer_words<16>(rx, off, raw[e]);
        }
        __builtin_amdgcn_sched_barrier(0);

        // The codes and scales of the expert's rows r0 .. r0 + 3 of this
        // wave's quad j.
        const int64_t erow = (int64_t)expert * a.R;
        uint32_t w[NMAT][R][BITS];
        St sv[NMAT][R], bv[NMAT][R];
        auto load = [&](int r0) {
#pragma unroll
            for (int t = 0; t < NMAT; ++t) {
                const __amdgpu_buffer_rsrc_t rw =
                    make_rsrc(reinterpret_cast<const char*>(a.wq[t]) + erow * row_bytes,
                              (uint32_t)a.R * row_bytes);
                const __amdgpu_buffer_rsrc_t rs =
                    make_rsrc(static_cast<const char*>(a.scales[t]) + erow * groups_row * SB,
                              (uint32_t)a.R * groups_row * SB);
                const __amdgpu_buffer_rsrc_t rb =
                    make_rsrc(static_cast<const char*>(a.biases[t]) + erow * groups_row * SB,
                              (uint32_t)a.R * groups_row * SB);
#pragma unroll
                for (int rho = 0; rho < R; ++rho) {
                    const int u = 16 * rho + blk, r = r0 + col;
                    const bool live = u < (int)units_row && r < Rr;
                    buffer_words<BITS, BITS == 8 ? 0 : kStreamPolicy>(
                        rw, live ? (uint32_t)r * row_bytes + (uint32_t)u * (4 * BITS) : OOB,
                        w[t][rho]);
                    const uint32_t so = live ? (uint32_t)r * groups_row * SB + gofs[rho] : OOB;
                    sv[t][rho] = buffer_elem<DT>(rs, so);
                    bv[t][rho] = buffer_elem<DT>(rb, so);
                }
            }
        };
        auto quad_row = [&](int j) {
            return ((int)blockIdx.x * kMoeRowQuads * kMoeRowWaves + j * kMoeRowWaves + wv) * 4;
        };
        load(quad_row(0));
        __builtin_amdgcn_sched_barrier(0);

        // Permuted slices and their sums into LDS (pair q of a slice holds the
        // activations of codes lo_code(q) and hi_code(q) of the unit).
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int idx = (int)threadIdx.x + THREADS * e, m = idx / UNITS, u = idx % UNITS;
            if (idx < ENTRIES) {
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

        for (int j = 0; j < kMoeRowQuads; ++j) {
            const int r0 = quad_row(j);
            if (r0 >= Rr)
                break;
            if (j > 0)
                load(r0);
            f32x4_t acc[NMAT][MC];
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
#pragma unroll
                for (int ch = 0; ch < MC; ++ch)
                    acc[t][ch] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int rho = 0; rho < R; ++rho) {
                const int u = 16 * rho + blk;
                f32x4_t c[NMAT][MC];
                Orient o[NMAT];
                uint32_t cp[NMAT][16];
#pragma unroll
                for (int t = 0; t < NMAT; ++t) {
#pragma unroll
                    for (int ch = 0; ch < MC; ++ch)
                        c[t][ch] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                    o[t] = orient<BITS>(E::to_f32(sv[t][rho]), E::to_f32(bv[t][rho]));
                    code_pairs<BITS, DT>(w[t][rho], o[t].flip, cp[t]);
                }
                auto code_pair = [&](int t, int, int p) -> uint32_t { return cp[t][p]; };
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u32x4_t xv[MC];
#pragma unroll
                    for (int ch = 0; ch < MC; ++ch)
                        xv[ch] = xl[4 * ch + col][q][u];
#pragma unroll
                    for (int t = 0; t < NMAT; ++t) {
                        const u32x2_t b0{code_pair(t, rho, 4 * q), code_pair(t, rho, 4 * q + 1)};
                        const u32x2_t b1{code_pair(t, rho, 4 * q + 2), code_pair(t, rho, 4 * q + 3)};
#pragma unroll
                        for (int ch = 0; ch < MC; ++ch) {
                            c[t][ch] = RowMfma<DT>::mma(u32x2_t{xv[ch].x, xv[ch].y}, b0, c[t][ch]);
                            c[t][ch] = RowMfma<DT>::mma(u32x2_t{xv[ch].z, xv[ch].w}, b1, c[t][ch]);
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < NMAT; ++t) {
#pragma unroll
                    for (int ch = 0; ch < MC; ++ch)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float xs = sl[u][4 * ch + i];
                            acc[t][ch][i] = __builtin_fmaf(o[t].s, c[t][ch][i],
                                                           __builtin_fmaf(o[t].b, xs, acc[t][ch][i]));
                        }
                }
                // One round's activation vectors live at a time.
                __builtin_amdgcn_sched_barrier(0);
            }
            // Sum over the sixteen blocks, then lanes 0..3 store weight row
            // r0 + lane for every pair of the tile.
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
#pragma unroll
                for (int ch = 0; ch < MC; ++ch)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = acc[t][ch][i];
                        v += dpp_f32<0x124>(v);
                        v += dpp_f32<0x128>(v);
                        v += __shfl_xor(v, 16, 64);
                        v += __shfl_xor(v, 32, 64);
                        acc[t][ch][i] = v;
                    }
            const int row = r0 + lane;
            if (lane < 4 && row < Rr) {
#pragma unroll
                for (int ch = 0; ch < MC; ++ch)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 4 * ch + i;
                        if (m < count) {
                            float v = acc[0][ch][i];
                            if constexpr (NMAT == 2)
                                v = silu_f32(acc[0][ch][i]) * acc[1][ch][i];
                            const uint32_t p = a.perm != nullptr ? (uint32_t)a.perm[start + m]
                                                                 : (uint32_t)(start + m);
                            buffer_store_elem<DT>(E::from_f32(v), ro,
                                                  (p * (uint32_t)a.R + (uint32_t)row) * (uint32_t)SB);
                        }
                    }
            }
        }
        __syncthreads();   // the slices are rebuilt for the next tile
    }
}

// Routed tiles of one pair (few pairs per expert, tile t = pair t) on the
// dot-product row kernel (rowstream.hpp, `qgemv_rowstream_kernel`): the block
// gathers the pair's activation row into LDS as permuted slices with their
// sums; a wave is 64 / KL slots of KL lanes, each slot owns D rows of the
// expert's matrix (of both matrices in the fused form) with its lane l on units
// l, l + KL, ..., and the slot's last lane stores the reduced rows, through
// SiLU(gate) * up in the fused form. Rows of few units (the down projection's
// K = 768 is 24 units) take KL = 32, so that fewer lanes idle.
template <int BITS, int DT, int UPL, int NMAT, int KL>
__global__ __launch_bounds__(256) void qgemv_moe_rowstream_kernel(GemvKernelArgs a)
{
    using PX = RowStreamPair<DT>;
    using E = Elem<DT>;
    using St = typename E::storage;
    static_assert(BITS == 2 || BITS == 4 || BITS == 8, "codes in whole 16-bit halves");
    constexpr int D = rowstream_depth<BITS, UPL * NMAT>();
    using CO = CodeOrder<BITS>;
    static_assert(KL == 32 || KL == 64, "32 or 64 lanes per row");
    constexpr int S = 64 / KL;                       // row slots per wave
    constexpr int UNITS = KL * UPL;                  // unit slots of the pair's row
    constexpr int EPT = (UNITS + 255) / 256;
    constexpr int SB = (int)sizeof(St);
    __shared__ u32x4_t xl[4][UNITS];
    __shared__ float sl[UNITS];

    const int lane = threadIdx.x & 63;
    const int kl = lane % KL, slot = lane / KL;
    const int wv = (int)(threadIdx.x >> 6);
    const int r0 = (((int)blockIdx.x * 4 + wv) * S + slot) * D;   // first weight row of the slot
    const int Rr = (int)a.R;
    const uint32_t units_row = (uint32_t)(a.K / 32);
    const uint32_t row_bytes = (uint32_t)a.K * BITS / 8;
    const uint32_t groups_row = (uint32_t)(a.K / a.gs);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out, a.out_bytes);
    uint32_t gofs[UPL];
#pragma unroll
    for (int j = 0; j < UPL; ++j)
        gofs[j] = (uint32_t)((32 * (kl + KL * j)) / a.gs) * SB;

    const int ntiles = gemv_num_tiles(a);
    for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
        int expert, start, count;
        if (!gemv_tile(a, tile, expert, start, count))
            continue;
        const uint32_t p = a.perm != nullptr ? (uint32_t)a.perm[start] : (uint32_t)start;
        const uint32_t tk = (uint32_t)a.top_k;
        const uint32_t xrow = (p / tk) * (uint32_t)a.outer + (p % tk) * (uint32_t)a.inner;
        uint32_t raw[EPT][16];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int u = (int)threadIdx.x + 256 * e;
            const bool live = u < UNITS && u < (int)units_row;
            buffer_words<16>(rx, live ? (xrow + 32u * (uint32_t)u) * (uint32_t)SB : OOB, raw[e]);
        }
        __builtin_amdgcn_sched_barrier(0);

        const int64_t erow = (int64_t)expert * a.R;
        uint32_t w[NMAT][D][UPL][BITS];
        St sv[NMAT][D][UPL], bv[NMAT][D][UPL];
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            const __amdgpu_buffer_rsrc_t rw =
                make_rsrc(reinterpret_cast<const char*>(a.wq[t]) + erow * row_bytes,
                          (uint32_t)a.R * row_bytes);
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(static_cast<const char*>(a.scales[t]) + erow * groups_row * SB,
                          (uint32_t)a.R * groups_row * SB);
            const __amdgpu_buffer_rsrc_t rb =
                make_rsrc(static_cast<const char*>(a.biases[t]) + erow * groups_row * SB,
                          (uint32_t)a.R * groups_row * SB);
#pragma unroll
            for (int d = 0; d < D; ++d)
#pragma unroll
                for (int j = 0; j < UPL; ++j) {
                    const int u = kl + KL * j, r = r0 + d;
                    const bool live = u < (int)units_row && r < Rr;
                    buffer_words<BITS, BITS == 8 ? 0 : kStreamPolicy>(
                        rw, live ? (uint32_t)r * row_bytes + (uint32_t)u * (4 * BITS) : OOB,
                        w[t][d][j]);
                    const uint32_t so = live ? (uint32_t)r * groups_row * SB + gofs[j] : OOB;
                    sv[t][d][j] = buffer_elem<DT>(rs, so);
                    bv[t][d][j] = buffer_elem<DT>(rb, so);
                }
        }
        __builtin_amdgcn_sched_barrier(0);

#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int u = (int)threadIdx.x + 256 * e;
            if (u < UNITS) {
                uint32_t q4[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int k0 = CO::lo_code(q), k1 = CO::hi_code(q);
                    const uint32_t lo = (raw[e][k0 / 2] >> (16 * (k0 & 1))) & 0xFFFFu;
                    const uint32_t hi = (raw[e][k1 / 2] >> (16 * (k1 & 1))) & 0xFFFFu;
                    q4[q] = lo | (hi << 16);
                }
                float sum = 0.0f;
#pragma unroll
                for (int k = 0; k < 32; ++k)
                    sum += E::to_f32((uint16_t)(raw[e][k / 2] >> (16 * (k & 1))));
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xl[q][u] = u32x4_t{q4[4 * q], q4[4 * q + 1], q4[4 * q + 2], q4[4 * q + 3]};
                sl[u] = sum;
            }
        }
        __syncthreads();
        uint32_t xr[UPL][16];
        float xs[UPL];
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
            const int u = kl + KL * j;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4_t v = xl[q][u];
                xr[j][4 * q] = v.x; xr[j][4 * q + 1] = v.y;
                xr[j][4 * q + 2] = v.z; xr[j][4 * q + 3] = v.w;
            }
            xs[j] = sl[u];
        }

        float acc[NMAT * D];
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
            for (int d = 0; d < D; ++d) {
                float total = 0.0f;
#pragma unroll
                for (int j = 0; j < UPL; ++j) {
                    const Orient o = orient<BITS>(E::to_f32(sv[t][d][j]), E::to_f32(bv[t][d][j]));
                    uint32_t cp[16];
                    code_pairs<BITS, DT>(w[t][d][j], o.flip, cp);
                    float part = 0.0f;
#pragma unroll
                    for (int pp = 0; pp < 16; ++pp)
                        part = PX::dot(cp[pp], xr[j][pp], part);
                    total = __builtin_fmaf(o.s, part, __builtin_fmaf(o.b, xs[j], total));
                }
                acc[t * D + d] = total;
            }
        reduce_slots<NMAT * D, KL>(acc);
        if (kl == KL - 1) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                float v = acc[d];
                if constexpr (NMAT == 2)
                    v = silu_f32(acc[d]) * acc[D + d];
                if (r0 + d < Rr)
                    buffer_store_elem<DT>(E::from_f32(v), ro,
                                          (p * (uint32_t)a.R + (uint32_t)(r0 + d)) * (uint32_t)SB);
            }
        }
        __syncthreads();   // the slices are rebuilt for the next tile
    }
}

// The down projection of an MoE block fused with its close, for few tokens
// (each pair its own tile): output row r of token t is
//   out[t, r] = sum_j rw[t*top_k + j] * o_j[r],  o_j = h[t*top_k + j] . W[e_j][r]
// (the ferrum-kernels MoE dispatch docs leave this weighted sum of a token's
// slots to the FFN; router weights come from the caller). A slot of KL lanes
// owns one row r and, for each of the token's top_k <= KM slots, loads that
// expert's row r (one resource over the whole stack), forms o_j exactly as
// the one-pair kernel above does (same units per lane, same dot chain, same
// lane reduction), rounds it to the activation type as the stored o would be,
// and sums the slots in slot order in fp32: the result is that of the two
// separate launches, with one launch and no o round trip. The block gathers
// all the token's pair rows into LDS as permuted slices with their sums.
// Slots whose id is outside [0, E) read zeros and add nothing.
template <int BITS, int DT, int UPL, int KL, int KM>
__global__ __launch_bounds__(256) void qgemv_moe_rowcombine_kernel(GemvKernelArgs a, const float* __restrict__ rw,
                                                                  int64_t n_tokens)
{
    using PX = RowStreamPair<DT>;
    using E = Elem<DT>;
    using St = typename E::storage;
    static_assert(BITS == 2 || BITS == 4 || BITS == 8, "codes in whole 16-bit halves");
    using CO = CodeOrder<BITS>;
    static_assert(KL == 32 || KL == 64, "32 or 64 lanes per row");
    constexpr int S = 64 / KL;                       // row slots per wave
    constexpr int UNITS = KL * UPL;                  // unit slots of one pair's row
    constexpr int ENTRIES = KM * UNITS;              // (slot, unit) slices of a token
    constexpr int EPT = (ENTRIES + 255) / 256;
    constexpr int SB = (int)sizeof(St);
    __shared__ u32x4_t xl[KM][4][UNITS];
    __shared__ float sl[KM][UNITS];

    const int lane = threadIdx.x & 63;
    const int kl = lane % KL, slot = lane / KL;
    const int wv = (int)(threadIdx.x >> 6);
    const int r0 = ((int)blockIdx.x * 4 + wv) * S + slot;   // the slot's output row
    const int Rr = (int)a.R;
    const int k = (int)a.top_k;
    const uint32_t units_row = (uint32_t)(a.K / 32);
    const uint32_t row_bytes = (uint32_t)a.K * BITS / 8;
    const uint32_t groups_row = (uint32_t)(a.K / a.gs);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out, a.out_bytes);
    const __amdgpu_buffer_rsrc_t rwq = make_rsrc(a.wq[0], (uint32_t)(a.n_experts * a.R) * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales[0], (uint32_t)(a.n_experts * a.R) * groups_row * SB);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.biases[0], (uint32_t)(a.n_experts * a.R) * groups_row * SB);
    uint32_t gofs[UPL];
#pragma unroll
    for (int j = 0; j < UPL; ++j)
        gofs[j] = (uint32_t)((32 * (kl + KL * j)) / a.gs) * SB;

    for (int64_t t = blockIdx.y; t < n_tokens; t += gridDim.y) {
        // The token's experts (the same in every thread); -1 for an absent or
        // invalid slot.
        int ex[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            const int e = j < k ? a.ids[t * k + j] : -1;
            ex[j] = (e >= 0 && e < a.n_experts) ? e : -1;
        }
        uint32_t raw[EPT][16];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int idx = (int)threadIdx.x + 256 * e, j = idx / UNITS, u = idx % UNITS;
            uint32_t off = OOB;
            if (idx < ENTRIES && u < (int)units_row) {
                int ej = -1;
#pragma unroll
                for (int jj = 0; jj < KM; ++jj)
                    ej = jj == j ? ex[jj] : ej;
                if (ej >= 0) {
                    const uint32_t xrow = (uint32_t)t * (uint32_t)a.outer + (uint32_t)j * (uint32_t)a.inner;
                    off = (xrow + 32u * (uint32_t)u) * (uint32_t)SB;
                }
            }
            buffer_words<16>(rx, off, raw[e]);
        }
        __builtin_amdgcn_sched_barrier(0);

        uint32_t w[KM][UPL][BITS];
        St sv[KM][UPL], bv[KM][UPL];
#pragma unroll
        for (int j = 0; j < KM; ++j)
#pragma unroll
            for (int jj = 0; jj < UPL; ++jj) {
                const int u = kl + KL * jj;
                const bool live = ex[j] >= 0 && u < (int)units_row && r0 < Rr;
                const uint32_t row = (uint32_t)(ex[j] < 0 ? 0 : ex[j]) * (uint32_t)Rr + (uint32_t)r0;
                buffer_words<BITS, BITS == 8 ? 0 : kStreamPolicy>(
                    rwq, live ? row * row_bytes + (uint32_t)u * (4 * BITS) : OOB, w[j][jj]);
                const uint32_t so = live ? row * groups_row * SB + gofs[jj] : OOB;
                sv[j][jj] = buffer_elem<DT>(rs, so);
                bv[j][jj] = buffer_elem<DT>(rb, so);
            }
        __builtin_amdgcn_sched_barrier(0);

#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int idx = (int)threadIdx.x + 256 * e, j = idx / UNITS, u = idx % UNITS;
            if (idx < ENTRIES) {
                uint32_t q4[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int k0 = CO::lo_code(q), k1 = CO::hi_code(q);
                    const uint32_t lo = (raw[e][k0 / 2] >> (16 * (k0 & 1))) & 0xFFFFu;
                    const uint32_t hi = (raw[e][k1 / 2] >> (16 * (k1 & 1))) & 0xFFFFu;
                    q4[q] = lo | (hi << 16);
                }
                float sum = 0.0f;
#pragma unroll
                for (int c = 0; c < 32; ++c)
                    sum += E::to_f32((uint16_t)(raw[e][c / 2] >> (16 * (c & 1))));
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xl[j][q][u] = u32x4_t{q4[4 * q], q4[4 * q + 1], q4[4 * q + 2], q4[4 * q + 3]};
                sl[j][u] = sum;
            }
        }
        __syncthreads();

        float acc[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            float total = 0.0f;
#pragma unroll
            for (int jj = 0; jj < UPL; ++jj) {
                const int u = kl + KL * jj;
                const Orient o = orient<BITS>(E::to_f32(sv[j][jj]), E::to_f32(bv[j][jj]));
                uint32_t cp[16];
                code_pairs<BITS, DT>(w[j][jj], o.flip, cp);
                float part = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4_t v = xl[j][q][u];
                    part = PX::dot(cp[4 * q], v.x, part);
                    part = PX::dot(cp[4 * q + 1], v.y, part);
                    part = PX::dot(cp[4 * q + 2], v.z, part);
                    part = PX::dot(cp[4 * q + 3], v.w, part);
                }
                total = __builtin_fmaf(o.s, part, __builtin_fmaf(o.b, sl[j][u], total));
            }
            acc[j] = total;
        }
        reduce_slots<KM, KL>(acc);
        if (kl == KL - 1 && r0 < Rr) {
            float v = 0.0f;
#pragma unroll
            for (int j = 0; j < KM; ++j)
                if (ex[j] >= 0)
                    v = __builtin_fmaf(rw[t * k + j], E::to_f32(E::from_f32(acc[j])), v);
            buffer_store_elem<DT>(E::from_f32(v), ro, ((uint32_t)t * (uint32_t)Rr + (uint32_t)r0) * (uint32_t)SB);
        }
        __syncthreads();   // the slices are rebuilt for the next token
    }
}

} // namespace qp
