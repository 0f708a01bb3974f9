// mfma_gemv.hpp — skinny products on the matrix cores: a tile of up to 16 * NB
// activation rows against weight rows streamed from HBM.
//
// Same product as the streaming kernel (emily lib/emily/quantization.ex,
// `quantized_matmul/2`; the MoE form of ferrum-kernels src/stacked_expert.rs,
// `gemv_moe_id_batched` and `gemv_moe_id_gate_up_silu`), for tiles of several
// activation rows, where dot products per row would multiply the vector work
// by the tile height:
//  - each wave owns 16 weight rows at a time and keeps a ring of D quads of
//    codes in flight; for quad j, unit 4j + g (32 codes) of row r is loaded
//    by lane 4r + g, so that four neighbouring lanes read one row's 64
//    contiguous bytes (the memory pipeline only merges neighbouring lanes),
//    and one ds_bpermute per word moves it to lane r + 16 g, where the
//    matrix-core A operand wants row r's k-group g;
//  - the codes are dequantized in fp32 (q * s' + b', the oracle's order) and
//    rounded to the activation type, giving four 8-element A fragments; the
//    weights are therefore rounded once to bf16/fp16, like the prefill GEMM;
//  - v_mfma_f32_16x16x32 contracts them with B fragments from an LDS table of
//    the tile's activation rows (filled by LDS DMA), stored fragment-major: B lane (m, g) of
//    fragment i of quad j holds x[m][32 (4j + g) + 8 i .. + 7] (the k's of
//    the A lane (r, g) fragment i, so both sides agree on the k order), and
//    the 64 lanes of one fragment read one contiguous kilobyte;
//  - up to NB column blocks of 16 rows share each dequantized fragment;
//  - each wave stages the scales and biases of its 16 rows and K range in
//    LDS with coalesced loads before the loop (read back as one 32-bit pair
//    per quad); loading them per quad would touch 16 rows' cache lines per
//    instruction for a few bytes each;
//  - KS waves may split one row block's K range; their partial sums meet in
//    LDS before the epilogue.
// Table rows past the tile hold zeros; weight rows past the end read zeros
// (raw buffer loads) and their stores drop, so the loop has no row branches.
#pragma once

#include "gemv_core.hpp"

namespace qp {

template <int DT> struct Mfma16;
template <> struct Mfma16<DT_BF16> {
    using frag_t = bf16x8_t;
    static __device__ __forceinline__ f32x4_t mfma(frag_t a, frag_t b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi)
    {
        return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
    }
};
template <> struct Mfma16<DT_F16> {
    using frag_t = f16x8_t;
    static __device__ __forceinline__ f32x4_t mfma(frag_t a, frag_t b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi)
    {
        return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)lo, (_Float16)hi});
    }
};

// Register budget per lane for THREADS-thread blocks (one block per CU).
template <int THREADS> constexpr int mfma_vgpr_budget() { return THREADS > 512 ? 160 : 240; }

// Ring depth (quads of codes in flight per lane) that fits the register budget.
template <int BITS, int NB, int NMAT, int THREADS>
constexpr int mfma_ring_depth()
{
    constexpr int slot = NMAT * BITS;
    constexpr int fixed = 32 * NB + 4 * NB * NMAT + 26 * NMAT + 40;
    int d = (mfma_vgpr_budget<THREADS>() - fixed) / slot;
    return d > 8 ? 8 : (d < 2 ? 2 : d);
}

// LDS: the activation table of 16 * NB rows x kpad values (4 KB per column
// block and quad), then one region holding first the waves' staged scales and
// biases and, after the main loop, the K-split partial sums.
__host__ __device__ constexpr uint32_t mfma_table_bytes(int nb, int kpad)
{
    return (uint32_t)nb * (uint32_t)kpad * 32u;
}
// Partial sums of the K-split waves: per wave NB * NMAT 16x16 fp32 tiles.
__host__ __device__ constexpr uint32_t mfma_red_bytes(int threads, int nb, int nmat)
{
    return (uint32_t)(threads / 64) * nb * nmat * 64 * 16;
}
// Staged scale/bias pairs: per wave and matrix, 16 rows x (kpad / KS / gs) groups.
__host__ __device__ constexpr uint32_t mfma_sb_bytes(int threads, int nmat, int kpad, int ks, int gs)
{
    return (uint32_t)(threads / 64) * (uint32_t)nmat * 16u * (uint32_t)(kpad / ks / gs) * 4u;
}
__host__ __device__ constexpr uint32_t mfma_lds_bytes(int threads, int nb, int nmat, int kpad, int ks,
                                                      int gs)
{
    const uint32_t red = ks > 1 ? mfma_red_bytes(threads, nb, nmat) : 0u;
    const uint32_t sb = mfma_sb_bytes(threads, nmat, kpad, ks, gs);
    return mfma_table_bytes(nb, kpad) + (red > sb ? red : sb);
}

// kpad: K rounded up to 128 * KS (whole quads per K-split wave).
// n_rg: row groups of 16 * (THREADS / 64 / KS) rows per expert (or matrix);
// the grid's x dimension must be n_rg (block x takes row group x).
template <int BITS, int DT, int NB, int NMAT, int THREADS>
__global__ __launch_bounds__(THREADS) void qgemv_mfma_kernel(GemvKernelArgs a, int kpad, int KS,
                                                            int n_rg)
{
    using M16 = Mfma16<DT>;
    using frag_t = typename M16::frag_t;
    using St = typename Elem<DT>::storage;
    using CB = CodeBytes<BITS>;
    constexpr int WAVES = THREADS / 64;
    constexpr int D = mfma_ring_depth<BITS, NB, NMAT, THREADS>();
    constexpr int NW = BITS;                 // words per unit
    constexpr int SB = (int)sizeof(St);
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char* const table = lds;
    char* const red = lds + mfma_table_bytes(NB, kpad);     // after the main loop

    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int RB = WAVES / KS;
    const int rb = wave / KS, ks = wave % KS;
    const int NQ = kpad / 128;               // quads per row
    const int UQ = NQ / KS;                  // quads per wave
    const int R = (int)a.R;
    const uint32_t row_bytes = (uint32_t)(a.K * BITS / 8);
    const uint32_t groups_row = (uint32_t)(a.K / a.gs);
    const uint32_t gshift = (uint32_t)(__builtin_ctz((unsigned)a.gs) - 5); // log2 units per group
    const int units = (int)(a.K / 32);
    const int NGW = kpad / KS / a.gs;        // groups per wave's K range
    char* const sbw = red + (uint32_t)wave * (uint32_t)(NMAT * 16 * NGW * 4); // this wave's pairs
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out, a.out_bytes);

    const int ntiles = gemv_num_tiles(a);
    for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
        int expert, start, count;
        if (!gemv_tile(a, tile, expert, start, count))
            continue;   // uniform over the block
        const int rows = count < 16 * NB ? count : 16 * NB;
        __amdgpu_buffer_rsrc_t rw[NMAT], rs[NMAT], rbias[NMAT];
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            const uint64_t erow = (uint64_t)expert * (uint64_t)R;
            rw[t] = make_rsrc(reinterpret_cast<const char*>(a.wq[t]) + erow * row_bytes,
                              (uint32_t)R * row_bytes);
            rs[t] = make_rsrc(static_cast<const char*>(a.scales[t]) + erow * groups_row * SB,
                              (uint32_t)R * groups_row * SB);
            rbias[t] = make_rsrc(static_cast<const char*>(a.biases[t]) + erow * groups_row * SB,
                                 (uint32_t)R * groups_row * SB);
        }

        // Weight ring of this lane: quad j -> unit 4 (ks * UQ + j) + (lane % 4)
        // of row n0 + lane / 4 (per matrix, the unit's words).
        uint32_t w[D][NMAT][NW];
        const int rg = (int)blockIdx.x;   // one row group per block (gridDim.x == n_rg)
        const int n0 = (rg * RB + rb) * 16;
        const int lrow = lane >> 2, lg = lane & 3;
        const uint32_t row_off =
            (rg < n_rg && n0 + lrow < R) ? (uint32_t)(n0 + lrow) * row_bytes : OOB;
        const int bp_addr = (4 * r16 + g4) * 4;   // ds_bpermute source: lane 4 r + g
        auto fetch = [&](int j, uint32_t (&dw)[NMAT][NW]) {
            const uint32_t u = (uint32_t)(4 * (ks * UQ + j) + lg);
            const uint32_t woff = row_off + u * (uint32_t)(4 * NW);
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
                buffer_words<NW>(rw[t], woff, dw[t]);
        };
        static_for<D>([&](auto J) { fetch(J < UQ ? (int)J : UQ - 1, w[J]); });

        // Scale/bias pairs of the wave's 16 rows and NGW groups: entry
        // (t, gi, r) = s | b << 16 at sbw + ((t * NGW + gi) * 16 + r) * 4.
        // Consecutive lanes read consecutive groups of a row; rows past the
        // end read zeros.
        {
            const int total = 16 * NGW;
            for (int e0 = lane; e0 < total; e0 += 4 * 64) {
                St sv[4][NMAT], bv[4][NMAT];
                static_for<4>([&](auto I) {
                    const int e = e0 + (int)I * 64;
                    const int r = e / NGW, gi = e % NGW;
                    const uint32_t off = (e < total && n0 + r < R)
                        ? ((uint32_t)(n0 + r) * groups_row + (uint32_t)(ks * NGW + gi)) * SB : OOB;
#pragma unroll
                    for (int t = 0; t < NMAT; ++t) {
                        sv[I][t] = buffer_elem<DT>(rs[t], off);
                        bv[I][t] = buffer_elem<DT>(rbias[t], off);
                    }
                });
                static_for<4>([&](auto I) {
                    const int e = e0 + (int)I * 64;
                    const int r = e / NGW, gi = e % NGW;
                    if (e < total) {
#pragma unroll
                        for (int t = 0; t < NMAT; ++t)
                            *reinterpret_cast<uint32_t*>(sbw + ((uint32_t)(t * NGW + gi) * 16u + (uint32_t)r) * 4u) =
                                (uint32_t)sv[I][t] | ((uint32_t)bv[I][t] << 16);
                    }
                });
            }
        }

        // Activation table (overlaps the first ring loads), filled by LDS DMA:
        // the 1 KB fragment block (nb, q, i) is one DMA instruction whose lane
        // (m, g) brings x[row 16 nb + m][32 (4 q + g) + 8 i .. + 7]. Rows past
        // the tile and units past K read zeros (offsets past the end). Each
        // lane resolves its rows' activation offsets once.
        {
            const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
            uint32_t xb[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = nb * 16 + r16;
                xb[nb] = OOB;
                if (row < rows) {
                    const uint32_t p = a.perm != nullptr ? (uint32_t)a.perm[start + row]
                                                         : (uint32_t)(start + row);
                    const uint32_t tk = (uint32_t)a.top_k;
                    xb[nb] = ((p / tk) * (uint32_t)a.outer + (p % tk) * (uint32_t)a.inner) * SB;
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                for (int q = wave; q < NQ; q += WAVES) {
                    const int unit = 4 * q + g4;
                    const uint32_t src = (xb[nb] != OOB && unit < units)
                        ? xb[nb] + (uint32_t)unit * 32u * SB : OOB;
                    char* dst = table + ((uint32_t)nb * (uint32_t)NQ + (uint32_t)q) * 4096u;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rx, (__attribute__((address_space(3))) void*)(dst + i * 1024),
                            16, src == OOB ? OOB : src + (uint32_t)(i * 8 * SB), 0, 0, 0);
                }
            }
        }
        // All of this lane's loads and DMA have landed: the table DMA was
        // issued after the ring's loads, so this costs no ring overlap, and no
        // load is left pending into the main loop (where it would make every
        // later write of a reused register wait for all memory traffic).
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        {
            f32x4_t acc[NMAT][NB];
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[t][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

            // B fragments of quad j for every column block, and this lane's
            // scale/bias pair of quad j for every matrix.
            struct Bq {
                frag_t f[NB][4];
                uint32_t sb[NMAT];
                uint32_t w[NMAT][NW];   // the quad's codes in operand order
            };
            const char* const bl = table + lane * 16;
            auto load_b = [&](int j, const uint32_t (&dw)[NMAT][NW], Bq& bq) {
#pragma unroll
                for (int t = 0; t < NMAT; ++t)
#pragma unroll
                    for (int i = 0; i < NW; ++i)
                        bq.w[t][i] = (uint32_t)__builtin_amdgcn_ds_bpermute(bp_addr, (int)dw[t][i]);
                const uint32_t q = (uint32_t)(ks * UQ + j);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        bq.f[nb][i] = *reinterpret_cast<const frag_t*>(
                            bl + ((uint32_t)nb * (uint32_t)NQ + q) * 4096u + (uint32_t)i * 1024u);
                const uint32_t gi = (uint32_t)(4 * j + g4) >> gshift;
#pragma unroll
                for (int t = 0; t < NMAT; ++t)
                    bq.sb[t] = *reinterpret_cast<const uint32_t*>(
                        sbw + (((uint32_t)t * (uint32_t)NGW + gi) * 16u + (uint32_t)r16) * 4u);
            };
            auto compute = [&](const Bq& bq) {
                const auto& bf = bq.f;
                const auto& dw = bq.w;
#pragma unroll
                for (int t = 0; t < NMAT; ++t) {
                    const float s = Elem<DT>::to_f32((St)(bq.sb[t] & 0xFFFFu));
                    const float b = Elem<DT>::to_f32((St)(bq.sb[t] >> 16));
                    uint32_t bw[CB::NBW];
                    CB::split(dw[t], bw);
                    static_for<4>([&](auto I) {
                        constexpr int i = decltype(I)::value;
                        uint32_t pk[4];
                        static_for<4>([&](auto P) {
                            constexpr int c = 8 * i + 2 * decltype(P)::value;
                            const float w0 = __builtin_fmaf(CB::template code<c>(bw), s, b);
                            const float w1 = __builtin_fmaf(CB::template code<c + 1>(bw), s, b);
                            pk[decltype(P)::value] = M16::pack2(w0, w1);
                        });
                        const frag_t af = __builtin_bit_cast(frag_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[t][nb] = M16::mfma(af, bf[nb][i], acc[t][nb]);
                    });
                }
            };

            // Full rounds of the ring; a refill past the wave's quads reloads
            // its last quad (in range, never used). The next quad's B
            // fragments are read from LDS while the current one computes.
            // Quad j + 1's operands (codes moved to operand order, B
            // fragments, scale/bias pairs) are prepared while quad j
            // computes; slot jj + 1 of the ring holds quad j + 1 (slot 0 of a
            // round was refilled with it during the previous slots).
            Bq bcur;
            load_b(0, w[0], bcur);
            int j0 = 0;
            for (; j0 + D <= UQ; j0 += D) {
                static_for<D>([&](auto J) {
                    constexpr int jj = decltype(J)::value;
                    const int j = j0 + jj;
                    Bq bnext;
                    load_b(j + 1 < UQ ? j + 1 : UQ - 1, w[(jj + 1) % D], bnext);
                    compute(bcur);
                    const int nj = j + D;
                    fetch(nj < UQ ? nj : UQ - 1, w[jj]);
                    bcur = bnext;
                });
            }
            // Remainder (UQ % D quads, in slots 0..rem-1; bcur holds slot 0's).
            const int rem = UQ - j0;
            static_for<D>([&](auto J) {
                constexpr int jj = decltype(J)::value;
                if (jj < rem) {
                    if constexpr (jj > 0)
                        load_b(j0 + jj, w[jj], bcur);
                    compute(bcur);
                }
            });

            // K-split partial sums meet in LDS (in the region that held the
            // staged scales, once every wave is past its main loop).
            if (KS > 1) {
                __syncthreads();
                if (ks != 0) {
#pragma unroll
                    for (int t = 0; t < NMAT; ++t)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            *reinterpret_cast<f32x4_t*>(
                                red + ((uint32_t)((wave * NMAT + t) * NB + nb) * 64 + lane) * 16) =
                                acc[t][nb];
                }
                __syncthreads();
                if (ks == 0) {
                    for (int k2 = 1; k2 < KS; ++k2) {
#pragma unroll
                        for (int t = 0; t < NMAT; ++t)
#pragma unroll
                            for (int nb = 0; nb < NB; ++nb)
                                acc[t][nb] += *reinterpret_cast<const f32x4_t*>(
                                    red + ((uint32_t)(((wave + k2) * NMAT + t) * NB + nb) * 64 + lane) * 16);
                    }
                }
                __syncthreads();
            }

            // Epilogue: lane l, register i holds weight row 4 (l / 16) + i of
            // the wave's 16, activation row l % 16 of the column block.
            if (ks == 0) {
                const int nbase = n0 + 4 * g4;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int m = nb * 16 + r16;
                    int64_t p = -1;
                    if (m < rows)
                        p = a.perm != nullptr ? (int64_t)a.perm[start + m] : (int64_t)(start + m);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = acc[0][nb][i];
                        if constexpr (NMAT == 2)
                            v = silu_f32(v) * acc[1][nb][i];
                        const int n = nbase + i;
                        const uint32_t off = (p >= 0 && n < R)
                            ? ((uint32_t)p * (uint32_t)R + (uint32_t)n) * (uint32_t)SB : OOB;
                        buffer_store_elem<DT>(Elem<DT>::from_f32(v), ro, off);
                    }
                }
            }
        }
        // Every wave is done with the table before the next tile refills it.
        __syncthreads();
    }
}

} // namespace qp
