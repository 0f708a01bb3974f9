// skinny4.hpp — skinny products (M = 3..16 activation rows) of 6-, 4-, 3-
// and 2-bit codes on the 16x16x32 matrix instruction, with row-contiguous code loads
// (emily lib/emily/quantization.ex, `quantized_matmul/2`; affine codes of
// `dequantize_defn/1`):
//   y[m, n] = sum_g s'[n,g] * sum_{k in g} x q + b'[n,g] * sum_{k in g} x.
//
// The layout of the matrix instruction (lane l = 16 kg + i): A is activation
// row i at k-slice kg (8 values), B is weight row n = i at k-slice kg, and
// the result holds activation rows 4 kg .. 4 kg + 3 of weight row n = i. So a
// lane works on one weight row throughout, and the scale, bias and
// orientation it applies are that row's own.
//
// A wave owns a K-slice of 16 units and up to four row groups of 16 weight
// rows. A row group's codes (16 rows x 16 units x 24, 16, 12 or 8 bytes)
// arrive as four loads per lane, each covering four rows with 384 (256, 192,
// 128) contiguous bytes of each (16 lanes per row); the wave writes them to its
// own LDS, [row][dword of the unit][unit], and every lane reads back its
// row's dwords holding k-slice kg of each unit (at 2 bits a dword holds two
// k-slices, 16 bits each; at 3 bits a 24-bit slice is aligned out of the two
// dwords it spans, at 6 bits a 48-bit one is two 24-bit halves of the two
// dwords it spans): the eight codes of one instruction per unit. A
// row group's scales and biases over the slice are one or two 16-byte loads
// per lane (its row's groups). Two row groups are in flight while one is
// computed. The activations of the slice are staged through the same LDS
// first (as in skinny.hpp), and the row groups' sums meet across the K-slice
// waves at the end.
#pragma once

#include "skinny.hpp"

namespace qp {

// Dwords per weight row in LDS: the slice's 16 units (BITS dwords each) plus
// 4 against bank conflicts; bytes of one row group's codes.
template <int BITS> __host__ __device__ constexpr uint32_t sk4_code_row() { return 16u * BITS + 4u; }
template <int BITS> __host__ __device__ constexpr uint32_t sk4_code_buf() { return 16u * sk4_code_row<BITS>() * 4u; }
__host__ __device__ constexpr uint32_t skinny4_wave_lds()
{
    // Activation staging (later two code buffers, then the partial sums),
    // then the group sums of the slice's activations.
    return 16u * kSkinnyXRow + 1024u;
}
static_assert(2 * sk4_code_buf<6>() <= 16 * kSkinnyXRow && (uint32_t)kSkinnyRG * 1024u <= 16 * kSkinnyXRow,
              "code buffers and partial sums within the staging region");

template <int BITS, int DT, int GU>
__global__ __launch_bounds__(64 * kSkinnyMaxWaves) void qgemv_skinny4_kernel(GemvKernelArgs a, SkinnyShape sh)
{
    static_assert(BITS == 2 || BITS == 3 || BITS == 4 || BITS == 6, "2-, 3-, 4- and 6-bit codes");
    // A lane's piece of a row per row quad: one unit, 24 bytes (6-bit), 16
    // (4-bit), 12 (3-bit) or 8 (2-bit). A dword holds one k-slice at 4 bits
    // and two (16 bits each) at 2; at 3 and 6 bits the 24- and 48-bit slices
    // straddle the unit's dwords.
    constexpr int PW = BITS;                        // dwords per unit
    constexpr uint32_t CR = sk4_code_row<BITS>();
    using M16 = SkMfma<DT>;
    using frag_t = typename M16::frag_t;
    using E = Elem<DT>;
    using St = typename E::storage;
    using C = ExactCvt<DT>;
    constexpr int NGS = kSkinnyKW / GU;            // groups per slice
    constexpr int SBW = NGS / 2;                   // dwords of a row's scales over the slice
    constexpr int SB = (int)sizeof(St);
    static_assert(SB == 2, "16-bit activations, scales and biases");
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nwaves = (int)(blockDim.x >> 6);
    const int ksi = wave / sh.wr, wri = wave % sh.wr;
    const int g = lane >> 4, l16 = lane & 15;
    const int R = (int)a.R;
    const int K = (int)a.K;
    const uint32_t row_bytes = (uint32_t)K * BITS / 8;
    const uint32_t G = (uint32_t)(K / a.gs);
    constexpr uint32_t WL = skinny4_wave_lds();
    char* const xst = lds + (uint32_t)wave * WL;            // staging; code buffers; partial sums
    char* const xsw = xst + 16u * kSkinnyXRow;               // [group][row] fp32
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out, a.out_bytes);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);

    const int rows = a.M < 16 ? a.M : 16;
    const int r_lo = (int)blockIdx.x * sh.rows_per_block;
    const int r_hi = (r_lo + sh.rows_per_block) < R ? (r_lo + sh.rows_per_block) : R;
    const int nrg_b = r_hi > r_lo ? (r_hi - r_lo + 15) / 16 : 0;
    const int nrg_w = wri < nrg_b ? (nrg_b - wri + sh.wr - 1) / sh.wr : 0;
    const uint32_t nrows = (uint32_t)(r_hi - r_lo);
    // Resources over the block's rows: rows past them read zeros.
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(reinterpret_cast<const char*>(a.wq[0]) + (uint64_t)r_lo * row_bytes,
                                                nrows * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<const char*>(a.scales[0]) + (uint64_t)r_lo * G * SB,
                                                nrows * G * SB);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(static_cast<const char*>(a.biases[0]) + (uint64_t)r_lo * G * SB,
                                                nrows * G * SB);
    // Activation row l16 (OOB past the rows of this launch).
    const uint32_t xoff = l16 < rows ? (uint32_t)l16 * (uint32_t)a.outer * SB : OOB;

    // Partial sums of the wave's row groups, kept over its K-slices.
    f32x4_t acc[kSkinnyRG];
#pragma unroll
    for (int r = 0; r < kSkinnyRG; ++r)
        acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int si = 0; si * sh.ks + ksi < sh.slices; ++si) {
        const int u0 = (si * sh.ks + ksi) * kSkinnyKW;   // first unit of the slice

        // Activations: the 16 rows' 1 KB of the slice, one load per row.
        u32x4_t raw[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t xr = (uint32_t)__builtin_amdgcn_readlane((int)xoff, r);
            const uint32_t off = (xr != OOB && u0 * 32 + 8 * lane < K) ? xr + (uint32_t)(u0 * 32 + 8 * lane) * 2u : OOB;
            raw[r] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
        }
        __builtin_amdgcn_sched_barrier(0);

        // The ring: row group rgi (rows 16 (wri + wr rgi) .. + 15 of the block).
        // Load q of lane l: row 4 q + l / 16 of the group, unit l % 16 of the
        // slice (4 BITS bytes); the row's scale and bias dwords over the slice.
        struct Slot {
            uint32_t c[4][PW];
            uint32_t s[SBW], b[SBW];
        };
        auto fetch = [&](int rgi, Slot& sl) {
            const uint32_t rg0 = 16u * (uint32_t)(wri + sh.wr * rgi);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t row = rg0 + 4u * (uint32_t)q + (uint32_t)g;
                const uint32_t off = row * row_bytes + ((uint32_t)u0 + (uint32_t)l16) * (4u * PW);
                if constexpr (PW == 6) {
                    const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
                    const u32x2_t t = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, off + 16u, 0, 0));
                    sl.c[q][0] = v.x; sl.c[q][1] = v.y; sl.c[q][2] = v.z; sl.c[q][3] = v.w;
                    sl.c[q][4] = t.x; sl.c[q][5] = t.y;
                } else if constexpr (PW == 4) {
                    const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
                    sl.c[q][0] = v.x; sl.c[q][1] = v.y; sl.c[q][2] = v.z; sl.c[q][3] = v.w;
                } else if constexpr (PW == 3) {
                    const auto v = __builtin_amdgcn_raw_buffer_load_b96(rw, off, 0, 0);
                    sl.c[q][0] = v[0]; sl.c[q][1] = v[1]; sl.c[q][2] = v[2];
                } else {
                    const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, off, 0, 0));
                    sl.c[q][0] = v.x; sl.c[q][1] = v.y;
                }
            }
            const uint32_t soff = ((rg0 + (uint32_t)l16) * G + (uint32_t)(u0 / GU)) * SB;
            if constexpr (SBW == 8) {
                const u32x4_t s0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, soff, 0, 0));
                const u32x4_t s1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, soff + 16, 0, 0));
                const u32x4_t b0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, soff, 0, 0));
                const u32x4_t b1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, soff + 16, 0, 0));
                sl.s[0] = s0.x; sl.s[1] = s0.y; sl.s[2] = s0.z; sl.s[3] = s0.w;
                sl.s[4] = s1.x; sl.s[5] = s1.y; sl.s[6] = s1.z; sl.s[7] = s1.w;
                sl.b[0] = b0.x; sl.b[1] = b0.y; sl.b[2] = b0.z; sl.b[3] = b0.w;
                sl.b[4] = b1.x; sl.b[5] = b1.y; sl.b[6] = b1.z; sl.b[7] = b1.w;
            } else if constexpr (SBW == 4) {
                const u32x4_t s0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, soff, 0, 0));
                const u32x4_t b0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, soff, 0, 0));
                sl.s[0] = s0.x; sl.s[1] = s0.y; sl.s[2] = s0.z; sl.s[3] = s0.w;
                sl.b[0] = b0.x; sl.b[1] = b0.y; sl.b[2] = b0.z; sl.b[3] = b0.w;
            } else {
                const u32x2_t s0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, soff, 0, 0));
                const u32x2_t b0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rb, soff, 0, 0));
                sl.s[0] = s0.x; sl.s[1] = s0.y;
                sl.b[0] = b0.x; sl.b[1] = b0.y;
            }
        };
        Slot ring[2];
        fetch(0, ring[0]);
        __builtin_amdgcn_sched_barrier(0);
        fetch(1, ring[1]);
        __builtin_amdgcn_sched_barrier(0);

        // Activation fragments (unit u: row l16, k-slice g), in the codes'
        // pair order, and the slice's group sums to xsw[group][row].
#pragma unroll
        for (int r = 0; r < 16; ++r)
            *reinterpret_cast<u32x4_t*>(xst + (uint32_t)r * kSkinnyXRow + 16u * (uint32_t)lane) = raw[r];
        frag_t xa[kSkinnyKW];
#pragma unroll
        for (int u = 0; u < kSkinnyKW; ++u) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xst + (uint32_t)l16 * kSkinnyXRow +
                                                                 (uint32_t)(u * 32 + 8 * g) * 2u);
            if constexpr (BITS == 6)   // byte codes keep the natural order
                xa[u] = __builtin_bit_cast(frag_t, v);
            else                       // the pair order 0, 2, 4, 6, 1, 3, 5, 7
                xa[u] = __builtin_bit_cast(frag_t, u32x4_t{__builtin_amdgcn_perm(v.y, v.x, 0x05040100u),
                                                           __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                                                           __builtin_amdgcn_perm(v.y, v.x, 0x07060302u),
                                                           __builtin_amdgcn_perm(v.w, v.z, 0x07060302u)});
        }
        static_for<NGS>([&](auto GI) {
            constexpr int gi = decltype(GI)::value;
            float p = 0.f;
#pragma unroll
            for (int u = gi * GU; u < gi * GU + GU; ++u) {
                const u32x4_t v = __builtin_bit_cast(u32x4_t, xa[u]);
                p = M16::pair_sum(v.x, p);
                p = M16::pair_sum(v.y, p);
                p = M16::pair_sum(v.z, p);
                p = M16::pair_sum(v.w, p);
            }
            p = rows_sum(p);
            if (g == 0)
                reinterpret_cast<float*>(xsw)[gi * 16 + l16] = p;
        });

        static_for<kSkinnyRG>([&](auto RGI) {
            constexpr int rgi = decltype(RGI)::value;
            Slot& sl = ring[rgi % 2];
            char* const cb = xst + (uint32_t)(rgi % 2) * sk4_code_buf<BITS>();   // the staging is done with
            __builtin_amdgcn_sched_barrier(0);
            // Codes to LDS as [row][dword of the unit][unit], then this
            // lane's row (l16) at its k-slice g: 16 consecutive dwords, one
            // per unit (dword g at 4 bits; dword g / 2 at 2 bits, whose half
            // g % 2 is the slice).
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t row = 4u * (uint32_t)q + (uint32_t)g;
                uint32_t* const d = reinterpret_cast<uint32_t*>(cb) + row * CR + (uint32_t)l16;
#pragma unroll
                for (int j = 0; j < PW; ++j)
                    d[16 * j] = sl.c[q][j];
            }
            // At 3 bits, slice g starts at bit 24 g: dword 3g / 4, byte 3g % 4,
            // and runs into the next dword (the last slice ends its dword).
            // At 6 bits, slice g starts at bit 48 g: dword 3g / 2, at its bit 0
            // (g even) or 16 (g odd), and ends in the next dword.
            const uint32_t gd = BITS == 4   ? (uint32_t)g
                                : BITS == 2 ? (uint32_t)g >> 1
                                : BITS == 3 ? (3u * (uint32_t)g) >> 2
                                            : (3u * (uint32_t)g) >> 1;
            auto read16 = [&](uint32_t j, uint32_t (&v16)[kSkinnyKW]) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
                        cb + ((uint32_t)l16 * CR + 16u * j + 4u * (uint32_t)i) * 4u);
                    v16[4 * i] = v.x; v16[4 * i + 1] = v.y; v16[4 * i + 2] = v.z; v16[4 * i + 3] = v.w;
                }
            };
            uint32_t dw[kSkinnyKW];
            read16(gd, dw);
            uint32_t dx[BITS == 6 ? kSkinnyKW : 1];   // 6-bit: codes 4..7 of the slice
            if constexpr (BITS == 6) {
                uint32_t nx[kSkinnyKW];
                read16(gd + 1u, nx);
                const bool odd = (g & 1) != 0;
#pragma unroll
                for (int u = 0; u < kSkinnyKW; ++u) {
                    const uint32_t a0 = __builtin_amdgcn_alignbyte(nx[u], dw[u], odd ? 2u : 0u);
                    dx[u] = odd ? nx[u] >> 8 : __builtin_amdgcn_alignbyte(nx[u], dw[u], 3u);
                    dw[u] = a0;   // codes 0..3 of the slice in the low 24 bits
                }
            }
            if constexpr (BITS == 3) {
                uint32_t nx[kSkinnyKW];
                read16(gd < 2u ? gd + 1u : 2u, nx);
                const uint32_t sh = (3u * (uint32_t)g) & 3u;
#pragma unroll
                for (int u = 0; u < kSkinnyKW; ++u)
                    dw[u] = __builtin_amdgcn_alignbyte(nx[u], dw[u], sh);   // slice g in the low 24 bits
            }
            uint32_t sv[SBW], bv[SBW];
#pragma unroll
            for (int i = 0; i < SBW; ++i) {
                sv[i] = sl.s[i];
                bv[i] = sl.b[i];
            }
            // The slot is free: the row group after next.
            if constexpr (rgi + 2 < kSkinnyRG)
                fetch(rgi + 2, sl);
            __builtin_amdgcn_sched_barrier(0);
            if (rgi < nrg_w) {
                static_for<NGS>([&](auto GI) {
                    constexpr int gi = decltype(GI)::value;
                    const uint32_t sw = sv[gi / 2], bw = bv[gi / 2];
                    const Orient o = orient<BITS>(E::to_f32((St)(sw >> (16 * (gi % 2)))),
                                                  E::to_f32((St)(bw >> (16 * (gi % 2)))));
                    f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int u = gi * GU; u < gi * GU + GU; ++u) {
                        u32x4_t bfr;
                        if constexpr (BITS == 4) {
                            const uint32_t lo = (dw[u] ^ o.flip) & 0x0F0F0F0Fu;
                            const uint32_t hi = ((dw[u] >> 4) ^ o.flip) & 0x0F0F0F0Fu;
                            bfr = u32x4_t{C::template fp8<false>(lo), C::template fp8<true>(lo),
                                          C::template fp8<false>(hi), C::template fp8<true>(hi)};
                        } else if constexpr (BITS == 6) {
                            // Codes 0..3 and 4..7 of the slice to bytes, complemented
                            // by the flip; byte pairs in the natural order.
                            const uint32_t c03 = code_bytes6(dw[u], o.flip), c47 = code_bytes6(dx[u], o.flip);
                            bfr = u32x4_t{C::template bytes<false>(c03), C::template bytes<true>(c03),
                                          C::template bytes<false>(c47), C::template bytes<true>(c47)};
                        } else if constexpr (BITS == 3) {
                            // The slice's 24 bits to bytes (even and odd codes),
                            // complemented by the flip: the 4-bit pair order.
                            uint32_t even, odd;
                            code_bytes3(dw[u], o.flip, even, odd);
                            bfr = u32x4_t{C::template fp8<false>(even), C::template fp8<true>(even),
                                          C::template fp8<false>(odd), C::template fp8<true>(odd)};
                        } else {
                            // The slice's 16 bits; even codes to nibbles 0..3 of
                            // lo, odd ones of hi, FP4 pairs per byte: the same
                            // pair order as the 4-bit codes.
                            const uint32_t h = (dw[u] >> (16u * ((uint32_t)g & 1u))) ^ o.flip;
                            const uint32_t lo = h & 0x3333u, hi = (h >> 2) & 0x3333u;
                            bfr = u32x4_t{C::template fp4<0>(lo), C::template fp4<1>(lo),
                                          C::template fp4<0>(hi), C::template fp4<1>(hi)};
                        }
                        d = M16::mma(xa[u], __builtin_bit_cast(frag_t, bfr), d);
                    }
                    const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(xsw + (uint32_t)((gi * 16 + 4 * g) * 4));
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[rgi][r] = __builtin_fmaf(o.s, d[r], __builtin_fmaf(o.b, xs[r], acc[rgi][r]));
                });
            }
        });
    }

    // The row groups' partial sums to LDS (over the staging region, which
    // every slice is done with), then the K-slices of each row group meet
    // and lanes store weight row n = 16 rg + l16 against activation rows
    // 4g .. 4g+3.
#pragma unroll
    for (int r = 0; r < kSkinnyRG; ++r)
        if (r < nrg_w)
            *reinterpret_cast<f32x4_t*>(xst + ((uint32_t)r * 64u + (uint32_t)lane) * 16u) = acc[r];
    __syncthreads();
    const int kmax = sh.ks < sh.slices ? sh.ks : sh.slices;
    for (int rg = wave; rg < nrg_b; rg += nwaves) {
        const int wr_of = rg % sh.wr, rgi = rg / sh.wr;
        f32x4_t tot = {0.f, 0.f, 0.f, 0.f};
        for (int k2 = 0; k2 < kmax; ++k2) {
            const int w2 = k2 * sh.wr + wr_of;
            tot += *reinterpret_cast<const f32x4_t*>(lds + (uint32_t)w2 * WL +
                                                     ((uint32_t)rgi * 64u + (uint32_t)lane) * 16u);
        }
        const int n = r_lo + 16 * rg + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g + r;
            const uint32_t off = (m < rows && n < r_hi) ? ((uint32_t)m * (uint32_t)R + (uint32_t)n) * (uint32_t)SB : OOB;
            buffer_store_elem<DT>(E::from_f32(tot[r]), ro, off);
        }
    }
}

template <int BITS, int DT, int GU>
hipError_t skinny4_launch_one(const GemvKernelArgs& k, const SkinnyShape& sh, dim3 grid, hipStream_t st)
{
    static bool attr_set = false;   // per instantiation; set before its first launch
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&qgemv_skinny4_kernel<BITS, DT, GU>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(kSkinnyMaxWaves * skinny4_wave_lds()));
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    const int waves = sh.ks * sh.wr;
    hipLaunchKernelGGL((qgemv_skinny4_kernel<BITS, DT, GU>), grid, dim3(64 * waves), waves * skinny4_wave_lds(), st, k, sh);
    return hipGetLastError();
}

template <int BITS, int DT>
hipError_t skinny4_launch(const GemvKernelArgs& k, const SkinnyShape& sh, dim3 grid, hipStream_t st)
{
    switch (k.gs) {
    case 32: return skinny4_launch_one<BITS, DT, 1>(k, sh, grid, st);
    case 64: return skinny4_launch_one<BITS, DT, 2>(k, sh, grid, st);
    case 128: return skinny4_launch_one<BITS, DT, 4>(k, sh, grid, st);
    }
    return hipErrorInvalidValue;
}

} // namespace qp
