// skinny.hpp — products of a few activation rows (3 to 16, or an MoE tile of
// up to 16 pairs) on the 16x16x32 matrix instruction, with the codes kept
// exact (emily lib/emily/quantization.ex, `quantized_matmul/2`; the MoE form
// of ferrum-kernels src/stacked_expert.rs, `gemv_moe_id_batched` and
// `gemv_moe_id_gate_up_silu`):
//   out[m, n] = sum_g s'[n,g] * sum_{k in g} x[m,k] q[n,k] + b'[n,g] * sum_{k in g} x[m,k].
//
// One instruction contracts 32 k: operand A holds the activations (lane
// (g, m): row m, k-slot 8g .. 8g+7), operand B the codes as exact 16-bit
// values (lane (g, n): weight row n, the same k-slot), and the 16x16 result
// lands as lane (g, n) holding weight row n against activation rows
// 4g .. 4g+3. Here every instruction takes one unit (32 consecutive codes) of
// 16 weight rows, so its k never spans two groups, and a group's units chain
// into one result that is folded at once:
//   acc += s_eff * D + b_eff * (sum of the group's activations),
// with the scale and bias oriented so that the folded bias does not cancel
// against the codes (codepair.hpp, `orient`).
//
// Codes. A wave reads an item: UI units of 16 weight rows, lane (g, n)
// loading the g-th quarter of row n's UI * 4 * BITS bytes (one 16- or 12-byte
// load, or two); a transpose across the wave's four rows of 16 lanes (four
// v_permlane*_swap per 32-bit word) then gives lane (g, n) the 8-code slice g
// of each unit. Each slice becomes four exact 16-bit pairs: FP8-E4M3
// conversions for codes up to 15 (3- and 4-bit, the 3-bit fields first spread
// to bytes), FP4-E2M1 for 2-bit codes, fp32 conversions of bytes for 6- and
// 8-bit codes. Activation k-slots follow the slice's pair order (even codes,
// then odd ones, for 2, 3 and 4 bits).
//
// Activations stay in registers: each wave owns a slice of KW = 16 units of
// K (64 VGPRs for 16 rows) and sweeps the weight rows of its block through
// it, so a block reads its activations once per slice, not once per row
// group. A block's waves split into ks slices along K times wr wave rows
// (every wr-th row group); the per-row-group partial sums meet in LDS at the
// end of the block. Each group's orientation is computed by one lane in four
// (the lanes of weight row n take groups g mod NG) and passed to the others
// with the same row swaps. Group sums of the activations are reduced across
// the four lane rows once per slice and kept in LDS next to the partial sums.
#pragma once

#include "codepair.hpp"
#include "gemv_core.hpp"

namespace qp {

template <int DT> struct SkMfma;
template <> struct SkMfma<DT_BF16> {
    using frag_t = bf16x8_t;
    static __device__ __forceinline__ f32x4_t mma(frag_t a, frag_t b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // acc + x.lo + x.hi for a pair of activations (one v_dot2 against 1, 1).
    static __device__ __forceinline__ float pair_sum(uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                               __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
    }
};
template <> struct SkMfma<DT_F16> {
    using frag_t = f16x8_t;
    static __device__ __forceinline__ f32x4_t mma(frag_t a, frag_t b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float pair_sum(uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, x), __builtin_bit_cast(f16x2_t, 0x3C003C00u),
                                      acc, false);
    }
};

// Lane rows: the wave as four rows of 16 lanes (row g = lanes 16g .. 16g+15).
// rows_transpose: on entry row g holds v[g][i] in r[i]; on exit v[i][g].
__device__ __forceinline__ void rows_transpose(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3)
{
    const auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);   // rows 2,3 of r0 <-> rows 0,1 of r2
    const auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);   // odd rows <-> even rows
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    r0 = c[0];
    r1 = c[1];
    r2 = d[0];
    r3 = d[1];
}
// The row exchange that leaves each instruction's 32 k inside one group when
// lane row g starts with unit g's slices 0..3 in r0..r3 (GU units per group):
// GU = 1 transposes (register f: slice g of unit f); GU = 2 swaps row pairs
// (register f: unit 2 (f / 2) + g % 2, slice f % 2 + 2 (g / 2)); GU = 4 keeps
// the rows (register f: slice f of unit g).
template <int GU>
__device__ __forceinline__ void rows_exchange(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3)
{
    if constexpr (GU == 1) {
        rows_transpose(r0, r1, r2, r3);
    } else if constexpr (GU == 2) {
        const auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
        const auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
        r0 = a[0];
        r2 = a[1];
        r1 = b[0];
        r3 = b[1];
    }
}
template <int GU> __device__ __forceinline__ int frag_unit(int f, int g)
{
    return GU == 1 ? f : GU == 2 ? 2 * (f / 2) + g % 2 : g;
}
template <int GU> __device__ __forceinline__ int frag_slice(int f, int g)
{
    return GU == 1 ? g : GU == 2 ? f % 2 + 2 * (g / 2) : f;
}

// Every lane gets rows 0 and 1's values of v, where rows g and g + 2 agree.
__device__ __forceinline__ void rows_gather2(uint32_t v, uint32_t (&o)[2])
{
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    o[0] = a[0];
    o[1] = a[1];
}
// Every lane gets the four rows' values of v.
__device__ __forceinline__ void rows_gather4(uint32_t v, uint32_t (&o)[4])
{
    const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);     // rows (0,1,0,1), (2,3,2,3)
    const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
    o[0] = b[0];
    o[1] = b[1];
    o[2] = c[0];
    o[3] = c[1];
}
// Sum over the four rows (the same order in every lane).
__device__ __forceinline__ float rows_sum(float v)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float s = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
    const uint32_t su = __builtin_bit_cast(uint32_t, s);
    const auto b = __builtin_amdgcn_permlane16_swap(su, su, false, false);
    return __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
}

// Per code width: UI units per item, LW registers per lane per item (the
// lane's quarter of the item's row bytes, plus scratch), the activation slot
// order, the exchange level XG the slices take for GU units per group, the
// slices after it, and fragment I's operand from them with every code
// complemented when flip is ~0.
template <int BITS> struct SkW;
template <> struct SkW<4> {
    static constexpr int UI = 4, LW = 4, WORDS = 4;
    static constexpr bool EO = true;   // slice pairs (0,2) (4,6) (1,3) (5,7)
    template <int GU> static constexpr int XG = GU;
    template <int GU> __device__ __forceinline__ static void prepare(uint32_t (&w)[LW])
    {
        rows_exchange<GU>(w[0], w[1], w[2], w[3]);
    }
    template <int DT, int I> __device__ __forceinline__ static u32x4_t frag(const uint32_t (&w)[LW], uint32_t flip)
    {
        using C = ExactCvt<DT>;
        const uint32_t lo = (w[I] ^ flip) & 0x0F0F0F0Fu;
        const uint32_t hi = ((w[I] >> 4) ^ flip) & 0x0F0F0F0Fu;
        return u32x4_t{C::template fp8<false>(lo), C::template fp8<true>(lo), C::template fp8<false>(hi),
                       C::template fp8<true>(hi)};
    }
};
template <> struct SkW<2> {
    static constexpr int UI = 8, LW = 4, WORDS = 4;   // the lane loads units 2g, 2g + 1
    static constexpr bool EO = true;
    template <int GU> static constexpr int XG = 1;   // fragment f: slice g of unit f
    template <int GU> __device__ __forceinline__ static void prepare(uint32_t (&w)[LW])
    {
        // Slice j (16 bits) of unit 2g in the low half, of unit 2g + 1 in the high.
        const uint32_t s0 = __builtin_amdgcn_perm(w[2], w[0], 0x05040100u);
        const uint32_t s1 = __builtin_amdgcn_perm(w[2], w[0], 0x07060302u);
        const uint32_t s2 = __builtin_amdgcn_perm(w[3], w[1], 0x05040100u);
        const uint32_t s3 = __builtin_amdgcn_perm(w[3], w[1], 0x07060302u);
        w[0] = s0;
        w[1] = s1;
        w[2] = s2;
        w[3] = s3;
        rows_transpose(w[0], w[1], w[2], w[3]);   // w[i]: this lane's slice of units 2i, 2i + 1
    }
    template <int DT, int I> __device__ __forceinline__ static u32x4_t frag(const uint32_t (&w)[LW], uint32_t flip)
    {
        using C = ExactCvt<DT>;
        constexpr int B = 2 * (I & 1);
        const uint32_t lo = (w[I / 2] ^ flip) & 0x33333333u;
        const uint32_t hi = ((w[I / 2] >> 2) ^ flip) & 0x33333333u;
        return u32x4_t{C::template fp4<B>(lo), C::template fp4<B + 1>(lo), C::template fp4<B>(hi),
                       C::template fp4<B + 1>(hi)};
    }
};
template <> struct SkW<8> {
    static constexpr int UI = 4, LW = 8, WORDS = 8;
    static constexpr bool EO = false;
    template <int GU> static constexpr int XG = GU;
    template <int GU> __device__ __forceinline__ static void prepare(uint32_t (&w)[LW])
    {
        rows_exchange<GU>(w[0], w[2], w[4], w[6]);   // first words of slices 0..3
        rows_exchange<GU>(w[1], w[3], w[5], w[7]);   // second words
    }
    template <int DT, int I> __device__ __forceinline__ static u32x4_t frag(const uint32_t (&w)[LW], uint32_t flip)
    {
        using C = ExactCvt<DT>;
        const uint32_t a = w[2 * I] ^ flip, b = w[2 * I + 1] ^ flip;
        return u32x4_t{C::template bytes<false>(a), C::template bytes<true>(a), C::template bytes<false>(b),
                       C::template bytes<true>(b)};
    }
};
template <> struct SkW<3> {
    static constexpr int UI = 4, LW = 4, WORDS = 3;   // w[3] is scratch
    static constexpr bool EO = true;
    template <int GU> static constexpr int XG = GU;
    template <int GU> __device__ __forceinline__ static void prepare(uint32_t (&w)[LW])
    {
        // Slice j = bytes 3j .. 3j+2 of the unit, in the low 24 bits.
        const uint32_t s1 = __builtin_amdgcn_alignbyte(w[1], w[0], 3);
        const uint32_t s2 = __builtin_amdgcn_alignbyte(w[2], w[1], 2);
        const uint32_t s3 = w[2] >> 8;
        w[1] = s1;
        w[2] = s2;
        w[3] = s3;
        rows_exchange<GU>(w[0], w[1], w[2], w[3]);
    }
    template <int DT, int I> __device__ __forceinline__ static u32x4_t frag(const uint32_t (&w)[LW], uint32_t flip)
    {
        using C = ExactCvt<DT>;
        uint32_t even, odd;
        code_bytes3(w[I], flip, even, odd);
        return u32x4_t{C::template fp8<false>(even), C::template fp8<true>(even), C::template fp8<false>(odd),
                       C::template fp8<true>(odd)};
    }
};
template <> struct SkW<6> {
    static constexpr int UI = 4, LW = 8, WORDS = 6;   // w[6], w[7] are scratch
    static constexpr bool EO = false;
    template <int GU> static constexpr int XG = GU;
    template <int GU> __device__ __forceinline__ static void prepare(uint32_t (&w)[LW])
    {
        // Slice j = bytes 6j .. 6j+5: codes 0..3 in h0[j], 4..7 in h1[j] (24 bits each).
        uint32_t h0[4], h1[4];
        h0[0] = w[0];
        h1[0] = __builtin_amdgcn_alignbyte(w[1], w[0], 3);
        h0[1] = __builtin_amdgcn_alignbyte(w[2], w[1], 2);
        h1[1] = w[2] >> 8;
        h0[2] = w[3];
        h1[2] = __builtin_amdgcn_alignbyte(w[4], w[3], 3);
        h0[3] = __builtin_amdgcn_alignbyte(w[5], w[4], 2);
        h1[3] = w[5] >> 8;
        rows_exchange<GU>(h0[0], h0[1], h0[2], h0[3]);
        rows_exchange<GU>(h1[0], h1[1], h1[2], h1[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = h0[i];
            w[2 * i + 1] = h1[i];
        }
    }
    template <int DT, int I> __device__ __forceinline__ static u32x4_t frag(const uint32_t (&w)[LW], uint32_t flip)
    {
        using C = ExactCvt<DT>;
        const uint32_t a = code_bytes6(w[2 * I], flip), b = code_bytes6(w[2 * I + 1], flip);
        return u32x4_t{C::template bytes<false>(a), C::template bytes<true>(a), C::template bytes<false>(b),
                       C::template bytes<true>(b)};
    }
};

// The lane's WORDS words of an item (one 16- or 12-byte load, or 16 + 16 /
// 16 + 8 bytes).
template <int BITS>
__device__ __forceinline__ void skinny_load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[SkW<BITS>::LW])
{
    if constexpr (BITS == 3) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
        w[0] = v[0];
        w[1] = v[1];
        w[2] = v[2];
    } else if constexpr (BITS == 6) {
        const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        const u32x2_t u = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off + 16, 0, 0));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        w[4] = u.x; w[5] = u.y;
    } else {
#pragma unroll
        for (int i = 0; i < SkW<BITS>::LW; i += 4) {
            const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * i, 0, 0));
            w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
        }
    }
}

constexpr int kSkinnyKW = 16;        // units per wave slice (64 VGPRs of activations)
constexpr int kSkinnyRG = 4;         // row groups per wave at most
constexpr int kSkinnyMaxWaves = 8;

// Items in flight per wave: about 48 VGPRs of codes and scales, a whole
// number of row groups' items of a slice.
template <int BITS, int NMAT, int NG> constexpr int skinny_ring()
{
    constexpr int per = NMAT * (SkW<BITS>::LW + (NG == 8 ? 4 : 2));
    constexpr int nq = kSkinnyKW / SkW<BITS>::UI;
    return 48 / per >= 2 * nq ? 2 * nq : nq;
}

// Launch shape: blocks of ks * wr waves over rows_per_block weight rows;
// `slices` K-slices of kSkinnyKW units.
struct SkinnyShape {
    int rows_per_block;
    int ks;
    int wr;
    int slices;
};

// LDS, per wave: first its activation slice as loaded (16 rows of 1 KB,
// each padded by 16 bytes so that a fragment read spreads over the banks);
// once the fragments are in registers the same bytes hold the partial sums
// of its row groups (NMAT x 1 KB each), the group sums of the slice (16
// groups x 16 rows, fp32) and one row group's scales and biases over the
// slice (16 rows x 16 groups x 2 x NMAT, 16-bit).
constexpr uint32_t kSkinnyXRow = kSkinnyKW * 64u + 16u;
__host__ __device__ constexpr uint32_t skinny_wave_lds(int nmat)
{
    const uint32_t rest = (uint32_t)(kSkinnyRG * nmat + 1 + nmat) * 1024u;
    return 16u * kSkinnyXRow > rest ? 16u * kSkinnyXRow : rest;
}
__host__ __device__ constexpr uint32_t skinny_lds_bytes(int waves, int nmat)
{
    return (uint32_t)waves * skinny_wave_lds(nmat);
}

template <int BITS, int DT, int NMAT, int GU>
__global__ __launch_bounds__(64 * kSkinnyMaxWaves) void qgemv_skinny_kernel(GemvKernelArgs a, SkinnyShape sh)
{
    using M16 = SkMfma<DT>;
    using frag_t = typename M16::frag_t;
    using E = Elem<DT>;
    using St = typename E::storage;
    using W = SkW<BITS>;
    constexpr int UI = W::UI, LW = W::LW;
    constexpr int NQ = kSkinnyKW / UI;               // items per row group of a slice
    constexpr int NG = UI / GU;                      // groups per item
    constexpr int NGL = NG == 8 ? 2 : 1;             // groups whose orientation a lane computes
    constexpr int NGS = kSkinnyKW / GU;              // groups per slice
    constexpr int SBL = 16 * NGS / 64;               // scales per lane and row group
    constexpr int D = skinny_ring<BITS, NMAT, NG>();
    static_assert(D % NQ == 0, "ring of whole row groups");
    constexpr int SB = (int)sizeof(St);
    static_assert(SB == 2, "16-bit activations, scales and biases");
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int nwaves = (int)(blockDim.x >> 6);
    const int ksi = wave / sh.wr, wri = wave % sh.wr;
    const int g = lane >> 4, l16 = lane & 15;
    const int R = (int)a.R;
    const int K = (int)a.K;
    const int units = K / 32;
    const uint32_t row_bytes = (uint32_t)K * BITS / 8;
    const uint32_t G = (uint32_t)(K / a.gs);
    constexpr uint32_t WL = skinny_wave_lds(NMAT);
    char* const xst = lds + (uint32_t)wave * WL;                              // [row][k] as loaded
    char* const red = xst;                                                    // [rg][t] x 1 KB
    char* const xsw = xst + (uint32_t)(kSkinnyRG * NMAT) * 1024u;             // [group][row] fp32
    uint16_t* const sbw = reinterpret_cast<uint16_t*>(xsw + 1024u);           // [t][s, b][row][group]
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out, a.out_bytes);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);

    const int ntiles = gemv_num_tiles(a);
    for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
        int expert, start, count;
        if (!gemv_tile(a, tile, expert, start, count))
            continue;   // uniform over the block
        const int rows = count < 16 ? count : 16;
        const int r_lo = (int)blockIdx.x * sh.rows_per_block;
        const int r_hi = (r_lo + sh.rows_per_block) < R ? (r_lo + sh.rows_per_block) : R;
        const int nrg_b = r_hi > r_lo ? (r_hi - r_lo + 15) / 16 : 0;          // row groups of the block
        const int nrg_w = wri < nrg_b ? (nrg_b - wri + sh.wr - 1) / sh.wr : 0;   // of this wave

        // Resources over the block's own rows: rows past them read zeros.
        __amdgpu_buffer_rsrc_t rw[NMAT], rs[NMAT], rb[NMAT];
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            const uint64_t row_lo = (uint64_t)expert * (uint64_t)R + (uint64_t)r_lo;
            const uint32_t nrows = (uint32_t)(r_hi - r_lo);
            rw[t] = make_rsrc(reinterpret_cast<const char*>(a.wq[t]) + row_lo * row_bytes, nrows * row_bytes);
            rs[t] = make_rsrc(static_cast<const char*>(a.scales[t]) + row_lo * G * SB, nrows * G * SB);
            rb[t] = make_rsrc(static_cast<const char*>(a.biases[t]) + row_lo * G * SB, nrows * G * SB);
        }
        // Activation row of lane (g, m): m = l16 (OOB past the tile).
        uint32_t xoff = OOB;
        if (l16 < rows) {
            const uint32_t p = a.perm != nullptr ? (uint32_t)a.perm[start + l16] : (uint32_t)(start + l16);
            const uint32_t tk = (uint32_t)a.top_k;
            xoff = ((p / tk) * (uint32_t)a.outer + (p % tk) * (uint32_t)a.inner) * SB;
        }

        for (int si = 0; si * sh.ks + ksi < sh.slices; ++si) {
            const int u0 = (si * sh.ks + ksi) * kSkinnyKW;   // first unit of the slice
            const int nitems = nrg_w * NQ;

            // Activations of the slice: fragment f of item q takes row l16 at
            // the unit and slice the code exchange gives lane row g there.
            constexpr int XG = W::template XG<GU>;
            // A wave with one slice loads its 16 rows whole (1 KB of a row
            // per instruction) and regroups them through LDS; a wave with
            // several slices keeps partial sums in that LDS between slices
            // and loads each fragment directly.
            const bool staged = sh.slices <= sh.ks;   // uniform
            u32x4_t raw[kSkinnyKW];
            if (staged) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t xr = (uint32_t)__builtin_amdgcn_readlane((int)xoff, r);
                    const uint32_t off = (xr != OOB && u0 * 32 + 8 * lane < K)
                        ? xr + (uint32_t)(u0 * 32 + 8 * lane) * 2u : OOB;
                    raw[r] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
                }
            } else {
#pragma unroll
                for (int u = 0; u < kSkinnyKW; ++u) {
                    const int un = u0 + (u / UI) * UI + frag_unit<XG>(u % UI, g);
                    const uint32_t off = (xoff != OOB && un < units)
                        ? xoff + (uint32_t)(un * 32 + 8 * frag_slice<XG>(u % UI, g)) * 2u : OOB;
                    raw[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
                }
            }
            // Activations are requested before the first codes (waiting for
            // them must not wait for codes too).
            __builtin_amdgcn_sched_barrier(0);

            // The ring: item j is row group rg = wri + wr (j / NQ), units
            // u0 + UI (j % NQ) ...; lane (g, n) loads quarter g of weight row
            // n's bytes of them. The first item of a row group also carries
            // its scales and biases over the slice (16 rows x NGS groups,
            // SBL per lane), which go to LDS when that item is processed.
            struct Slot {
                uint32_t w[NMAT][LW];
                St sb[NMAT][2][SBL];
            };
            Slot ring[D];
            // Per lane, once per slice: the byte offsets of its first row
            // group's codes and scales in the block; an item adds whole row
            // groups and units to them. No test guards the code loads: rows
            // past the block are out of range, and a unit past K (an item
            // straddling the end of a row) reads codes that meet zero
            // activations. Groups past K / gs would read another row's
            // scales, so those lanes' offsets get the out-of-range bit.
            const int row0 = 16 * wri + l16;
            const int lane_grp = NG == 1 ? 0 : g % (NG < 4 ? NG : 4);
            const uint32_t wbase = (uint32_t)row0 * row_bytes + (uint32_t)u0 * (4u * BITS) + (uint32_t)(UI * BITS * g);
            const uint32_t wstep = 16u * (uint32_t)sh.wr * row_bytes, sstep = 16u * (uint32_t)sh.wr * G * SB;
            uint32_t sboff[SBL];                                  // scale v = lane + 64 i: row v / NGS, group v % NGS
#pragma unroll
            for (int i = 0; i < SBL; ++i) {
                const int v = lane + 64 * i, gl = u0 / GU + v % NGS;
                sboff[i] = (((uint32_t)(16 * wri + v / NGS) * G + (uint32_t)gl) * SB) | ((uint32_t)gl >= G ? OOB : 0u);
            }
            auto fetch = [&](int j, auto Q, Slot& sl) {
                constexpr int q = decltype(Q)::value;
                const uint32_t rgi = (uint32_t)(j / NQ);
                const uint32_t woff = wbase + rgi * wstep + (uint32_t)(q * UI * 4 * BITS);
#pragma unroll
                for (int t = 0; t < NMAT; ++t) {
                    skinny_load<BITS>(rw[t], woff, sl.w[t]);
                    if constexpr (q == 0) {
#pragma unroll
                        for (int i = 0; i < SBL; ++i) {
                            sl.sb[t][0][i] = __builtin_amdgcn_raw_buffer_load_b16(rs[t], sboff[i] + rgi * sstep, 0, 0);
                            sl.sb[t][1][i] = __builtin_amdgcn_raw_buffer_load_b16(rb[t], sboff[i] + rgi * sstep, 0, 0);
                        }
                    }
                }
            };
            static_for<D>([&](auto J) {
                fetch((int)J, std::integral_constant<int, (int)J % NQ>{}, ring[J]);
                __builtin_amdgcn_sched_barrier(0);   // slot by slot, in order
            });

            if (staged) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    *reinterpret_cast<u32x4_t*>(xst + (uint32_t)r * kSkinnyXRow + 16u * (uint32_t)lane) = raw[r];
#pragma unroll
                for (int u = 0; u < kSkinnyKW; ++u) {
                    const int ur = (u / UI) * UI + frag_unit<XG>(u % UI, g);
                    raw[u] = *reinterpret_cast<const u32x4_t*>(
                        xst + (uint32_t)l16 * kSkinnyXRow + (uint32_t)(ur * 32 + 8 * frag_slice<XG>(u % UI, g)) * 2u);
                }
            }
            // Activation slots in the codes' pair order.
            frag_t xa[kSkinnyKW];
#pragma unroll
            for (int u = 0; u < kSkinnyKW; ++u) {
                u32x4_t v = raw[u];
                if constexpr (W::EO)
                    v = u32x4_t{__builtin_amdgcn_perm(raw[u].y, raw[u].x, 0x05040100u),
                                __builtin_amdgcn_perm(raw[u].w, raw[u].z, 0x05040100u),
                                __builtin_amdgcn_perm(raw[u].y, raw[u].x, 0x07060302u),
                                __builtin_amdgcn_perm(raw[u].w, raw[u].z, 0x07060302u)};
                xa[u] = __builtin_bit_cast(frag_t, v);
            }

            // Group sums of the slice's activations: per unit a dot2 against
            // (1, 1) per pair, per group over its units, then over the four
            // lane rows; stored as xsw[group][row].
            static_for<kSkinnyKW / GU>([&](auto GI) {
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

            f32x4_t acc[NMAT];
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
                acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

            auto process = [&](int j, auto Q, const Slot& sl) {
                constexpr int q = decltype(Q)::value;
                __builtin_amdgcn_sched_barrier(0);
                // Orientation of the lane's group(s); then every lane gets the item's NG.
                float se[NMAT][NG], be[NMAT][NG];
                uint32_t fl[NMAT][NG];
                // The slot is read here and not earlier: an empty asm per
                // value keeps the compiler from hoisting work on it (which
                // would wait for its load before earlier items run).
                uint32_t sv[NMAT][NGL], bv[NMAT][NGL];
                uint32_t cw[NMAT][LW];
#pragma unroll
                for (int t = 0; t < NMAT; ++t) {
                    if constexpr (q == 0) {
                        // The row group's scales and biases to LDS.
#pragma unroll
                        for (int i = 0; i < SBL; ++i) {
                            uint32_t a0 = sl.sb[t][0][i], a1 = sl.sb[t][1][i];
                            asm volatile("" : "+v"(a0), "+v"(a1));
                            sbw[(t * 2 + 0) * 16 * NGS + lane + 64 * i] = (uint16_t)a0;
                            sbw[(t * 2 + 1) * 16 * NGS + lane + 64 * i] = (uint16_t)a1;
                        }
                    }
#pragma unroll
                    for (int h = 0; h < NGL; ++h) {
                        const int e = l16 * NGS + q * NG + lane_grp + 4 * h;
                        sv[t][h] = sbw[(t * 2 + 0) * 16 * NGS + e];
                        bv[t][h] = sbw[(t * 2 + 1) * 16 * NGS + e];
                    }
#pragma unroll
                    for (int i = 0; i < W::WORDS; ++i) {
                        cw[t][i] = sl.w[t][i];
                        asm volatile("" : "+v"(cw[t][i]));
                    }
                }
#pragma unroll
                for (int t = 0; t < NMAT; ++t) {
#pragma unroll
                    for (int h = 0; h < NGL; ++h) {
                        const Orient o = orient<BITS>(E::to_f32((St)sv[t][h]), E::to_f32((St)bv[t][h]));
                        const uint32_t vs = __builtin_bit_cast(uint32_t, o.s), vb = __builtin_bit_cast(uint32_t, o.b);
                        if constexpr (NG == 1) {
                            se[t][0] = o.s;
                            be[t][0] = o.b;
                            fl[t][0] = o.flip;
                        } else if constexpr (NG == 2) {
                            uint32_t s2[2], b2[2], f2[2];
                            rows_gather2(vs, s2);
                            rows_gather2(vb, b2);
                            rows_gather2(o.flip, f2);
#pragma unroll
                            for (int i = 0; i < 2; ++i) {
                                se[t][i] = __builtin_bit_cast(float, s2[i]);
                                be[t][i] = __builtin_bit_cast(float, b2[i]);
                                fl[t][i] = f2[i];
                            }
                        } else {
                            uint32_t s4[4], b4[4], f4[4];
                            rows_gather4(vs, s4);
                            rows_gather4(vb, b4);
                            rows_gather4(o.flip, f4);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                se[t][4 * h + i] = __builtin_bit_cast(float, s4[i]);
                                be[t][4 * h + i] = __builtin_bit_cast(float, b4[i]);
                                fl[t][4 * h + i] = f4[i];
                            }
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < NMAT; ++t)
                    W::template prepare<GU>(cw[t]);
                __builtin_amdgcn_sched_barrier(0);
                static_for<NG>([&](auto JG) {
                    constexpr int jg = decltype(JG)::value;
                    const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(
                        xsw + (uint32_t)(((q * NG + jg) * 16 + 4 * g) * 4));
#pragma unroll
                    for (int t = 0; t < NMAT; ++t) {
                        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
                        static_for<GU>([&](auto UU) {
                            constexpr int i = jg * GU + decltype(UU)::value;
                            const u32x4_t bw = W::template frag<DT, i>(cw[t], fl[t][jg]);
                            d = M16::mma(xa[q * UI + i], __builtin_bit_cast(frag_t, bw), d);
                        });
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[t][r] = __builtin_fmaf(se[t][jg], d[r], __builtin_fmaf(be[t][jg], xs[r], acc[t][r]));
                    }
                });
                // Last item of a row group: its partial sums go to LDS.
                if constexpr (q == NQ - 1) {
                    const int rgi = j / NQ;
#pragma unroll
                    for (int t = 0; t < NMAT; ++t) {
                        f32x4_t* dst = reinterpret_cast<f32x4_t*>(
                            red + ((uint32_t)(rgi * NMAT + t) * 64u + (uint32_t)lane) * 16u);
                        if (si == 0)
                            *dst = acc[t];
                        else
                            *dst = *dst + acc[t];
                        acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            // The whole item sequence of a slice, unrolled: ring slots are
            // never carried around a loop or through a branch (either makes
            // the compiler copy a slot, which waits for its load to land).
            // Refills past the wave's items read zeros.
            static_for<kSkinnyRG * NQ>([&](auto JJ) {
                constexpr int j = decltype(JJ)::value;
                if (j < nitems)
                    process(j, std::integral_constant<int, j % NQ>{}, ring[j % D]);
                if constexpr (j + D < kSkinnyRG * NQ)
                    fetch(j + D, std::integral_constant<int, j % NQ>{}, ring[j % D]);
            });
        }

        // The K-slices of each row group meet; lanes store weight row
        // n = 16 rg + l16 against activation rows 4g .. 4g+3.
        __syncthreads();
        const int kmax = sh.ks < sh.slices ? sh.ks : sh.slices;
        for (int rg = wave; rg < nrg_b; rg += nwaves) {
            const int wr_of = rg % sh.wr, rgi = rg / sh.wr;
            f32x4_t tot[NMAT];
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
                tot[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            for (int k2 = 0; k2 < kmax; ++k2) {
                const int w2 = k2 * sh.wr + wr_of;
#pragma unroll
                for (int t = 0; t < NMAT; ++t)
                    tot[t] += *reinterpret_cast<const f32x4_t*>(
                        lds + (uint32_t)w2 * WL + ((uint32_t)(rgi * NMAT + t) * 64u + (uint32_t)lane) * 16u);
            }
            const int n = r_lo + 16 * rg + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * g + r;
                float v = tot[0][r];
                if constexpr (NMAT == 2)
                    v = silu_f32(tot[0][r]) * tot[1][r];
                uint32_t off = OOB;
                if (m < rows && n < r_hi) {
                    const uint32_t pr = a.perm != nullptr ? (uint32_t)a.perm[start + m] : (uint32_t)(start + m);
                    off = (pr * (uint32_t)R + (uint32_t)n) * (uint32_t)SB;
                }
                buffer_store_elem<DT>(E::from_f32(v), ro, off);
            }
        }
        // Every wave is done with the partial sums before the next tile.
        __syncthreads();
    }
}

} // namespace qp

namespace qp {

// Launch one instance (the LDS size is set once per instance).
template <int BITS, int DT, int NMAT, int GU>
hipError_t skinny_launch_one(const GemvKernelArgs& k, const SkinnyShape& sh, dim3 grid, hipStream_t st)
{
    static bool attr_set = false;   // per instantiation; set before its first launch
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&qgemv_skinny_kernel<BITS, DT, NMAT, GU>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)skinny_lds_bytes(kSkinnyMaxWaves, NMAT));
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    const int waves = sh.ks * sh.wr;
    hipLaunchKernelGGL((qgemv_skinny_kernel<BITS, DT, NMAT, GU>), grid, dim3(64 * waves),
                       skinny_lds_bytes(waves, NMAT), st, k, sh);
    return hipGetLastError();
}

template <int BITS, int DT, int NMAT>
hipError_t skinny_launch(const GemvKernelArgs& k, const SkinnyShape& sh, dim3 grid, hipStream_t st)
{
    switch (k.gs) {
    case 32: return skinny_launch_one<BITS, DT, NMAT, 1>(k, sh, grid, st);
    case 64: return skinny_launch_one<BITS, DT, NMAT, 2>(k, sh, grid, st);
    case 128: return skinny_launch_one<BITS, DT, NMAT, 4>(k, sh, grid, st);
    }
    return hipErrorInvalidValue;
}

// Waves along K (one per slice, at most 8) and along row groups (the rest of
// the 8 waves, at most the row groups there are).
inline SkinnyShape skinny_waves(int64_t K, int64_t rgs_per_block)
{
    SkinnyShape sh{};
    const int64_t units = K / 32;
    sh.slices = (int)((units + kSkinnyKW - 1) / kSkinnyKW);
    sh.ks = sh.slices < kSkinnyMaxWaves ? sh.slices : kSkinnyMaxWaves;
    int64_t wr = kSkinnyMaxWaves / sh.ks;
    wr = wr < rgs_per_block ? wr : rgs_per_block;
    sh.wr = (int)(wr < 1 ? 1 : wr);
    return sh;
}

// Dense shape: about one block per CU over contiguous row ranges, in whole
// row groups (a partial group costs a full one's work: at 14336 x 4096, M =
// 16, 64 rows per block (224 blocks) measured 15.0-15.2 us against 15.1-15.5
// us for 56 rows (256 blocks); fewer rows per block, more blocks, were
// slower: 32 rows 20.2 us, 16 rows 28.5 us, each block setting up the
// activations again).
inline void skinny_dense_shape(int64_t N, int64_t K, SkinnyShape* sh, dim3* grid)
{
    int64_t rpb = (N + 255) / 256;
    rpb = (rpb + 15) / 16 * 16;
    *sh = skinny_waves(K, (rpb + 15) / 16);
    const int64_t cap = 16 * (int64_t)sh->wr * kSkinnyRG;
    rpb = rpb < cap ? rpb : cap;
    sh->rows_per_block = (int)rpb;
    *grid = dim3((unsigned)((N + rpb - 1) / rpb), 1);
}

// MoE shape: row blocks per tile, fewer rows per block until the largest
// possible tile list gives about 512 blocks.
inline void skinny_moe_shape(int64_t R, int64_t K, int64_t max_tiles, SkinnyShape* sh, unsigned* gx)
{
    *sh = skinny_waves(K, (R + 15) / 16);
    int rgw = kSkinnyRG;
    while (rgw > 1 && max_tiles * ((R + 16 * sh->wr * rgw - 1) / (16 * sh->wr * rgw)) < 512)
        rgw /= 2;
    sh->rows_per_block = 16 * sh->wr * rgw;
    *gx = (unsigned)((R + sh->rows_per_block - 1) / sh->rows_per_block);
}

} // namespace qp
