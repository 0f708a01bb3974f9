// skinny.hpp — products of a few activation rows (3 to 16, or an MoE tile of
// up to 16 pairs) on the 16x16x32 matrix instruction, with the codes kept
// exact (emily lib/emily/quantization.ex, `quantized_matmul/2`; the MoE form
// of ferrum-kernels src/stacked_expert.rs, `gemv_moe_id_batched` and
// `gemv_moe_id_gate_up_silu`):
//   out[m, n] = sum_g s'[n,g] * sum_{k in g} x[m,k] q[n,k] + b'[n,g] * sum_{k in g} x[m,k].
//
// One instruction contracts 32 consecutive k: operand B holds the codes (lane
// (g, n) of the wave: weight row n, codes 8g .. 8g+7 of the k-block) as exact
// 16-bit values, operand A the activations (lane (g, i): row i of A, the same
// k). A chunk is 128 k of 16 weight rows: lane (g, n) owns unit 4c + g (32
// codes) of row n and feeds codes 8j .. 8j+7 of it to instruction j = 0..3, so
// that instruction mixes the four units of the chunk. The 16 rows of A keep
// their groups apart: with SLOTS = 128 / group_size groups per chunk, row i of
// A is activation row i % MS of group slot i / MS (MS = 16 / SLOTS), and a lane
// of A whose slot is not its unit's group reads zeros. Output lane (g, n) then
// holds weight row n against four activation rows of one group slot, the
// slot of its own unit: one group's sum per lane, folded at once as
//   acc += s_eff * D + b_eff * (sum of the group's activations),
// with the group's scale and bias oriented so that the folded bias does not
// cancel against the codes (codepair.hpp, `orient`). More activation rows than
// MS take MP passes of the same codes against further rows of A.
//
// Activations: the tile's rows sit in LDS as a table (row m at m * row_stride,
// natural order), with each group's sum beside it; each row group's scales
// and biases sit there too. Every wave first issues its share of those as
// LDS DMA (1 KB per instruction, every offset in a register of its own so no
// transfer waits for another), then its first chunks of codes, then waits
// once for the DMA alone: a load that had to land before the next was issued
// costs a full memory latency under the weight stream. Group sums come from
// the table afterwards (a dot2 with (1, 1) per lane, then a fixed butterfly
// over the group's lanes). One block per CU covers a range of weight rows: its waves split into
// n_rg groups of 16 rows and ks waves along K (interleaved chunks), so the
// table is filled once per block, not once per 16 rows. Codes are loaded row
// by row (four neighbouring lanes read one row's 4 units, 16 * BITS contiguous
// bytes) and moved to operand order with one ds_bpermute per word.
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
};
template <> struct SkMfma<DT_F16> {
    using frag_t = f16x8_t;
    static __device__ __forceinline__ f32x4_t mma(frag_t a, frag_t b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// acc + x.lo + x.hi for a pair of 16-bit activations (one v_dot2 against 1, 1).
template <int DT> struct RowStreamPairSk;
template <> struct RowStreamPairSk<DT_BF16> {
    static __device__ __forceinline__ float dot(uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                               __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
    }
};
template <> struct RowStreamPairSk<DT_F16> {
    static __device__ __forceinline__ float dot(uint32_t x, float acc)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, x), __builtin_bit_cast(f16x2_t, 0x3C003C00u),
                                      acc, false);
    }
};

// The 16 exact code pairs of one unit in natural order (pair q = codes 2q and
// 2q + 1), every code first complemented when flip is ~0.
template <int BITS, int DT>
__device__ __forceinline__ void natural_pairs(const uint32_t* win, uint32_t flip, uint32_t (&p)[16])
{
    using C = ExactCvt<DT>;
    uint32_t w[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i)
        w[i] = win[i] ^ flip;
    if constexpr (BITS == 4) {
        // lo / hi bytes hold codes 8i + 2b / 8i + 2b + 1; byte-interleave them
        // into codes 8i .. 8i+3 and 8i+4 .. 8i+7, each converted as FP8 pairs.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
            const uint32_t a = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
            const uint32_t b = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
            p[4 * i + 0] = C::template fp8<false>(a);
            p[4 * i + 1] = C::template fp8<true>(a);
            p[4 * i + 2] = C::template fp8<false>(b);
            p[4 * i + 3] = C::template fp8<true>(b);
        }
    } else if constexpr (BITS == 2) {
        // t0 byte j = codes 4j | 4j+1 << 4, t1 byte j = codes 4j+2 | 4j+3 << 4
        // (of word i's 16), each byte an FP4 pair.
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t t0 = (w[i] & 0x03030303u) | ((w[i] << 2) & 0x30303030u);
            const uint32_t t1 = ((w[i] >> 4) & 0x03030303u) | ((w[i] >> 2) & 0x30303030u);
            p[8 * i + 0] = C::template fp4<0>(t0);
            p[8 * i + 1] = C::template fp4<0>(t1);
            p[8 * i + 2] = C::template fp4<1>(t0);
            p[8 * i + 3] = C::template fp4<1>(t1);
            p[8 * i + 4] = C::template fp4<2>(t0);
            p[8 * i + 5] = C::template fp4<2>(t1);
            p[8 * i + 6] = C::template fp4<3>(t0);
            p[8 * i + 7] = C::template fp4<3>(t1);
        }
    } else if constexpr (BITS == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[2 * i + 0] = C::pack((float)(w[i] & 0xFFu), (float)((w[i] >> 8) & 0xFFu));
            p[2 * i + 1] = C::pack((float)((w[i] >> 16) & 0xFFu), (float)(w[i] >> 24));
        }
    } else {
        static_for<16>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            p[q] = C::pack((float)unit_code<BITS, 2 * q>(w), (float)unit_code<BITS, 2 * q + 1>(w));
        });
    }
}

// Launch shape of one call: blocks of n_rg * ks waves, each block a range of
// rows_per_block weight rows; the activation table has mt rows of row_stride
// bytes (K * 2 rounded up to 1 KB, plus 16 so that rows fall on different
// banks).
struct SkinnyShape {
    int rows_per_block;
    int n_rg;
    int ks;
    int mt;
    int row_stride;
};

constexpr int kSkinnyMaxWaves = 8;
constexpr uint32_t kSkinnyLdsBytes = 156 * 1024;

__host__ __device__ constexpr int skinny_row_stride(int64_t K)
{
    return (int)((K * 2 + 1023) / 1024 * 1024 + 16);
}
// LDS: the table, the group sums [groups][mt] (fp32), each row group's scale
// and bias rows (16 rows x groups, rounded up to 1 KB per array and matrix),
// a zero fragment; the K-split partial sums reuse the table once every wave is
// done with it.
__host__ __device__ constexpr uint32_t skinny_sb_bytes(int64_t K, int gs, int nmat)
{
    return (uint32_t)((16 * (K / gs) * 2 + 1023) / 1024 * 1024) * 2u * (uint32_t)nmat;
}
__host__ __device__ constexpr uint32_t skinny_lds_bytes(int64_t K, int gs, int mt, int waves, int mp,
                                                         int nmat, int ks)
{
    const uint32_t table = (uint32_t)mt * (uint32_t)skinny_row_stride(K);
    const uint32_t red = (uint32_t)waves * (uint32_t)(nmat * mp) * 64u * 16u;
    const uint32_t xg = (uint32_t)((K + 127) / 128 * (128 / gs)) * (uint32_t)mt * 4u;
    const uint32_t n_rg = (uint32_t)((waves + ks - 1) / ks);
    return (table > red ? table : red) + xg + n_rg * skinny_sb_bytes(K, gs, nmat) + 64u;
}

// Chunks of codes in flight per wave: about 16 VGPRs of codes (each ring
// slot costs the compiler about four times its codes in registers, and a
// spill reload waits for every load in flight).
template <int BITS, int NMAT, int MP> constexpr int skinny_ring()
{
    constexpr int d = 16 / (NMAT * BITS * (MP > 2 ? 2 : 1));
    return d < 2 ? 2 : (d > 8 ? 8 : d);
}

// Load instructions per unit of BITS words (buffer_words: 16-, 8- or 4-byte
// loads).
template <int BITS> constexpr int skinny_loads_per_unit()
{
    return BITS % 4 == 0 ? BITS / 4 : BITS % 2 == 0 ? BITS / 2 : BITS;
}

// Table pieces (1 KB of one row) a wave issues per round of DMA.
constexpr int kSkinnyXPieces = 4;

// LDS DMA of 16 bytes per lane from byte offset src (OOB: zeros) to
// dst + 16 * lane.
__device__ __forceinline__ void skinny_dma(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t src)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, src, 0, 0, 0);
}

template <int BITS, int DT, int NMAT, int SLOTS, int MP>
__global__ __launch_bounds__(64 * kSkinnyMaxWaves) void qgemv_skinny_kernel(GemvKernelArgs a,
                                                                            SkinnyShape sh)
{
    using M16 = SkMfma<DT>;
    using frag_t = typename M16::frag_t;
    using E = Elem<DT>;
    using St = typename E::storage;
    static_assert(SLOTS == 1 || SLOTS == 2 || SLOTS == 4, "group_size 128, 64 or 32");
    constexpr int MS = 16 / SLOTS;                   // activation rows per pass
    static_assert(MP * MS <= 16, "at most 16 activation rows");
    constexpr int D = skinny_ring<BITS, NMAT, MP>();
    constexpr int SB = (int)sizeof(St);
    static_assert(SB == 2, "16-bit scales and biases");
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = (int)(blockDim.x >> 6);
    const int rg = wave / sh.ks, ks = wave % sh.ks;
    const int g = lane >> 4, r16 = lane & 15;        // operand lane: k-slice g, row r16
    const int lrow = lane >> 2, lg = lane & 3;       // load lane: row lrow, unit 4c + lg
    const int gslot = (g * SLOTS) >> 2;              // group slot of this lane's unit
    const int R = (int)a.R;
    const int K = (int)a.K;
    const uint32_t row_bytes = (uint32_t)K * BITS / 8;
    const uint32_t groups_row = (uint32_t)(K / a.gs);
    const int units = K / 32;
    const int NC = (K + 127) / 128;                  // chunks per row
    const int nj = ks < NC ? (NC - ks + sh.ks - 1) / sh.ks : 0;   // this wave's chunks
    const int GC = NC * SLOTS;                       // group slots along K (padded)
    char* const table = lds;
    const uint32_t table_bytes = (uint32_t)sh.mt * (uint32_t)sh.row_stride;
    const uint32_t red_bytes = (uint32_t)nwaves * (uint32_t)(NMAT * MP) * 1024u;
    char* const xg = lds + (table_bytes > red_bytes ? table_bytes : red_bytes);
    const uint32_t sb_bytes = skinny_sb_bytes(K, a.gs, NMAT);
    const uint32_t sb_arr = sb_bytes / (2u * NMAT);                    // one array of one row group
    char* const sbs = xg + (uint32_t)GC * (uint32_t)sh.mt * 4u;         // [row group][matrix][s, b]
    char* const sbg = sbs + (uint32_t)rg * sb_bytes;                   // this wave's row group
    char* const zero = sbs + (uint32_t)sh.n_rg * sb_bytes;
    if (tid < 4)
        reinterpret_cast<uint32_t*>(zero)[tid * 4 + 0] = reinterpret_cast<uint32_t*>(zero)[tid * 4 + 1] =
            reinterpret_cast<uint32_t*>(zero)[tid * 4 + 2] = reinterpret_cast<uint32_t*>(zero)[tid * 4 + 3] = 0u;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out, a.out_bytes);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const int bp_addr = (4 * r16 + g) * 4;           // ds_bpermute source: lane 4 n + g

    const int ntiles = gemv_num_tiles(a);
    for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
        int expert, start, count;
        if (!gemv_tile(a, tile, expert, start, count))
            continue;   // uniform over the block
        const int rows = count < sh.mt ? count : sh.mt;
        const int r_lo = (int)blockIdx.x * sh.rows_per_block;
        const int r_hi = (r_lo + sh.rows_per_block) < R ? (r_lo + sh.rows_per_block) : R;
        const int n0 = r_lo + 16 * rg;               // this wave's first weight row

        __amdgpu_buffer_rsrc_t rw[NMAT], rs[NMAT], rb[NMAT];
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            const uint64_t erow = (uint64_t)expert * (uint64_t)R;
            rw[t] = make_rsrc(reinterpret_cast<const char*>(a.wq[t]) + erow * row_bytes,
                              (uint32_t)R * row_bytes);
            rs[t] = make_rsrc(static_cast<const char*>(a.scales[t]) + erow * groups_row * SB,
                              (uint32_t)R * groups_row * SB);
            rb[t] = make_rsrc(static_cast<const char*>(a.biases[t]) + erow * groups_row * SB,
                              (uint32_t)R * groups_row * SB);
        }

        // 1. Row offsets of the tile's activation rows: lane m < 16 holds row
        //    m's byte offset (OOB past the tile).
        uint32_t xoff_l = OOB;
        if (lane < rows) {
            const uint32_t p = a.perm != nullptr ? (uint32_t)a.perm[start + lane]
                                                 : (uint32_t)(start + lane);
            const uint32_t tk = (uint32_t)a.top_k;
            xoff_l = ((p / tk) * (uint32_t)a.outer + (p % tk) * (uint32_t)a.inner) * SB;
        }
        __builtin_amdgcn_s_waitcnt(0);   // nothing else is in flight yet

        // 2. LDS DMA of the table: piece q = wave + nwaves i is row q / ppr,
        //    bytes (q % ppr) KB of it (bytes past K read zeros); then the
        //    scale and bias rows of this wave's row group (by its first wave
        //    along K). Rounds of kSkinnyXPieces pieces; offsets stay live
        //    until the wait below.
        const int ppr = (sh.row_stride - 16) / 1024;
        const int pieces = sh.mt * ppr;
        const int per_wave = (pieces + nwaves - 1) / nwaves;
        uint32_t xo[kSkinnyXPieces];
        for (int q0 = 0; q0 < per_wave; q0 += kSkinnyXPieces) {
            if (q0 > 0)
                __builtin_amdgcn_s_waitcnt(0);   // more than one round: before any code load
#pragma unroll
            for (int i = 0; i < kSkinnyXPieces; ++i) {
                const int q = wave + nwaves * (q0 + i);
                const int m = q / ppr, part = q % ppr;
                const uint32_t rowoff = (uint32_t)__builtin_amdgcn_readlane((int)xoff_l, m < 16 ? m : 0);
                const uint32_t kb = (uint32_t)part * 1024u + (uint32_t)lane * 16u;
                xo[i] = (q0 + i < per_wave && q < pieces && m < rows && kb < (uint32_t)K * 2u && rowoff != OOB)
                    ? rowoff + kb : OOB;
                if (q0 + i < per_wave && q < pieces)
                    skinny_dma(rx, table + (uint32_t)m * (uint32_t)sh.row_stride + (uint32_t)part * 1024u, xo[i]);
            }
        }
        // Scale and bias rows: 16-byte DMA pieces, except for a row group that
        // ends past the matrix or an array that does not start on 16 bytes,
        // which go element by element (the range check would not return a
        // piece that crosses the buffer's end whole).
        uint32_t so[4 * NMAT];
        {
            const uint32_t bytes = 16u * groups_row * (uint32_t)SB;   // one array of 16 rows
            const uint32_t base = (uint32_t)n0 * groups_row * (uint32_t)SB;
            const int npc = (int)(sb_arr / 1024u);
            const uint64_t eoff = (uint64_t)expert * (uint64_t)R * groups_row * SB;
#pragma unroll
            for (int t = 0; t < NMAT; ++t) {
                const bool plain = n0 + 16 > R ||
                    ((reinterpret_cast<uintptr_t>(a.scales[t]) + eoff) & 15u) != 0 ||
                    ((reinterpret_cast<uintptr_t>(a.biases[t]) + eoff) & 15u) != 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t off = (uint32_t)i * 1024u + (uint32_t)lane * 16u;
                    so[4 * t + i] = off < bytes ? base + off : OOB;
                    if (ks == 0 && !plain && i < npc) {
                        skinny_dma(rs[t], sbg + (uint32_t)(2 * t) * sb_arr + (uint32_t)i * 1024u, so[4 * t + i]);
                        skinny_dma(rb[t], sbg + (uint32_t)(2 * t + 1) * sb_arr + (uint32_t)i * 1024u, so[4 * t + i]);
                    }
                }
                if (ks == 0 && !plain)
                    for (int i = 4; i < npc; ++i) {   // longer scale rows (K / gs above 128)
                        const uint32_t off = (uint32_t)i * 1024u + (uint32_t)lane * 16u;
                        const uint32_t o2 = off < bytes ? base + off : OOB;
                        skinny_dma(rs[t], sbg + (uint32_t)(2 * t) * sb_arr + (uint32_t)i * 1024u, o2);
                        skinny_dma(rb[t], sbg + (uint32_t)(2 * t + 1) * sb_arr + (uint32_t)i * 1024u, o2);
                    }
                if (ks == 0 && plain) {
                    // Elements up to 15 G + GC: the padded group slots of row
                    // 15 read zeros, as they do after the DMA.
                    const uint32_t n_el = 15u * groups_row + (uint32_t)GC;
                    for (uint32_t e = (uint32_t)lane; e < n_el; e += 64u) {
                        // Rows past the matrix read zeros.
                        const uint32_t off = e < 16u * groups_row ? base + e * (uint32_t)SB : OOB;
                        reinterpret_cast<uint16_t*>(sbg + (uint32_t)(2 * t) * sb_arr)[e] =
                            __builtin_amdgcn_raw_buffer_load_b16(rs[t], off, 0, 0);
                        reinterpret_cast<uint16_t*>(sbg + (uint32_t)(2 * t + 1) * sb_arr)[e] =
                            __builtin_amdgcn_raw_buffer_load_b16(rb[t], off, 0, 0);
                    }
                }
            }
        }

        // 3. The code ring: chunk j of this wave is c = ks + KS j; load lane
        //    (lrow, lg) reads unit 4c + lg of row n0 + lrow. Rows past the
        //    block or the matrix, units past K and chunks past the wave's read
        //    zeros.
        const bool lrow_ok = n0 + lrow < r_hi && rg < sh.n_rg;
        uint32_t w[D][NMAT][BITS];
        auto fetch = [&](int j, uint32_t (&dw)[NMAT][BITS]) {
            const int c = ks + sh.ks * j;
            const int u = 4 * c + lg;
            const uint32_t woff = (j < nj && lrow_ok && u < units)
                ? (uint32_t)(n0 + lrow) * row_bytes + (uint32_t)u * (4 * BITS) : OOB;
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
                buffer_words<BITS>(rw[t], woff, dw[t]);
        };
        static_for<D>([&](auto J) {
            fetch(J, w[J]);
            __builtin_amdgcn_sched_barrier(0);
        });
        // The DMA (issued first) has landed once at most the ring's loads are
        // outstanding.
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(D * NMAT * skinny_loads_per_unit<BITS>()) : "memory");
#pragma unroll
        for (int i = 0; i < kSkinnyXPieces; ++i)
            asm volatile("" :: "v"(xo[i]));
#pragma unroll
        for (int i = 0; i < 4 * NMAT; ++i)
            asm volatile("" :: "v"(so[i]));
        __syncthreads();

        // 3b. Group sums: the lanes of one group (gs / 8 of them) each take 8
        //     activations with dot2 and meet in a butterfly; the group's first
        //     lane writes xg[group * mt + m].
        {
            using PX = RowStreamPairSk<DT>;
            const int lpg = a.gs / 8;
            for (int i = 0; i < per_wave; ++i) {
                const int q = wave + nwaves * i;
                if (q < pieces) {
                    const int m = q / ppr, part = q % ppr;
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
                        table + (uint32_t)m * (uint32_t)sh.row_stride + (uint32_t)part * 1024u + (uint32_t)lane * 16u);
                    float sum = PX::dot(v.x, 0.0f);
                    sum = PX::dot(v.y, sum);
                    sum = PX::dot(v.z, sum);
                    sum = PX::dot(v.w, sum);
                    for (int off = 1; off < lpg; off <<= 1)
                        sum += __shfl_xor(sum, off, 64);
                    const uint32_t k0 = (uint32_t)part * 512u + (uint32_t)lane * 8u;
                    if (lane % lpg == 0 && k0 < (uint32_t)(NC * 128))
                        reinterpret_cast<float*>(xg)[(k0 / (uint32_t)a.gs) * (uint32_t)sh.mt + (uint32_t)m] = sum;
                }
            }
        }
        __syncthreads();

        // 4. Stream the chunks.
        f32x4_t acc[NMAT][MP];
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
            for (int p = 0; p < MP; ++p)
                acc[t][p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        auto process = [&](int j, const uint32_t (&dw)[NMAT][BITS]) {
            __builtin_amdgcn_sched_barrier(0);
            const int c = ks + sh.ks * j;
            const int grp = c * SLOTS + gslot;       // this lane's group slot along K
            uint32_t cp[NMAT][16];
            Orient o[NMAT];
#pragma unroll
            for (int t = 0; t < NMAT; ++t) {
                uint32_t wo[BITS];
#pragma unroll
                for (int i = 0; i < BITS; ++i)
                    wo[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(bp_addr, (int)dw[t][i]);
                const uint32_t e = (uint32_t)r16 * groups_row + (uint32_t)grp;
                const St sv = reinterpret_cast<const St*>(sbg + (uint32_t)(2 * t) * sb_arr)[e];
                const St bv = reinterpret_cast<const St*>(sbg + (uint32_t)(2 * t + 1) * sb_arr)[e];
                o[t] = orient<BITS>(E::to_f32(sv), E::to_f32(bv));
                natural_pairs<BITS, DT>(wo, o[t].flip, cp[t]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < MP; ++p) {
                // Operand A: row i = r16 of A is activation row p MS + i % MS of
                // group slot i / MS; a lane whose slot is not its unit's reads
                // the zero fragment.
                const int m = p * MS + (r16 % MS);
                const bool match = (r16 / MS) == gslot;
                const char* ab = match
                    ? table + (uint32_t)m * (uint32_t)sh.row_stride +
                          (uint32_t)(32 * (4 * c + g)) * 2u
                    : zero;
                const int astep = match ? 16 : 0;
                frag_t af[4];
#pragma unroll
                for (int im = 0; im < 4; ++im)
                    af[im] = *reinterpret_cast<const frag_t*>(ab + im * astep);
                // This lane's four output rows: activation rows
                // p MS + (4 g + r) % MS of its own group slot.
                const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(
                    xg + ((uint32_t)grp * (uint32_t)sh.mt + (uint32_t)(p * MS + (4 * g) % MS)) * 4u);
#pragma unroll
                for (int t = 0; t < NMAT; ++t) {
                    f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int im = 0; im < 4; ++im)
                        d = M16::mma(af[im],
                                     __builtin_bit_cast(frag_t, u32x4_t{cp[t][4 * im], cp[t][4 * im + 1],
                                                                         cp[t][4 * im + 2], cp[t][4 * im + 3]}),
                                     d);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[t][p][r] = __builtin_fmaf(o[t].s, d[r], __builtin_fmaf(o[t].b, xs[r], acc[t][p][r]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int j0 = 0; j0 < nj; j0 += D) {
            static_for<D>([&](auto J) {
                const int j = j0 + (int)J;
                if (j < nj) {
                    process(j, w[J]);
                    fetch(j + D, w[J]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
        }

        // 5. Group slots of one activation row meet (lanes g apart), then the
        //    K-split waves meet in LDS (over the table, which every wave is
        //    done with).
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
            for (int p = 0; p < MP; ++p)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = acc[t][p][r];
                    if constexpr (SLOTS == 4)
                        v += __shfl_xor(v, 16, 64);
                    if constexpr (SLOTS >= 2)
                        v += __shfl_xor(v, 32, 64);
                    acc[t][p][r] = v;
                }
        __syncthreads();
        if (sh.ks > 1) {
            if (ks != 0) {
#pragma unroll
                for (int t = 0; t < NMAT; ++t)
#pragma unroll
                    for (int p = 0; p < MP; ++p)
                        *reinterpret_cast<f32x4_t*>(lds + ((uint32_t)((wave * NMAT + t) * MP + p) * 64u +
                                                           (uint32_t)lane) * 16u) = acc[t][p];
            }
            __syncthreads();
            if (ks == 0) {
                for (int k2 = 1; k2 < sh.ks; ++k2) {
#pragma unroll
                    for (int t = 0; t < NMAT; ++t)
#pragma unroll
                        for (int p = 0; p < MP; ++p)
                            acc[t][p] += *reinterpret_cast<const f32x4_t*>(
                                lds + ((uint32_t)(((wave + k2) * NMAT + t) * MP + p) * 64u + (uint32_t)lane) * 16u);
                }
            }
        }

        // 6. Lanes of group slot 0 store: weight row n0 + r16, activation rows
        //    p MS + 4 g + r.
        if (ks == 0 && (4 * g) < MS) {
            const int n = n0 + r16;
#pragma unroll
            for (int p = 0; p < MP; ++p)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = p * MS + 4 * g + r;
                    float v = acc[0][p][r];
                    if constexpr (NMAT == 2)
                        v = silu_f32(acc[0][p][r]) * acc[1][p][r];
                    uint32_t off = OOB;
                    if (m < rows && n < r_hi && rg < sh.n_rg) {
                        const uint32_t pr = a.perm != nullptr ? (uint32_t)a.perm[start + m]
                                                              : (uint32_t)(start + m);
                        off = (pr * (uint32_t)R + (uint32_t)n) * (uint32_t)SB;
                    }
                    buffer_store_elem<DT>(E::from_f32(v), ro, off);
                }
        }
        // Every wave is done with the table and the partial sums before the
        // next tile refills them.
        __syncthreads();
    }
}

} // namespace qp

namespace qp {

// Group slots per 128-k chunk for a group size, and the passes that cover
// `rows` activation rows (1, 2 or 4 passes of 16 / slots rows).
inline int skinny_slots(int gs) { return gs == 128 ? 1 : gs == 64 ? 2 : 4; }
inline int skinny_passes(int rows, int gs)
{
    const int ms = 16 / skinny_slots(gs);
    const int mp = (rows + ms - 1) / ms;
    return mp <= 1 ? 1 : mp <= 2 ? 2 : 4;
}

// Launch one instance (the LDS size is set once per instance).
template <int BITS, int DT, int NMAT, int SLOTS, int MP>
hipError_t skinny_launch_one(const GemvKernelArgs& k, const SkinnyShape& sh, dim3 grid, hipStream_t st)
{
    if constexpr (MP * (16 / SLOTS) > 16) {
        return hipErrorInvalidValue;
    } else {
        static bool attr_set = false;   // per instantiation; set before its first launch
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(
                reinterpret_cast<const void*>(&qgemv_skinny_kernel<BITS, DT, NMAT, SLOTS, MP>),
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSkinnyLdsBytes);
            if (e != hipSuccess)
                return e;
            attr_set = true;
        }
        const int waves = sh.n_rg * sh.ks;
        const uint32_t lds = skinny_lds_bytes(k.K, k.gs, sh.mt, waves, MP, NMAT, sh.ks);
        hipLaunchKernelGGL((qgemv_skinny_kernel<BITS, DT, NMAT, SLOTS, MP>), grid, dim3(64 * waves), lds,
                           st, k, sh);
        return hipGetLastError();
    }
}

template <int BITS, int DT, int NMAT>
hipError_t skinny_launch(const GemvKernelArgs& k, const SkinnyShape& sh, dim3 grid, hipStream_t st)
{
    const int slots = skinny_slots(k.gs), mp = sh.mt / (16 / slots);
    switch (slots * 8 + mp) {
    case 1 * 8 + 1: return skinny_launch_one<BITS, DT, NMAT, 1, 1>(k, sh, grid, st);
    case 2 * 8 + 1: return skinny_launch_one<BITS, DT, NMAT, 2, 1>(k, sh, grid, st);
    case 2 * 8 + 2: return skinny_launch_one<BITS, DT, NMAT, 2, 2>(k, sh, grid, st);
    case 4 * 8 + 1: return skinny_launch_one<BITS, DT, NMAT, 4, 1>(k, sh, grid, st);
    case 4 * 8 + 2: return skinny_launch_one<BITS, DT, NMAT, 4, 2>(k, sh, grid, st);
    case 4 * 8 + 4: return skinny_launch_one<BITS, DT, NMAT, 4, 4>(k, sh, grid, st);
    }
    return hipErrorInvalidValue;
}

// Table rows (a multiple of 16 / slots, at most 16) for `rows` activation
// rows, shrunk until the table of a K-long row fits the LDS; 0 if not even
// one pass fits.
inline int skinny_table_rows(int rows, int64_t K, int gs, int waves, int nmat, int ks)
{
    const int ms = 16 / skinny_slots(gs);
    for (int mp = skinny_passes(rows < 16 ? rows : 16, gs); mp >= 1; mp /= 2)
        if (skinny_lds_bytes(K, gs, mp * ms, waves, mp, nmat, ks) <= kSkinnyLdsBytes)
            return mp * ms;
    return 0;
}

// Dense launch shape: about one block per CU over contiguous row ranges, up to
// 8 waves per block as groups of 16 rows times waves along K.
inline void skinny_dense_shape(int64_t N, int64_t K, int mt, SkinnyShape* sh, dim3* grid)
{
    const int64_t nrg = (N + 15) / 16;
    const int nc = (int)((K + 127) / 128);
    int64_t blocks;
    int rows;
    if (nrg >= 256) {
        blocks = 256;
        rows = (int)((N + 255) / 256);
        if ((rows + 15) / 16 > kSkinnyMaxWaves) {
            rows = 16 * kSkinnyMaxWaves;
            blocks = (N + rows - 1) / rows;
        }
    } else {
        blocks = nrg;
        rows = 16;
    }
    sh->rows_per_block = rows;
    sh->n_rg = (rows + 15) / 16;
    int ks = kSkinnyMaxWaves / sh->n_rg;
    ks = ks < 1 ? 1 : (ks > nc ? nc : ks);
    sh->ks = ks;
    sh->mt = mt;
    sh->row_stride = skinny_row_stride(K);
    *grid = dim3((unsigned)blocks, 1);
}

} // namespace qp
