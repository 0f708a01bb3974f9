// gemv_core.hpp — the streaming GEMV kernel shared by the dense decode path
// (qgemv.hip) and the MoE path (moe.hip).
//
// Product (emily lib/emily/quantization.ex, `quantized_matmul/2` and
// `dequantize_defn/1` docs): out[m, r] = sum_k x[m, k] * (q[r, k] * s'[r, g]
// + b'[r, g]), g = k / gs, codes packed LSB-first in each row's u32 stream.
// MoE form (ferrum-kernels src/stacked_expert.rs, `gemv_moe_id_batched`
// docs): activation row m of a tile is pair p's row a + (p/top_k)*outer +
// (p%top_k)*inner, the weights are expert e's slice of the stacked tensor, and
// the result goes to out[p, r]. The dense product is the special case of one
// tile holding pairs 0..M-1 with top_k = 1, outer = K, inner = 0.
//
// Design (HBM-bound at small M):
//  - a row is spread over KL lanes (a power of two); each lane owns U units of
//    32 codes (U*bits consecutive words) and keeps the tile's activations for
//    that K-slice in registers for every row it visits, so activations are read
//    once per block and weights once per tile;
//  - weight words come in as 128/64/32-bit non-temporal loads; the next row's
//    words are requested before the current row is computed and reduced;
//  - the affine map is folded out of the inner loop:
//      sum_k x w' = sum_groups s' * (sum q x) + b' * (sum x),
//    with each unit's sum x computed once in the prologue and the group's
//    bias taken at the end of the grid nearer zero (codepair.hpp, `orient`);
//  - activations are held as fp32 and every code is converted exactly and
//    accumulated with an fp32 FMA (this kernel serves fp32 activations, 3- and
//    6-bit codes and MoE tiles of a few pairs; the 2-, 4- and 8-bit decode
//    with 16-bit activations runs on the row kernels);
//  - partial sums are reduced across a row's lanes with cross-lane shuffles,
//    through LDS when a row spans more than one wave;
//  - NMAT = 2 streams a gate and an up matrix together and writes
//    SiLU(gate) * up (ferrum-kernels `gemv_moe_id_gate_up_silu` docs).
#pragma once

#include "codepair.hpp"
#include "common.hpp"

namespace qp {

// Largest tile height (activation rows per launch) the register budget allows:
// activations take MT * 32 * U VGPRs (fp32) for U <= 2 units of 32 codes per
// lane.
template <int BITS, int DT>
constexpr int gemv_max_mt()
{
    return 2;
}

constexpr int GEMV_THREADS = 256;

// Activations of one 32-code unit as fp32, and their sum: one exact code
// conversion and one FMA per code.
template <int BITS, int DT> struct UnitX {
    float xf[32];
    float xsum;

    __device__ __forceinline__ void load(const float (&xv)[32])
    {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            xf[c] = xv[c];
            s += xv[c];
        }
        xsum = s;
    }

    // acc + sum over the unit's 32 codes of q * x, each code complemented
    // (q -> 2^BITS - 1 - q) when flip is ~0.
    __device__ __forceinline__ float qdot(const uint32_t* w, uint32_t flip, float acc) const
    {
        uint32_t wf[BITS];
#pragma unroll
        for (int i = 0; i < BITS; ++i)
            wf[i] = w[i] ^ flip;
        static_for<32>([&](auto C) {
            acc = __builtin_fmaf((float)unit_code<BITS, C>(wf), xf[C], acc);
        });
        return acc;
    }
};

// Arguments of the streaming kernel. Element pointers are raw storage.
struct GemvKernelArgs {
    const void* x;           // activations
    int64_t top_k, outer, inner; // pair p's row: x + (p/top_k)*outer + (p%top_k)*inner
    const int32_t* perm;     // pair list (nullptr: identity)
    const TileDesc* tiles;   // tiles (nullptr: see `ids`)
    const int32_t* n_tiles;  // device tile count (with `tiles`)
    const int32_t* ids;      // without `tiles`: tile t is pair t alone, of expert ids[t]
                             // (ids outside [0, E) skip their pair); both null: one
                             // tile of pairs 0..M-1, expert 0
    int n_pairs, n_experts;  // with `ids`
    int M;                   // pairs of the single tile when tiles == nullptr
    const uint32_t* wq[2];   // [E, R, K*bits/32]
    const void* scales[2];   // [E, R, K/gs]
    const void* biases[2];
    int64_t R, K;            // rows per expert, input features
    int gs;
    int KL;                  // lanes per row
    void* out;               // [pairs, R]
    uint32_t out_bytes;      // size of `out` in bytes (< 2^31)
    uint32_t x_bytes;        // bytes of activations reachable from `x` (< 2^31; read
                             // by the matrix-core kernel's table DMA)
};

// Tiles of a launch and tile t's expert, first pair slot and pair count;
// false when tile t has nothing to compute (a pair with an invalid id).
__device__ __forceinline__ int gemv_num_tiles(const GemvKernelArgs& a)
{
    return a.tiles != nullptr ? *a.n_tiles : a.ids != nullptr ? a.n_pairs : 1;
}
__device__ __forceinline__ bool gemv_tile(const GemvKernelArgs& a, int tile, int& expert,
                                          int& start, int& count)
{
    if (a.tiles != nullptr) {
        const TileDesc d = a.tiles[tile];
        expert = d.expert;
        start = d.start;
        count = d.count;
        return true;
    }
    if (a.ids != nullptr) {
        expert = a.ids[tile];
        start = tile;
        count = 1;
        return expert >= 0 && expert < a.n_experts;
    }
    expert = 0;
    start = 0;
    count = a.M;
    return true;
}

// Buffer resource over `bytes` bytes at `p` (raw, untyped). Loads past the end
// return zeros and stores past the end are dropped, which is what lets the
// kernels below run without bounds branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// Byte offset that is always past the end of a resource (its stores drop).
constexpr uint32_t OOB = 0x80000000u;

// Cache policy for weight codes read once per launch (sc0 | nt): the loads
// skip the L1 and stream through the L2 without displacing reused lines
// (activations, scales). Taken where it measured faster: the one-row stream
// at 2, 3, 4 and 6 bits (4-bit 14336 x 4096: 10.05 -> 9.84 us; 2-bit:
// 10.1 -> 9.8 us; cross-word 4096 x 4096: 7.6 -> 7.1 us). The 8-bit one-row
// stream (14.5 -> 20.1 us), two rows and the matrix-core tiles were slower
// with it and keep the default policy.
constexpr int kStreamPolicy = 3;

template <int NW, int POLICY = 0>
__device__ __forceinline__ void buffer_words(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                             uint32_t (&w)[NW])
{
    if constexpr (NW == 3) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, POLICY);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
    } else if constexpr (NW == 6) {
        const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
        const u32x2_t u = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off + 16, 0, POLICY));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        w[4] = u.x; w[5] = u.y;
    } else if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW; i += 4) {
            const u32x4_t v = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * i, 0, POLICY));
            w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
        }
    } else if constexpr (NW % 2 == 0) {
#pragma unroll
        for (int i = 0; i < NW; i += 2) {
            const u32x2_t v = __builtin_bit_cast(
                u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off + 4 * i, 0, POLICY));
            w[i] = v.x; w[i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i)
            w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, POLICY);
    }
}

template <int DT>
__device__ __forceinline__ typename Elem<DT>::storage buffer_elem(__amdgpu_buffer_rsrc_t r,
                                                                  uint32_t off)
{
    if constexpr (DT == DT_F32)
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    else
        return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

template <int DT>
__device__ __forceinline__ void buffer_store_elem(typename Elem<DT>::storage v,
                                                  __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    if constexpr (DT == DT_F32)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

// Activation words per unit in the block's table: fp32 values.
template <int BITS, int DT>
constexpr int unit_table_words()
{
    return 32;
}

// Ring depth that fits the register budget of a kernel instance: activation
// registers (pairs or fp32 values per unit, two sums per group) plus D ring
// slots of weight words and scale/bias values, plus about 40 for addressing
// and accumulators.
template <int BITS, int DT, int MT, int U, int G, int NMAT, int BUDGET>
constexpr int ring_depth()
{
    const int per_unit = 40; // 32 fp32 values and conversion temporaries
    const int xr = MT * U * per_unit + MT * G * 2;
    const int slot = NMAT * (U * BITS + 2 * G);
    for (int d = 4; d > 1; --d)
        if (xr + d * slot + 56 + 8 * MT <= BUDGET)
            return d;
    return 1;
}

// One wave streams whole rows: a row is spread over KL lanes (KL a power of
// two <= 64), so a wave covers RPW = 64 / KL rows per pass. Waves take passes
// p = gw, gw + GW, ... (gw = global wave id, GW = waves along the grid's x).
// Each lane owns U units of 32 codes; they fall into G groups (G = 1 when the
// whole slice lies in one quantization group, else G = U).
//
//  1. The block prepares the tile's activation table (fp32 activations and
//     their sums for every lane slot and activation row) in LDS, each
//     thread one (row, unit, lane slot) item, so the conversion work is done
//     once per block rather than once per wave.
//  2. Every wave keeps D passes of weight words in flight (a ring refilled as
//     it is consumed). The activation loads are issued first and the ring
//     right after, so waiting for the activations never waits for weights.
//  3. All loads and stores are raw buffer accesses: rows past the end read
//     zeros and their stores are dropped, so the loop has no bounds branches
//     and the compiler's memory-counter waits cover exactly one ring slot.
//  4. The D slots' partial sums are reduced together (interleaved DPP steps)
//     and stored at the end of each ring cycle.
template <int BITS, int DT, int MT, int U, int G, int KL, int NMAT, int MAXT>
__global__ __launch_bounds__(MAXT) void qgemv_stream_kernel(GemvKernelArgs a)
{
    using E = Elem<DT>;
    using St = typename E::storage;
    using UX = UnitX<BITS, DT>;
    static_assert(G == 1 || G == U, "a lane slice is one group or one group per unit");
    constexpr int UPG = U / G;                              // units per group
    constexpr int D = ring_depth<BITS, DT, MT, U, G, NMAT, (131072 / MAXT < 512 ? 131072 / MAXT : 512)>();
    constexpr int NW = U * BITS;
    constexpr int RPW = 64 / KL;
    constexpr int NP = unit_table_words<BITS, DT>();        // table words per unit
    constexpr int UWORDS = NP + 1;                          // + the unit's sum
    constexpr int ITEMS = MT * U * KL;                      // table items per tile
    constexpr int XV = 32 * (int)sizeof(St) / 16;           // 16-byte vectors per unit
    constexpr int SB = (int)sizeof(St);
    __shared__ uint32_t table[MT * U * UWORDS * KL];       // [m][u][word][kl]

    const int lane = threadIdx.x & 63;
    const int kl = lane & (KL - 1);
    const int sub = lane / KL;
    const uint32_t row_bytes = (uint32_t)(a.K * BITS / 8);
    const uint32_t groups_row = (uint32_t)(a.K / a.gs);
    const int R = (int)a.R;
    const int nthreads = (int)blockDim.x; // a multiple of 64, >= 256, <= MAXT
    const int gw = (int)blockIdx.x * (nthreads / 64) + (int)(threadIdx.x / 64);
    const int GW = (int)gridDim.x * (nthreads / 64);
    const int passes = (R + RPW - 1) / RPW;
    uint32_t sboff[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        sboff[g] = (uint32_t)(((kl * U + g * UPG) * 32) / a.gs) * SB;
    const St* xs = static_cast<const St*>(a.x);

    const int ntiles = gemv_num_tiles(a);
    for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
        int expert, start, count;
        if (!gemv_tile(a, tile, expert, start, count))
            continue;   // uniform over the block
        int64_t pair[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            int64_t p = -1;
            if (m < count)
                p = a.perm != nullptr ? (int64_t)a.perm[start + m] : (int64_t)(start + m);
            pair[m] = p;
        }

        // 1a. Activation loads for this thread's table items (clamped so every
        //     thread issues the same loads; only in-range items are stored).
        constexpr int IPT = (ITEMS + 255) / 256;
        u32x4_t xraw[IPT][XV];
        bool it_live[IPT];
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            int item = (int)threadIdx.x + i * nthreads;
            item = item < ITEMS ? item : ITEMS - 1;
            const int it_kl = item % KL, it_u = (item / KL) % U, it_m = item / (KL * U);
            int64_t it_pair = pair[0];
            bool live = false;
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (m == it_m && pair[m] >= 0) {
                    it_pair = pair[m];
                    live = true;
                }
            it_live[i] = live;
            const St* xrow = xs + (it_pair / a.top_k) * a.outer + (it_pair % a.top_k) * a.inner;
            const u32x4_t* p =
                reinterpret_cast<const u32x4_t*>(xrow + (int64_t)(it_kl * U + it_u) * 32);
#pragma unroll
            for (int v = 0; v < XV; ++v)
                xraw[i][v] = p[v];
        }

        // 2. The weight ring.
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
        const uint32_t lane_off = (uint32_t)(kl * NW * 4);
        uint32_t w[D][NMAT][NW];
        St sv[D][NMAT][G], bv[D][NMAT][G];
        auto fetch = [&](int p, uint32_t (&dw)[NMAT][NW], St (&ds)[NMAT][G],
                         St (&db)[NMAT][G]) {
            const uint32_t r = (uint32_t)(p * RPW + sub);
#pragma unroll
            for (int t = 0; t < NMAT; ++t) {
                buffer_words<NW, (MT == 1 && BITS != 8) ? kStreamPolicy : 0>(
                    rw[t], r * row_bytes + lane_off, dw[t]);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    ds[t][g] = buffer_elem<DT>(rs[t], r * groups_row * SB + sboff[g]);
                    db[t][g] = buffer_elem<DT>(rb[t], r * groups_row * SB + sboff[g]);
                }
            }
        };
        // Scheduling barriers keep each ring slot's loads together and in slot
        // order, here and in the stream loop: if the scheduler sinks a slot's
        // scale/bias loads behind later slots, the memory-counter wait before
        // that slot's use has to drain nearly the whole ring.
        __builtin_amdgcn_sched_barrier(0);
        static_for<D>([&](auto J) {
            fetch(gw + J * GW, w[J], sv[J], bv[J]);
            __builtin_amdgcn_sched_barrier(0);
        });

        // 1b. Build the table items and share them through LDS.
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int item = (int)threadIdx.x + i * nthreads;
            const int it_kl = item % KL, it_u = (item / KL) % U, it_m = item / (KL * U);
            float xv[32];
            const St* e = reinterpret_cast<const St*>(&xraw[i][0]);
            const bool live = it_live[i];
            static_for<32>([&](auto C) { xv[C] = live ? E::to_f32(e[C]) : 0.f; });
            UX ux;
            ux.load(xv);
            if (item < ITEMS) {
                uint32_t* dst = table + ((it_m * U + it_u) * UWORDS) * KL + it_kl;
                static_for<32>([&](auto C) {
                    dst[C * KL] = __builtin_bit_cast(uint32_t, ux.xf[C]);
                });
                dst[NP * KL] = __builtin_bit_cast(uint32_t, ux.xsum);
            }
        }
        __syncthreads();
        UX ux[MT][U];
        float gsum[MT][G];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int g = 0; g < G; ++g)
                gsum[m][g] = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t* src = table + ((m * U + u) * UWORDS) * KL + kl;
                static_for<32>([&](auto C) {
                    ux[m][u].xf[C] = __builtin_bit_cast(float, src[C * KL]);
                });
                gsum[m][u / UPG] += __builtin_bit_cast(float, src[NP * KL]);
            }
        }

        // Output resource; non-writer lanes store out of range (dropped).
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out, a.out_bytes);
        const bool writer = segment_writer(kl, KL);

        // 3. Stream.
        for (int p0 = gw; p0 < passes; p0 += D * GW) {
            float acc[D][NMAT][MT];
            static_for<D>([&](auto J) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < NMAT; ++t) {
                    Orient o[G];
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        o[g] = orient<BITS>(E::to_f32(sv[J][t][g]), E::to_f32(bv[J][t][g]));
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        float r = 0.f;
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            float c = 0.f;
#pragma unroll
                            for (int u = g * UPG; u < (g + 1) * UPG; ++u)
                                c = ux[m][u].qdot(w[J][t] + u * BITS, o[g].flip, c);
                            r = __builtin_fmaf(o[g].s, c, __builtin_fmaf(o[g].b, gsum[m][g], r));
                        }
                        acc[J][t][m] = r;
                    }
                }
                fetch(p0 + (J + D) * GW, w[J], sv[J], bv[J]);
                __builtin_amdgcn_sched_barrier(0);
            });
            // 4. Reduce the D slots together, then store.
            reduce_slots<D * NMAT * MT, KL>(&acc[0][0][0]);
            static_for<D>([&](auto J) {
                const int row = (p0 + J * GW) * RPW + sub;
                const bool ok = writer && row < R && p0 + J * GW < passes;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    float v = acc[J][0][m];
                    if constexpr (NMAT == 2)
                        v = silu_f32(acc[J][0][m]) * acc[J][1][m];
                    const uint32_t off = (ok && pair[m] >= 0)
                        ? (uint32_t)((pair[m] * a.R + row) * SB) : OOB;
                    buffer_store_elem<DT>(E::from_f32(v), ro, off);
                }
            });
        }
        __syncthreads(); // the table is rebuilt for the next tile
    } // tiles
}

// Lanes per row for slices of U units; 0 unless K splits into a power-of-two
// lane count that fits one wave.
inline int gemv_lanes_per_row(int64_t K, int U)
{
    if (K <= 0 || K % (32 * U) != 0)
        return 0;
    int64_t kl = K / (32 * U);
    if (kl < 1 || kl > 64 || (kl & (kl - 1)) != 0)
        return 0;
    return (int)kl;
}

// Fallback for any K (multiple of 32) and tiles of up to 16 pairs: one wave per
// row, lanes stride over the row's units, activations read per unit; each code
// is dequantized (q * s' + b') and accumulated in fp32.
template <int BITS, int DT, int NMAT>
__global__ __launch_bounds__(256) void qgemv_generic_kernel(GemvKernelArgs a)
{
    using E = Elem<DT>;
    using St = typename E::storage;
    const int ntiles = gemv_num_tiles(a);
    for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
    int expert, start, count;
    if (!gemv_tile(a, tile, expert, start, count))
        continue;   // uniform over the block
    const int lane = threadIdx.x & 63;
    const int64_t K = a.K, R = a.R;
    const int64_t units = K / 32, words_row = K * BITS / 32, groups_row = K / a.gs;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / 64);
    const St* xs = static_cast<const St*>(a.x);
    const St* xrow[16];
    int64_t pair[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        pair[m] = -1;
        xrow[m] = nullptr;
        if (m < count) {
            pair[m] = a.perm != nullptr ? (int64_t)a.perm[start + m] : (int64_t)(start + m);
            xrow[m] = xs + (pair[m] / a.top_k) * a.outer + (pair[m] % a.top_k) * a.inner;
        }
    }
    St* outs = static_cast<St*>(a.out);
    for (int64_t row = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64; row < R;
         row += nwaves) {
        float acc[NMAT][16];
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
            for (int m = 0; m < 16; ++m)
                acc[t][m] = 0.f;
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            const int64_t rr = (int64_t)expert * R + row;
            const uint32_t* wrow = a.wq[t] + rr * words_row;
            const St* srow = static_cast<const St*>(a.scales[t]) + rr * groups_row;
            const St* brow = static_cast<const St*>(a.biases[t]) + rr * groups_row;
            for (int64_t u = lane; u < units; u += 64) {
                uint32_t w[BITS];
#pragma unroll
                for (int i = 0; i < BITS; ++i)
                    w[i] = wrow[u * BITS + i];
                const int64_t g = (u * 32) / a.gs;
                const float s = E::to_f32(srow[g]);
                const float b = E::to_f32(brow[g]);
                static_for<32>([&](auto C) {
                    const float wv = affine_weight((float)unit_code<BITS, C>(w), s, b);
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        if (m < count)
                            acc[t][m] = __builtin_fmaf(E::to_f32(xrow[m][u * 32 + C]), wv,
                                                       acc[t][m]);
                });
            }
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            if (m < count) {
                float v = segment_sum<64>(acc[0][m]);
                if constexpr (NMAT == 2)
                    v = silu_f32(v) * segment_sum<64>(acc[1][m]);
                if (lane == 0)
                    outs[pair[m] * R + row] = E::from_f32(v);
            }
        }
    }
    } // tiles
}

} // namespace qp
