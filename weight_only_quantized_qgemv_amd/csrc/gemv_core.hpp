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
//      sum_k x w' = sum_units s' * (sum q x) + b' * (sum x),
//    with each unit's sum x computed once in the prologue;
//  - 16-bit activations: codes are OR-ed into the mantissa of 128.0 (bf16) or
//    1024.0 (fp16), two per register, and fed to v_dot2 with pre-scaled
//    activation pairs (unpack_plan.hpp); fp32 activations and 8-bit codes with
//    bf16 use per-code conversion and fp32 FMA;
//  - partial sums are reduced across a row's lanes with cross-lane shuffles,
//    through LDS when a row spans more than one wave;
//  - NMAT = 2 streams a gate and an up matrix together and writes
//    SiLU(gate) * up (ferrum-kernels `gemv_moe_id_gate_up_silu` docs).
#pragma once

#include "common.hpp"
#include "unpack_plan.hpp"

namespace qp {

template <int DT> struct Dot2Traits;
template <> struct Dot2Traits<DT_BF16> {
    static constexpr int MANT = 7;
    static constexpr uint32_t MAGIC2 = 0x43004300u; // 128.0 in both bf16 halves
    static constexpr float MAGIC = 128.0f;
    using pair_t = bf16x2_t;
    static __device__ __forceinline__ float dot(uint32_t v, pair_t x, float acc)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v), x, acc, false);
    }
    static __device__ __forceinline__ pair_t make(float lo, float hi)
    {
        return pair_t{(__bf16)lo, (__bf16)hi};
    }
    static __device__ __forceinline__ float lo_f(pair_t p) { return (float)p.x; }
    static __device__ __forceinline__ float hi_f(pair_t p) { return (float)p.y; }
};
template <> struct Dot2Traits<DT_F16> {
    static constexpr int MANT = 10;
    static constexpr uint32_t MAGIC2 = 0x64006400u; // 1024.0 in both fp16 halves
    static constexpr float MAGIC = 1024.0f;
    using pair_t = f16x2_t;
    static __device__ __forceinline__ float dot(uint32_t v, pair_t x, float acc)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, v), x, acc, false);
    }
    static __device__ __forceinline__ pair_t make(float lo, float hi)
    {
        return pair_t{(_Float16)lo, (_Float16)hi};
    }
    static __device__ __forceinline__ float lo_f(pair_t p) { return (float)p.x; }
    static __device__ __forceinline__ float hi_f(pair_t p) { return (float)p.y; }
};

// Whether (BITS, DT) takes the dot2 path.
template <int BITS, int DT>
constexpr bool use_dot2()
{
    if constexpr (DT == DT_F32)
        return false;
    else
        return make_unpack_plan(BITS, Dot2Traits<DT>::MANT).feasible;
}

// Largest tile height (activation rows per launch) the register budget allows.
template <int BITS, int DT>
constexpr int gemv_max_mt()
{
    return use_dot2<BITS, DT>() ? 8 : 2;
}

constexpr int GEMV_THREADS = 256;

template <int BITS, int DT, bool DOT2> struct UnitX;

// Activations of one 32-code unit for the dot2 path: pre-scaled pairs, the
// magic-offset sum and the plain sum.
template <int BITS, int DT> struct UnitX<BITS, DT, true> {
    using T = Dot2Traits<DT>;
    static constexpr UnpackPlan P = make_unpack_plan(BITS, T::MANT);
    typename T::pair_t xp[P.n_pair];
    float xoff, xsum;

    __device__ __forceinline__ void load(const float (&xv)[32])
    {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 32; ++c)
            s += xv[c];
        xsum = s;
        float off = 0.f;
#pragma unroll
        for (int j = 0; j < P.n_pair; ++j) {
            const PlanPair pp = P.pair[j];
            float lo = pp.lo >= 0 ? xv[pp.lo] * (1.0f / float(1 << pp.lo_off)) : 0.f;
            float hi = pp.hi >= 0 ? xv[pp.hi] * (1.0f / float(1 << pp.hi_off)) : 0.f;
            xp[j] = T::make(lo, hi);
            off += T::lo_f(xp[j]) + T::hi_f(xp[j]);
        }
        xoff = off * T::MAGIC;
    }

    // Sum over the unit's 32 codes of q * x.
    __device__ __forceinline__ float qdot(const uint32_t* w) const
    {
        uint32_t win[P.n_win];
#pragma unroll
        for (int i = 0; i < P.n_win; ++i) {
            const int wb = P.win_bit[i], wi = wb / 32, sh = wb % 32;
            if (sh == 0)
                win[i] = w[wi];
            else if (wi + 1 < BITS)
                win[i] = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh);
            else
                win[i] = w[wi] >> sh;
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < P.n_pair; ++j) {
            const PlanPair pp = P.pair[j];
            constexpr uint32_t cm = (1u << BITS) - 1u;
            const uint32_t mask = (pp.lo >= 0 ? cm << pp.lo_off : 0u) |
                                  (pp.hi >= 0 ? cm << (16 + pp.hi_off) : 0u);
            const uint32_t v = (win[pp.win] & mask) | T::MAGIC2;
            acc = T::dot(v, xp[j], acc);
        }
        return acc - xoff;
    }
};

// fp32 path: activations as fp32, one conversion and one FMA per code.
template <int BITS, int DT> struct UnitX<BITS, DT, false> {
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

    __device__ __forceinline__ float qdot(const uint32_t* w) const
    {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < 32; ++c)
            acc = __builtin_fmaf((float)unit_code<BITS>(w, c), xf[c], acc);
        return acc;
    }
};

// Work description of one tile: `count` (<= MT) pairs of one expert, taken
// from positions [start, start + count) of the pair list.
struct TileDesc {
    int expert;
    int start;
    int count;
};

// Arguments of the streaming kernel. Element pointers are raw storage.
struct GemvKernelArgs {
    const void* x;           // activations
    int64_t top_k, outer, inner; // pair p's row: x + (p/top_k)*outer + (p%top_k)*inner
    const int32_t* perm;     // pair list (nullptr: identity)
    const TileDesc* tiles;   // tiles (nullptr: one tile of pairs 0..M-1, expert 0)
    const int32_t* n_tiles;  // device tile count (with `tiles`)
    int M;                   // pairs of the single tile when tiles == nullptr
    const uint32_t* wq[2];   // [E, R, K*bits/32]
    const void* scales[2];   // [E, R, K/gs]
    const void* biases[2];
    int64_t R, K;            // rows per expert, input features
    int gs;
    int KL;                  // lanes per row
    void* out;               // [pairs, R]
};

__device__ __forceinline__ float silu_f32(float z)
{
    return z / (1.0f + expf(-z));
}

template <int BITS, int DT, int MT, int U, int NMAT>
__global__ __launch_bounds__(GEMV_THREADS) void qgemv_stream_kernel(GemvKernelArgs a)
{
    using E = Elem<DT>;
    using St = typename E::storage;
    constexpr bool DOT2 = use_dot2<BITS, DT>();
    constexpr int NW = U * BITS;
    __shared__ float red[GEMV_THREADS / 64][NMAT][MT];

    // Tiles: blocks stride over them along y (block-uniform bounds, so every
    // barrier below is reached by the whole block).
    const int ntiles = a.tiles != nullptr ? *a.n_tiles : 1;
    for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
    int expert = 0, start = 0, count = a.M;
    if (a.tiles != nullptr) {
        const TileDesc d = a.tiles[tile];
        expert = d.expert;
        start = d.start;
        count = d.count;
    }

    const int KL = a.KL;
    const int tid = threadIdx.x;
    const int kl = tid & (KL - 1);
    const int slot = tid / KL;
    const int RP = GEMV_THREADS / KL;
    const int64_t K = a.K, R = a.R;
    const int64_t words_row = K * BITS / 32;
    const int64_t groups_row = K / a.gs;

    int64_t pair[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        int64_t p = -1;
        if (m < count)
            p = a.perm != nullptr ? (int64_t)a.perm[start + m] : (int64_t)(start + m);
        pair[m] = p;
    }

    // Prologue: this lane's activations for every row of the tile.
    UnitX<BITS, DT, DOT2> ux[MT][U];
    const St* xs = static_cast<const St*>(a.x);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const St* xrow = nullptr;
        if (pair[m] >= 0)
            xrow = xs + (pair[m] / a.top_k) * a.outer + (pair[m] % a.top_k) * a.inner;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float xv[32];
            const int64_t k0 = ((int64_t)kl * U + u) * 32;
#pragma unroll
            for (int c = 0; c < 32; ++c)
                xv[c] = xrow != nullptr ? E::to_f32(xrow[k0 + c]) : 0.f;
            ux[m][u].load(xv);
        }
    }
    int64_t gidx[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        gidx[u] = (((int64_t)kl * U + u) * 32) / a.gs;

    const uint32_t* wbase[NMAT];
    const St* sbase[NMAT];
    const St* bbase[NMAT];
#pragma unroll
    for (int t = 0; t < NMAT; ++t) {
        wbase[t] = a.wq[t] + (int64_t)expert * R * words_row + (int64_t)kl * NW;
        sbase[t] = static_cast<const St*>(a.scales[t]) + (int64_t)expert * R * groups_row;
        bbase[t] = static_cast<const St*>(a.biases[t]) + (int64_t)expert * R * groups_row;
    }

    const int64_t stride_rows = (int64_t)gridDim.x * RP;
    int64_t row = (int64_t)blockIdx.x * RP + slot;

    uint32_t w[NMAT][NW];
    St sv[NMAT][U], bv[NMAT][U];
    auto fetch = [&](int64_t r, uint32_t (&dw)[NMAT][NW], St (&ds)[NMAT][U], St (&db)[NMAT][U]) {
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            load_words<NW>(wbase[t] + r * words_row, dw[t]);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                ds[t][u] = sbase[t][r * groups_row + gidx[u]];
                db[t][u] = bbase[t][r * groups_row + gidx[u]];
            }
        }
    };
    if (row < R)
        fetch(row, w, sv, bv);

    St* outs = static_cast<St*>(a.out);
    for (int64_t base = (int64_t)blockIdx.x * RP; base < R; base += stride_rows) {
        const int64_t nrow = row + stride_rows;
        uint32_t wn[NMAT][NW];
        St svn[NMAT][U], bvn[NMAT][U];
        if (nrow < R)
            fetch(nrow, wn, svn, bvn);

        float acc[NMAT][MT];
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                acc[t][m] = 0.f;
        if (row < R) {
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float s = E::to_f32(sv[t][u]), b = E::to_f32(bv[t][u]);
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const float qx = ux[m][u].qdot(w[t] + u * BITS);
                        acc[t][m] =
                            __builtin_fmaf(s, qx, __builtin_fmaf(b, ux[m][u].xsum, acc[t][m]));
                    }
                }
        }
        // Reduce over the KL lanes of the row.
        bool have = false;
        if (KL <= 64) {
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    for (int off = 1; off < KL; off <<= 1)
                        acc[t][m] += __shfl_xor(acc[t][m], off, 64);
            have = kl == 0 && row < R;
        } else {
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    acc[t][m] = segment_sum<64>(acc[t][m]);
            const int wave = tid / 64;
            if ((tid & 63) == 0)
#pragma unroll
                for (int t = 0; t < NMAT; ++t)
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        red[wave][t][m] = acc[t][m];
            __syncthreads();
            if (kl == 0) {
                const int wpr = KL / 64;
#pragma unroll
                for (int t = 0; t < NMAT; ++t)
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        float s = 0.f;
                        for (int i = 0; i < wpr; ++i)
                            s += red[wave + i][t][m];
                        acc[t][m] = s;
                    }
            }
            __syncthreads();
            have = kl == 0 && row < R;
        }
        if (have) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (pair[m] >= 0) {
                    float v = acc[0][m];
                    if constexpr (NMAT == 2)
                        v = silu_f32(acc[0][m]) * acc[1][m];
                    outs[pair[m] * R + row] = E::from_f32(v);
                }
            }
        }
        row = nrow;
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
#pragma unroll
            for (int i = 0; i < NW; ++i)
                w[t][i] = wn[t][i];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                sv[t][u] = svn[t][u];
                bv[t][u] = bvn[t][u];
            }
        }
    }
    } // tiles
}

// Lanes per row for slices of U units; 0 when K does not split into a power of
// two lane count that fits one block.
inline int gemv_lanes_per_row(int64_t K, int U)
{
    if (K <= 0 || K % (32 * U) != 0)
        return 0;
    int64_t kl = K / (32 * U);
    if (kl < 1 || kl > GEMV_THREADS || (kl & (kl - 1)) != 0)
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
    const int ntiles = a.tiles != nullptr ? *a.n_tiles : 1;
    for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
    int expert = 0, start = 0, count = a.M;
    if (a.tiles != nullptr) {
        const TileDesc d = a.tiles[tile];
        expert = d.expert;
        start = d.start;
        count = d.count;
    }
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
#pragma unroll
                for (int c = 0; c < 32; ++c) {
                    const float wv = (float)unit_code<BITS>(w, c) * s + b;
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        if (m < count)
                            acc[t][m] = __builtin_fmaf(E::to_f32(xrow[m][u * 32 + c]), wv,
                                                       acc[t][m]);
                }
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
