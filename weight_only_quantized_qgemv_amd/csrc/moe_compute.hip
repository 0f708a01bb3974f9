// moe_compute.hip — the compute launch of the MoE path over the device-written
// tile list (see moe.hip for the routing). Compiled once per bit width
// (QP_BITS) and per form (QP_NMAT: 1 = plain product, 2 = fused
// SiLU(gate) * up), so the kernel instantiations spread over parallel
// translation units.
#include "gemv_core.hpp"
#include "skinny.hpp"
#include "gemm_core.hpp"
#include "moe_rows.hpp"
#include "launch.hpp"

#if !defined(QP_BITS) || !defined(QP_NMAT)
#error "moe_compute.hip needs QP_BITS and QP_NMAT"
#endif

namespace qp {

namespace {

template <int DT> using St = typename Elem<DT>::storage;

// Grid: y strides over the device-written tiles (bounded by max_tiles), x
// spreads each tile's row passes over waves; about 4096 waves in total.
template <int BITS, int DT, int MT, int U, int KL, int NMAT>
hipError_t run_tiles(GemvKernelArgs k, int64_t max_tiles, hipStream_t st)
{
    constexpr int D = ring_depth<BITS, DT, MT, U, U, NMAT, 512>();
    constexpr int RPW = 64 / KL;
    const int64_t passes = (k.R + RPW - 1) / RPW;
    int64_t gy = max_tiles < 65535 ? max_tiles : 65535;
    if (gy < 1)
        gy = 1;
    int64_t waves = (passes + D - 1) / D;
    const int64_t cap = (4096 + gy - 1) / gy;
    waves = waves < cap ? waves : cap;
    const int64_t gx = (waves + 3) / 4;
    k.KL = KL;
    hipLaunchKernelGGL((qgemv_stream_kernel<BITS, DT, MT, U, U, KL, NMAT, GEMV_THREADS>),
                       dim3((int)gx, (int)gy), dim3(GEMV_THREADS), 0, st, k);
    return hipGetLastError();
}

template <int BITS, int DT, int NMAT>
hipError_t run_generic(GemvKernelArgs k, int64_t max_tiles, hipStream_t st)
{
    int64_t gy = max_tiles < 65535 ? max_tiles : 65535;
    if (gy < 1)
        gy = 1;
    int64_t gx = (k.R + 3) / 4;
    int64_t cap = 4096 / gy;
    cap = cap < 1 ? 1 : cap;
    gx = gx < cap ? gx : cap;
    k.KL = 64;
    hipLaunchKernelGGL((qgemv_generic_kernel<BITS, DT, NMAT>), dim3((int)gx, (int)gy), dim3(256),
                       0, st, k);
    return hipGetLastError();
}

template <int BITS, int DT, int MT, int NMAT>
hipError_t run_mt(GemvKernelArgs k, int64_t max_tiles, hipStream_t st)
{
    // One wave per row at K = 2048.
    if (k.K == 32 * 64)
        return run_tiles<BITS, DT, MT, 1, 64, NMAT>(k, max_tiles, st);
    // Eight rows per wave at K = 768, one pair per tile (two pairs' fp32
    // slices of three units would not fit the registers).
    if constexpr (MT == 1) {
        if (k.K == 3 * 32 * 8)
            return run_tiles<BITS, DT, MT, 3, 8, NMAT>(k, max_tiles, st);
    }
    return run_generic<BITS, DT, NMAT>(k, max_tiles, st);
}

// Matrix-core tiles of up to 16 pairs with exact codes (skinny.hpp): grid x
// over row blocks of the expert's matrix, y over the device-written tiles.
template <int BITS, int DT, int NMAT>
hipError_t run_skinny_tiles(GemvKernelArgs k, int64_t max_tiles, hipStream_t st)
{
    if constexpr (DT == DT_F32) {
        (void)k; (void)max_tiles; (void)st;
        return hipErrorInvalidValue;
    } else {
        int64_t gy = max_tiles < 65535 ? max_tiles : 65535;
        gy = gy < 1 ? 1 : gy;
        SkinnyShape sh{};
        unsigned gx = 0;
        skinny_moe_shape(k.R, k.K, max_tiles, &sh, &gx);
        return skinny_launch<BITS, DT, NMAT>(k, sh, dim3(gx, (unsigned)gy), st);
    }
}

// Routed GEMM (gemm_core.hpp): tiles of BM pairs of one expert times BN / NMAT
// rows of each of its NMAT matrices, four waves side by side along the rows
// (each weight fragment is built by one wave only). The blocks are
// persistent: the grid is the smaller of the largest possible work list
// ((tile, row block) items) and the blocks the GPU holds at once, and each
// block walks its XCD's stretch of the device-written list. Three activation
// stages and four code / scale stages: 64 KB of LDS at 4-bit, so two blocks
// share a CU (four activation stages measured the same).
#ifndef QP_MOE_GEMM_NA
#define QP_MOE_GEMM_NA 3
#endif
#ifndef QP_MOE_GEMM_NC
#define QP_MOE_GEMM_NC 4
#endif
constexpr int kMoeGemmBN = 256;
constexpr int kMoeGemmThreads = 256;

template <int BITS, int DT, int NMAT, int BM>
hipError_t run_gemm_tiles(const MoeArgs& a, const MoeRouting& r, hipStream_t st)
{
    // 32-pair tiles of the plain form (few pairs per expert, a short K such as
    // the down projection's) take 128-row blocks: an XCD's 64 blocks then keep
    // about 3 MB of codes live instead of 6, under its 4 MB L2, so the four
    // k-steps that read one 128-byte code line find it there (down at 64
    // tokens over 128 experts: 42.1 -> 38.1 us; 64-pair tiles measured the
    // same either way).
    constexpr int BN = (NMAT == 1 && BM == 32) ? 128 : kMoeGemmBN, NT = kMoeGemmThreads;
    constexpr int NA = QP_MOE_GEMM_NA, NC = QP_MOE_GEMM_NC;
    constexpr int LDS = gemm::lds_bytes<BITS, BM, BN, NT, NA, NC>();
    static_assert(LDS <= 160 * 1024, "LDS budget");
    const void* kern = reinterpret_cast<const void*>(
        &gemm::qgemm_tile_kernel<BITS, DT, BM, BN, NT, 1, NMAT, true, NA, NC>);
    static bool attr_set = false; // per instantiation; set before its first launch
    static int per_cu = 0;        // blocks of this kernel one CU holds at once
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
        if (e != hipSuccess)
            return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, NT, LDS);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    const int64_t P = a.n_tokens * a.top_k;
    GemmArgs g{};
    g.x = a.a;
    for (int t = 0; t < 2; ++t) {
        const int src = NMAT == 2 ? t : 0;
        g.wq[t] = a.wq[src];
        g.scales[t] = a.scales[src];
        g.biases[t] = a.biases[src];
    }
    g.y = a.out;
    g.M = 0;
    g.N = (int)a.n_rows;
    g.K = (int)a.n_cols;
    g.gs = a.gs;
    g.x_bytes = (uint32_t)(((a.n_tokens - 1) * a.a_outer + (a.top_k - 1) * a.a_inner + a.n_cols) * 2);
    g.y_bytes = (uint32_t)(P * a.n_rows * 2);
    g.sb_bytes = (uint32_t)((a.E * a.n_rows * (a.n_cols / a.gs) * 2 + 3) & ~int64_t(3));
    g.tiles_n = (int)((a.n_rows + BN / NMAT - 1) / (BN / NMAT));
    g.perm = r.perm;
    g.tdesc = static_cast<const TileDesc*>(r.tiles);
    g.n_tiles = r.n_tiles;
    g.top_k = (int)a.top_k;
    g.outer_b = (uint32_t)(a.a_outer * 2);
    g.inner_b = (uint32_t)(a.a_inner * 2);
    int cus = 0;
    hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess)
        return e;
    const int64_t resident = std::max<int64_t>(8, (int64_t)std::max(per_cu, 1) * cus / 8 * 8);
    const int64_t blocks = std::min((r.max_tiles * g.tiles_n + 7) / 8 * 8, resident);
    hipLaunchKernelGGL((gemm::qgemm_tile_kernel<BITS, DT, BM, BN, NT, 1, NMAT, true, NA, NC>),
                       dim3((unsigned)blocks), dim3(NT), LDS, st, g);
    return hipGetLastError();
}

// Four-row matrix-instruction tiles of up to 8 pairs (moe_rows.hpp): grid x
// covers the expert's rows 64 at a time, y strides over the tiles.
template <int BITS, int DT, int NMAT>
hipError_t run_rowmfma_tiles(const GemvKernelArgs& k, int64_t max_tiles, hipStream_t st)
{
    if constexpr ((BITS == 2 || BITS == 4 || BITS == 8) && DT != DT_F32) {
        int64_t gy = max_tiles < 65535 ? max_tiles : 65535;
        gy = gy < 1 ? 1 : gy;
        constexpr int rows = 4 * kMoeRowWaves * kMoeRowQuads;
        const dim3 grid((unsigned)((k.R + rows - 1) / rows), (unsigned)gy);
        const dim3 block(64 * kMoeRowWaves);
        const int64_t rounds = (k.K / 32 + 15) / 16;
        if (rounds <= 1)
            hipLaunchKernelGGL((qgemv_moe_rowmfma_kernel<BITS, DT, 1, NMAT, 2>), grid, block, 0, st, k);
        else if (rounds <= 2)
            hipLaunchKernelGGL((qgemv_moe_rowmfma_kernel<BITS, DT, 2, NMAT, 2>), grid, block, 0, st, k);
        else if (rounds <= 4)
            hipLaunchKernelGGL((qgemv_moe_rowmfma_kernel<BITS, DT, 4, NMAT, 2>), grid, block, 0, st, k);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    } else {
        (void)k; (void)max_tiles; (void)st;
        return hipErrorInvalidValue;
    }
}

// One-pair tiles on the dot-product row kernel (moe_rows.hpp): grid x covers
// the expert's rows 4 D at a time, y strides over the tiles.
template <int BITS, int DT, int NMAT, int UPL, int KL>
hipError_t run_rowstream_tiles_upl(const GemvKernelArgs& k, int64_t max_tiles, hipStream_t st)
{
    constexpr int D = rowstream_depth<BITS, UPL * NMAT>();
    constexpr int ROWS = 4 * (64 / KL) * D;          // weight rows of a block
    int64_t gy = max_tiles < 65535 ? max_tiles : 65535;
    gy = gy < 1 ? 1 : gy;
    const dim3 grid((unsigned)((k.R + ROWS - 1) / ROWS), (unsigned)gy);
    hipLaunchKernelGGL((qgemv_moe_rowstream_kernel<BITS, DT, UPL, NMAT, KL>), grid, dim3(256), 0, st,
                       k);
    return hipGetLastError();
}

template <int BITS, int DT, int NMAT>
hipError_t run_rowstream_tiles(const GemvKernelArgs& k, int64_t max_tiles, hipStream_t st)
{
    if constexpr ((BITS == 2 || BITS == 4 || BITS == 8) && DT != DT_F32) {
        const int64_t units = k.K / 32;
        const bool narrow = units <= 32;
        if (narrow) return run_rowstream_tiles_upl<BITS, DT, NMAT, 1, 32>(k, max_tiles, st);
        if (units <= 64) return run_rowstream_tiles_upl<BITS, DT, NMAT, 1, 64>(k, max_tiles, st);
        if (units <= 128) return run_rowstream_tiles_upl<BITS, DT, NMAT, 2, 64>(k, max_tiles, st);
        return hipErrorInvalidValue;
    } else {
        (void)k; (void)max_tiles; (void)st;
        return hipErrorInvalidValue;
    }
}

template <int BITS, int DT, int NMAT>
hipError_t run_moe(const MoeArgs& a, const MoeRouting& r, hipStream_t st)
{
    GemvKernelArgs k{};
    k.x = a.a;
    k.top_k = a.top_k;
    k.outer = a.a_outer;
    k.inner = a.a_inner;
    k.perm = r.perm;
    k.tiles = static_cast<const TileDesc*>(r.tiles);
    k.n_tiles = r.n_tiles;
    if (r.tiles == nullptr) {   // no routing launch: pair t is tile t
        k.ids = a.ids;
        k.n_pairs = (int)(a.n_tokens * a.top_k);
        k.n_experts = (int)a.E;
    }
    k.M = 0;
    for (int t = 0; t < 2; ++t) {
        const int src = NMAT == 2 ? t : 0;
        k.wq[t] = a.wq[src];
        k.scales[t] = a.scales[src];
        k.biases[t] = a.biases[src];
    }
    k.R = a.n_rows;
    k.K = a.n_cols;
    k.gs = a.gs;
    k.out = a.out;
    // The streaming kernel reads activation rows as 16-byte vectors and uses
    // 32-bit offsets inside one expert matrix and the output.
    const int64_t es = (int64_t)sizeof(St<DT>);
    const int64_t P = a.n_tokens * a.top_k;
    const bool x_vec = reinterpret_cast<uintptr_t>(a.a) % 16 == 0 &&
                       (a.a_outer * es) % 16 == 0 && (a.a_inner * es) % 16 == 0 &&
                       a.n_rows * (a.n_cols * BITS / 8) < (int64_t(1) << 31) &&
                       a.n_rows * (a.n_cols / a.gs) * es < (int64_t(1) << 31) &&
                       P * a.n_rows * es < (int64_t(1) << 31);
    k.out_bytes = (uint32_t)(x_vec ? P * a.n_rows * es : 0);
    const int64_t x_span = ((a.n_tokens - 1) * a.a_outer + (a.top_k - 1) * a.a_inner + a.n_cols) * es;
    k.x_bytes = (uint32_t)(x_span < (int64_t(1) << 31) ? x_span : 0);
    if constexpr (DT == DT_F32) {
        return run_generic<BITS, DT, NMAT>(k, r.max_tiles, st);
    } else {
        if (r.rowmfma > 0)
            return run_rowmfma_tiles<BITS, DT, NMAT>(k, r.max_tiles, st);
        if (r.rowstream > 0)
            return run_rowstream_tiles<BITS, DT, NMAT>(k, r.max_tiles, st);
        if (r.gemm_bm == 64)
            return run_gemm_tiles<BITS, DT, NMAT, 64>(a, r, st);
        if (r.gemm_bm == 32)
            return run_gemm_tiles<BITS, DT, NMAT, 32>(a, r, st);
        if (r.nb > 0)
            return run_skinny_tiles<BITS, DT, NMAT>(k, r.max_tiles, st);
        if (!x_vec)
            return run_generic<BITS, DT, NMAT>(k, r.max_tiles, st);
        switch (r.mt) {
        case 1: return run_mt<BITS, DT, 1, NMAT>(k, r.max_tiles, st);
        case 2: return run_mt<BITS, DT, 2, NMAT>(k, r.max_tiles, st);
        }
        return run_generic<BITS, DT, NMAT>(k, r.max_tiles, st);
    }
}

#if QP_NMAT == 1 && (QP_BITS == 2 || QP_BITS == 4 || QP_BITS == 8)
// The fused down projection and slot combine: grid x covers the output rows
// (4 waves x 64 / KL rows per block), y the tokens.
template <int BITS, int DT, int UPL, int KL>
hipError_t run_rowcombine_upl(const GemvKernelArgs& k, const float* rw, int64_t n_tokens, hipStream_t st)
{
    constexpr int ROWS = 4 * (64 / KL);
    int64_t gy = n_tokens < 65535 ? n_tokens : 65535;
    gy = gy < 1 ? 1 : gy;
    const dim3 grid((unsigned)((k.R + ROWS - 1) / ROWS), (unsigned)gy);
    hipLaunchKernelGGL((qgemv_moe_rowcombine_kernel<BITS, DT, UPL, KL, kMoeCombineMaxTopK>), grid, dim3(256), 0,
                       st, k, rw, n_tokens);
    return hipGetLastError();
}

template <int BITS, int DT>
hipError_t run_rowcombine(const MoeArgs& a, const float* rw, void* out, hipStream_t st)
{
    GemvKernelArgs k{};
    k.x = a.a;
    k.top_k = a.top_k;
    k.outer = a.a_outer;
    k.inner = a.a_inner;
    k.ids = a.ids;
    k.n_pairs = (int)(a.n_tokens * a.top_k);
    k.n_experts = (int)a.E;
    k.wq[0] = k.wq[1] = a.wq[0];
    k.scales[0] = k.scales[1] = a.scales[0];
    k.biases[0] = k.biases[1] = a.biases[0];
    k.R = a.n_rows;
    k.K = a.n_cols;
    k.gs = a.gs;
    k.out = out;
    k.out_bytes = (uint32_t)(a.n_tokens * a.n_rows * 2);
    k.x_bytes = (uint32_t)(((a.n_tokens - 1) * a.a_outer + (a.top_k - 1) * a.a_inner + a.n_cols) * 2);
    const int64_t units = a.n_cols / 32;
    if (units <= 32) return run_rowcombine_upl<BITS, DT, 1, 32>(k, rw, a.n_tokens, st);
    if (units <= 64) return run_rowcombine_upl<BITS, DT, 1, 64>(k, rw, a.n_tokens, st);
    if (units <= 128) return run_rowcombine_upl<BITS, DT, 2, 64>(k, rw, a.n_tokens, st);
    return hipErrorInvalidValue;
}
#endif

} // namespace

#if QP_NMAT == 1 && (QP_BITS == 2 || QP_BITS == 4 || QP_BITS == 8)
hipError_t QP_CAT(QP_CAT(launch_moe_b, QP_BITS), _dc)(const MoeArgs& a, const float* rw, void* out,
                                                      hipStream_t st)
{
    switch (a.dt) {
    case DT_F16: return run_rowcombine<QP_BITS, DT_F16>(a, rw, out, st);
    case DT_BF16: return run_rowcombine<QP_BITS, DT_BF16>(a, rw, out, st);
    }
    return hipErrorInvalidValue;
}
#endif

hipError_t QP_CAT(QP_CAT(QP_CAT(launch_moe_b, QP_BITS), _n), QP_NMAT)(const MoeArgs& a,
                                                                       const MoeRouting& r,
                                                                       hipStream_t st)
{
    switch (a.dt) {
    case DT_F32: return run_moe<QP_BITS, DT_F32, QP_NMAT>(a, r, st);
    case DT_F16: return run_moe<QP_BITS, DT_F16, QP_NMAT>(a, r, st);
    case DT_BF16: return run_moe<QP_BITS, DT_BF16, QP_NMAT>(a, r, st);
    }
    return hipErrorInvalidValue;
}

} // namespace qp
