// moe.hip — MoE over stacked experts (ferrum-kernels src/stacked_expert.rs,
// `gemv_moe_id`, `gemv_moe_id_batched`, `gemv_moe_id_gate_up_silu` docs):
//   out[p, :] = a_row(p) @ dequant(W[ids[p]])^T,
//   a_row(p) = a + (p/top_k)*outer + (p%top_k)*inner,
// optionally fused as SiLU(gate) * up.
//
// Two launches, no host synchronisation (the page's point about removing the
// device-to-host read of tokens-per-expert before the GEMM):
//  1. routing: one block counts pairs per expert (LDS atomics), scans the
//     counts, writes a tile list (each tile: up to MT pairs of one expert) and
//     scatters the pair indices into expert order, all in the workspace;
//  2. compute: over the tile list, one of the routed tile GEMM
//     (gemm_core.hpp), the skinny matrix-core kernel (skinny.hpp) or the
//     streaming GEMV (gemv_core.hpp); blocks past the device-written tile
//     count exit at once. Each tile streams its expert's weights once, so an
//     expert's weights are read once per launch when its pairs fit one tile.
// With at most one pair per expert on average (tiles of one pair), the
// routing launch is skipped: the compute launch takes pair t as tile t.
// Each pair's accumulation order does not depend on its slot in a tile, so the
// (unordered) scatter cannot change any output value.
#include "gemv_core.hpp"
#include "skinny.hpp"
#include "launch.hpp"

namespace qp {

namespace {

constexpr int ROUTE_THREADS = 1024;
constexpr int kMaxExperts = 4096;

struct WsLayout {
    size_t hdr, perm, tiles, total;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(int64_t P, int64_t E)
{
    WsLayout l{};
    l.hdr = 0;
    l.perm = align256(16);
    l.tiles = l.perm + align256((size_t)(P > 0 ? P : 1) * 4);
    l.total = l.tiles + align256((size_t)(P + E + 1) * sizeof(TileDesc));
    return l;
}

} // namespace

// hdr[0] = number of tiles, hdr[1] = number of pairs with an invalid id.
// One block: the first ids are loaded before anything else (their latency
// overlaps the clearing of the counts), the per-expert pair and tile counts
// are scanned by the first wave alone (each lane owns a contiguous run of
// experts; shuffles, no block barriers), so the block synchronises three
// times in all.
__global__ __launch_bounds__(ROUTE_THREADS) void moe_route_kernel(
    const int32_t* __restrict__ ids, int P, int E, int MT, int32_t* __restrict__ hdr,
    int32_t* __restrict__ perm, TileDesc* __restrict__ tiles)
{
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_cur[kMaxExperts];
    __shared__ int s_invalid;
    constexpr int PRE = 4;   // ids per thread loaded up front
    const int tid = threadIdx.x;
    int pre[PRE];
#pragma unroll
    for (int i = 0; i < PRE; ++i) {
        const int p = tid + i * ROUTE_THREADS;
        pre[i] = p < P ? ids[p] : -1;
    }
    for (int e = tid; e < E; e += ROUTE_THREADS)
        s_cnt[e] = 0;
    if (tid == 0)
        s_invalid = 0;
    __syncthreads();
    int invalid = 0;
#pragma unroll
    for (int i = 0; i < PRE; ++i) {
        const int e = pre[i];
        if (e >= 0 && e < E)
            atomicAdd(&s_cnt[e], 1);
        else if (tid + i * ROUTE_THREADS < P)
            ++invalid;
    }
    for (int p = tid + PRE * ROUTE_THREADS; p < P; p += ROUTE_THREADS) {
        const int e = ids[p];
        if (e >= 0 && e < E)
            atomicAdd(&s_cnt[e], 1);
        else
            ++invalid;
    }
    if (invalid)
        atomicAdd(&s_invalid, invalid);
    __syncthreads();

    // Wave 0: lane l owns experts [l * ept, (l + 1) * ept); exclusive scans
    // of the pair and tile counts across the lanes, then the tile list and
    // the scatter cursors.
    if (tid < 64) {
        const int lane = tid;
        const int ept = (E + 63) / 64;
        const int e0 = lane * ept;
        int my_pairs = 0, my_tiles = 0;
        for (int e = e0; e < e0 + ept && e < E; ++e) {
            my_pairs += s_cnt[e];
            my_tiles += (s_cnt[e] + MT - 1) / MT;
        }
        int inc_p = my_pairs, inc_t = my_tiles;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int tp = __shfl_up(inc_p, off, 64);
            const int tt = __shfl_up(inc_t, off, 64);
            if (lane >= off) {
                inc_p += tp;
                inc_t += tt;
            }
        }
        int pair_off = inc_p - my_pairs, tile_off = inc_t - my_tiles;
        for (int e = e0; e < e0 + ept && e < E; ++e) {
            const int c = s_cnt[e];
            for (int j = 0; j * MT < c; ++j) {
                TileDesc d;
                d.expert = e;
                d.start = pair_off + j * MT;
                d.count = (c - j * MT) < MT ? (c - j * MT) : MT;
                tiles[tile_off++] = d;
            }
            s_cur[e] = pair_off;
            pair_off += c;
        }
        if (lane == 63) {
            hdr[0] = inc_t;
            hdr[1] = s_invalid;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PRE; ++i) {
        const int e = pre[i];
        if (e >= 0 && e < E)
            perm[atomicAdd(&s_cur[e], 1)] = tid + i * ROUTE_THREADS;
    }
    for (int p = tid + PRE * ROUTE_THREADS; p < P; p += ROUTE_THREADS) {
        const int e = ids[p];
        if (e >= 0 && e < E)
            perm[atomicAdd(&s_cur[e], 1)] = p;
    }
}

size_t moe_workspace_bytes(int64_t n_pairs, int64_t num_experts)
{
    return ws_layout(n_pairs, num_experts).total;
}

namespace {

int pick_mt(int64_t P, int64_t E, int mtmax)
{
    int mt = 1;
    while (mt < mtmax && (int64_t)mt * E < P)
        mt <<= 1;
    return mt;
}

} // namespace

int moe_tile_height(int64_t n_pairs, int64_t num_experts, int, int)
{
    // The register-resident kernel holds up to 2 activation rows (fp32
    // activations and exact fp32 codes, whatever the precision).
    return pick_mt(n_pairs, num_experts, 2);
}

hipError_t launch_moe_route(const MoeArgs& a, int mt, MoeRouting* r, hipStream_t st)
{
    const int64_t P = a.n_tokens * a.top_k;
    WsLayout l = ws_layout(P, a.E);
    char* ws = static_cast<char*>(a.workspace);
    int32_t* hdr = reinterpret_cast<int32_t*>(ws + l.hdr);
    int32_t* perm = reinterpret_cast<int32_t*>(ws + l.perm);
    TileDesc* tiles = reinterpret_cast<TileDesc*>(ws + l.tiles);
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(ROUTE_THREADS), 0, st, a.ids, (int)P,
                       (int)a.E, mt, hdr, perm, tiles);
    r->n_tiles = hdr;
    r->perm = perm;
    r->tiles = tiles;
    r->mt = mt;
    // Each tile holds >= 1 pair and each expert leaves at most one partial tile.
    int64_t max_tiles = (P + mt - 1) / mt + a.E;
    r->max_tiles = max_tiles < P ? max_tiles : P;
    return hipGetLastError();
}

#ifndef QP_MOE_GEMM_MIN_PAIRS
#define QP_MOE_GEMM_MIN_PAIRS 16
#endif
constexpr int64_t kMoeGemmMinPairsPerExpert = QP_MOE_GEMM_MIN_PAIRS;

int moe_mfma_nb(const MoeArgs& a)
{
    if (a.dt == DT_F32)
        return 0;
    const int64_t P = a.n_tokens * a.top_k;
    // Matrix-core tiles pay off once experts see a few pairs each on average.
    if (P < 2 * a.E || P < 32)
        return 0;
    const int64_t es = 2;
    const bool vec = reinterpret_cast<uintptr_t>(a.a) % 16 == 0 && (a.a_outer * es) % 16 == 0 &&
                     (a.a_inner * es) % 16 == 0;
    const int64_t x_span = ((a.n_tokens - 1) * a.a_outer + (a.top_k - 1) * a.a_inner + a.n_cols) * es;
    const bool small = x_span < (int64_t(1) << 31) &&
                       a.n_rows * (a.n_cols * a.bits / 8) < (int64_t(1) << 31) &&
                       a.n_rows * (a.n_cols / a.gs) * es < (int64_t(1) << 31) &&
                       P * a.n_rows * es < (int64_t(1) << 31);
    if (!vec || !small)
        return 0;
    // Tiles of 16 pairs (activation rows read in 16-byte pieces).
    return a.n_cols % 32 == 0 ? 1 : 0;
}

int moe_rowmfma_mt(const MoeArgs& a)
{
    if (a.dt == DT_F32 || !(a.bits == 2 || a.bits == 4 || a.bits == 8) || a.n_cols % 32 != 0 ||
        a.n_cols > 2048)
        return 0;
    const int64_t P = a.n_tokens * a.top_k;
    // The fused gate + up form at two to four pairs per expert: measured 59.4
    // against 72.6 us at 256 pairs and 68.4 against 75.3 us at 512 pairs over
    // 128 experts ([768, 2048] matrices, 4-bit), where the 16-pair
    // matrix-core tiles took it. At 128 and 1024 pairs, and for the plain
    // down projection (against the routed GEMM), it was slower.
    const bool dense_enough = a.fused_silu && P >= 2 * a.E && P <= 4 * a.E;
    if (!dense_enough)
        return 0;
    const int64_t es = 2;
    const bool vec = reinterpret_cast<uintptr_t>(a.a) % 16 == 0 && (a.a_outer * es) % 16 == 0 &&
                     (a.a_inner * es) % 16 == 0;
    const int64_t x_span = ((a.n_tokens - 1) * a.a_outer + (a.top_k - 1) * a.a_inner + a.n_cols) * es;
    const bool small = x_span < (int64_t(1) << 31) &&
                       a.n_rows * (a.n_cols * a.bits / 8) < (int64_t(1) << 31) &&
                       a.n_rows * (a.n_cols / a.gs) * es < (int64_t(1) << 31) &&
                       P * a.n_rows * es < (int64_t(1) << 31);
    return vec && small ? 8 : 0;
}

bool moe_rowstream_ok(const MoeArgs& a, int mt)
{
    if (mt != 1 || a.dt == DT_F32 || !(a.bits == 2 || a.bits == 4 || a.bits == 8) ||
        a.n_cols % 32 != 0 || a.n_cols > 4096)
        return false;
    // Measured on 128 experts, 4-bit ([768, 2048] gate / up, [2048, 768]
    // down), device time of graph-replayed calls: the fused form 6.4 against
    // 6.8 us at 8 pairs, 8.1 against 9.0 at 16, 13.1 against 16.1 at 32, 22.6
    // against 23.0 at 64, level or slower from 128 pairs; the down projection
    // (32-lane row slots for its 24 units) 4.1 against 5.7 us at 8 pairs, 5.8
    // against 7.5 at 16, 9.7 against 11.8 at 32, 16.5 against 20.8 at 64 and
    // 29.7 against 32.4 at 128.
    const int64_t P = a.n_tokens * a.top_k;
    if (a.fused_silu ? 2 * P > a.E : P > a.E)
        return false;
    const int64_t es = 2;
    const bool vec = reinterpret_cast<uintptr_t>(a.a) % 16 == 0 && (a.a_outer * es) % 16 == 0 &&
                     (a.a_inner * es) % 16 == 0;
    const int64_t x_span = ((a.n_tokens - 1) * a.a_outer + (a.top_k - 1) * a.a_inner + a.n_cols) * es;
    return vec && x_span < (int64_t(1) << 31) &&
           a.n_rows * (a.n_cols * a.bits / 8) < (int64_t(1) << 31) &&
           a.n_rows * (a.n_cols / a.gs) * es < (int64_t(1) << 31) &&
           P * a.n_rows * es < (int64_t(1) << 31);
}

int moe_gemm_bm(const MoeArgs& a)
{
    if (a.dt == DT_F32 || a.n_cols % 64 != 0)
        return 0;
    const int64_t P = a.n_tokens * a.top_k;
    // The routed GEMM dequantizes each expert's weights once per tile (of 32
    // or 64 pairs); it takes over from the GEMV tiles once experts see enough pairs each.
    // The skinny tiles read a tile's activations once per row block, which
    // costs relatively more at short K: for the plain form with K <= 1024
    // (the down projection) the routed GEMM won from 2 pairs per expert
    // (measured 53 vs 60 us at 4, 47 vs 54 us at 2, [128, 2048, 768]).
    const int64_t min_pairs =
        (!a.fused_silu && a.n_cols <= 1024) ? 2 : kMoeGemmMinPairsPerExpert;
    if (P < min_pairs * a.E)
        return 0;
    const int64_t es = 2;
    const bool vec = reinterpret_cast<uintptr_t>(a.a) % 16 == 0 && (a.a_outer * es) % 16 == 0 &&
                     (a.a_inner * es) % 16 == 0;
    const int64_t x_span = ((a.n_tokens - 1) * a.a_outer + (a.top_k - 1) * a.a_inner + a.n_cols) * es;
    // Scales / biases are read as aligned dwords over the whole stack.
    const bool sb = reinterpret_cast<uintptr_t>(a.scales[0]) % 4 == 0 &&
                    reinterpret_cast<uintptr_t>(a.biases[0]) % 4 == 0 &&
                    (!a.fused_silu || (reinterpret_cast<uintptr_t>(a.scales[1]) % 4 == 0 &&
                                       reinterpret_cast<uintptr_t>(a.biases[1]) % 4 == 0));
    const bool small = x_span < (int64_t(1) << 31) &&
                       a.n_rows * (a.n_cols * a.bits / 8) < (int64_t(1) << 31) &&
                       a.E * a.n_rows * (a.n_cols / a.gs) * es < (int64_t(1) << 30) &&
                       P * a.n_rows * es < (int64_t(1) << 31);
    // 32-pair tiles below 16 pairs per expert: the down projection of 128
    // experts measured 42.6 against 46.1 us at 4 pairs per expert and 42.9
    // against 47.1 at 8; at 32 pairs per expert, where many experts would
    // need two 32-pair tiles (their weights dequantized twice), 55.5 against
    // 50.5 us.
    if (!(vec && sb && small))
        return 0;
    return P < 16 * a.E ? 32 : 64;
}

MoeRouting moe_plan(const MoeArgs& a)
{
    MoeRouting r{};
    const int64_t P = a.n_tokens * a.top_k;
    const int rm = moe_rowmfma_mt(a);
    const int bm = rm > 0 ? 0 : moe_gemm_bm(a);
    const int nb = rm > 0 || bm > 0 ? 0 : moe_mfma_nb(a);
    r.mt = rm > 0 ? rm : bm > 0 ? bm : nb > 0 ? 16 * nb : moe_tile_height(P, a.E, a.bits, a.dt);
    // One pair per tile: tile t is pair t itself, read straight from ids by
    // the compute launch, and the routing launch is skipped.
    r.max_tiles = P;
    r.nb = nb;
    r.gemm_bm = bm;
    r.rowmfma = rm;
    r.rowstream = moe_rowstream_ok(a, r.mt) ? 1 : 0;
    return r;
}

hipError_t launch_moe_compute(const MoeArgs& a, const MoeRouting& r, hipStream_t st)
{
    const bool f = a.fused_silu;
    switch (a.bits) {
    case 2: return f ? launch_moe_b2_n2(a, r, st) : launch_moe_b2_n1(a, r, st);
    case 3: return f ? launch_moe_b3_n2(a, r, st) : launch_moe_b3_n1(a, r, st);
    case 4: return f ? launch_moe_b4_n2(a, r, st) : launch_moe_b4_n1(a, r, st);
    case 6: return f ? launch_moe_b6_n2(a, r, st) : launch_moe_b6_n1(a, r, st);
    case 8: return f ? launch_moe_b8_n2(a, r, st) : launch_moe_b8_n1(a, r, st);
    }
    return hipErrorInvalidValue;
}

bool moe_down_combine_ok(const MoeArgs& a)
{
    // Where the down projection would run on one-pair tiles (so the fused
    // kernel reads each expert row once per token, as those tiles do), with
    // at most kMoeCombineMaxTopK slots per token, and the whole stack, its
    // scales and the output addressable with 32-bit offsets.
    if (a.fused_silu || a.top_k < 1 || a.top_k > kMoeCombineMaxTopK)
        return false;
    if (!moe_rowstream_ok(a, 1) || moe_plan(a).rowstream == 0)
        return false;
    const int64_t es = 2;
    const int64_t stack = a.E * a.n_rows;
    return stack * (a.n_cols * a.bits / 8) < (int64_t(1) << 31) &&
           stack * (a.n_cols / a.gs) * es < (int64_t(1) << 31) &&
           a.n_tokens * a.n_rows * es < (int64_t(1) << 31);
}

hipError_t launch_moe_down_combine(const MoeArgs& a, const float* rw, void* out, hipStream_t st)
{
    switch (a.bits) {
    case 2: return launch_moe_b2_dc(a, rw, out, st);
    case 4: return launch_moe_b4_dc(a, rw, out, st);
    case 8: return launch_moe_b8_dc(a, rw, out, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_moe(const MoeArgs& a, hipStream_t st)
{
    MoeRouting r = moe_plan(a);
    if (r.mt > 1)
        if (hipError_t e = launch_moe_route(a, r.mt, &r, st); e != hipSuccess)
            return e;
    return launch_moe_compute(a, r, st);
}

hipError_t launch_moe_pair(const MoeArgs& a, const MoeArgs& b, hipStream_t st)
{
    MoeRouting ra = moe_plan(a), rb = moe_plan(b);
    if (ra.mt > 1)
        if (hipError_t e = launch_moe_route(a, ra.mt, &ra, st); e != hipSuccess)
            return e;
    if (hipError_t e = launch_moe_compute(a, ra, st); e != hipSuccess)
        return e;
    if (rb.mt > 1) {
        if (rb.mt == ra.mt) {
            // Same ids, pair count, expert count and tile height: the tables
            // the first call's routing wrote are the second call's.
            rb.n_tiles = ra.n_tiles;
            rb.perm = ra.perm;
            rb.tiles = ra.tiles;
            rb.max_tiles = ra.max_tiles;
        } else if (hipError_t e = launch_moe_route(b, rb.mt, &rb, st); e != hipSuccess) {
            return e;
        }
    }
    return launch_moe_compute(b, rb, st);
}

} // namespace qp
