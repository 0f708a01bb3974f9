// gemm_core.hpp — the matrix-core tile kernel behind the prefill GEMM and the
// routed MoE GEMM: a block computes a BM x BN tile of x @ dequant(W)^T.
//
// The product is the one of emily lib/emily/quantization.ex,
// `quantized_matmul/2` (x [M, K] times the packed [N, K] weight, transposed),
// and for MoE the one of ferrum-kernels src/stacked_expert.rs
// (`gemv_moe_id_batched`, `gemv_moe_id_gate_up_silu`): the activation rows of
// a tile are the pairs one expert serves, gathered through the pair
// permutation, and the weights are that expert's matrix of the stack.
//  - block tile BM x BN x 64 (two 32-code units of every weight row per step),
//    waves in 2 x (WAVES / 2), each wave a (BM/2) x (BN/(WAVES/2)) tile of
//    v_mfma_f32_32x32x16 instructions accumulating in fp32;
//  - each step, the block stages its activation tile [BM][64] and its weight
//    tile [BN][64] in LDS: weight codes are unpacked (emily
//    `dequantize_defn/1` layout) and dequantized in fp32 (q * s' + b') then
//    rounded to the activation type, so every weight is dequantized once per
//    block row;
//  - two LDS stages: the next step's global loads are issued before the
//    current step's MFMAs and written to the other stage interleaved with
//    them (one barrier per step, no branch in the loop body);
//  - LDS rows are 128 bytes (64 x 16-bit); 16-byte chunks are XOR-swizzled by
//    (row / 2) % 8 so that the 16 rows one 16-lane phase of a fragment read
//    touches at one chunk hit distinct banks;
//  - all global accesses are raw buffer accesses: rows past the tile read
//    zeros and their stores drop, so ragged shapes need no branches;
//  - blocks are mapped to tiles XCD by XCD (block b runs on XCD b % 8), each
//    XCD taking a contiguous run of tiles, so blocks that share an activation
//    strip share an L2.
// Fused gate / up (NMAT = 2): the weight tile holds BN / 2 gate rows then the
// same BN / 2 up rows; each wave's fragments pair a gate column with its up
// column in the same lane, and the epilogue writes SiLU(gate) * up.
#pragma once

#include "common.hpp"

namespace qp {

struct GemmArgs {
    const void* x;             // dense: [M, K]; routed: the rows pairs point at
    const uint32_t* wq[2];     // dense: [N, K*bits/32]; routed: [E, N, K*bits/32], [1] = up
    const void* scales[2];     // [(E,) N, K/gs], 4-byte aligned
    const void* biases[2];
    void* y;                   // dense: [M, N]; routed: [pairs, N]
    int M, N, K, gs;           // routed: N = rows per expert matrix
    uint32_t x_bytes;          // bytes of x reachable (< 2^31)
    uint32_t y_bytes;          // bytes of y (< 2^31)
    uint32_t sb_bytes;         // bytes of each scales / biases array, rounded up to 4 (< 2^31)
    // Dense tile grid: tiles_n tiles along N, `tiles` in all, per_xcd per XCD.
    int tiles_n, tiles, per_xcd;
    // Routed form: the tile list written by the routing kernel.
    const int32_t* perm;       // pair indices in expert order
    const TileDesc* tdesc;     // tiles of up to BM pairs of one expert
    const int32_t* n_tiles;    // device tile count
    int top_k;
    uint32_t outer_b, inner_b; // pair p's row: x + (p/top_k)*outer_b + (p%top_k)*inner_b bytes
};

namespace gemm {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}

template <int DT> struct MfmaTraits;
template <> struct MfmaTraits<DT_BF16> {
    using frag_t = bf16x8_t;
    static __device__ __forceinline__ f32x16_t mfma(frag_t a, frag_t b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // Two fp32 values rounded (nearest even) into one packed 16-bit pair.
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi)
    {
        return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
    }
};
template <> struct MfmaTraits<DT_F16> {
    using frag_t = f16x8_t;
    static __device__ __forceinline__ f32x16_t mfma(frag_t a, frag_t b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi)
    {
        return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)lo, (_Float16)hi});
    }
};

constexpr int BK = 64;          // k per step: two units of 32 codes
constexpr int ROW_BYTES = 128;  // one LDS row of activations / weights: 64 x 16-bit
constexpr uint32_t OOB = 0x80000000u; // an offset past every buffer here

// Byte offset of 16-byte chunk c (0..7) of LDS row r: chunks are XOR-swizzled
// by (r / 2) % 8. Two 128-byte rows fill one 256-byte sweep of the banks, so
// the 16 rows a 16-lane phase of a fragment read (or of a dequantized-weight
// write) touches at one chunk land on 16 different 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * ROW_BYTES + ((c ^ swz(r)) << 4); }

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds_base, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma12(__amdgpu_buffer_rsrc_t r, char* lds_base, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds_base, 12, voff, 0, 0, 0);
}

// Weight codes of one row for one step (64 codes) and how they are moved:
// CS-byte DMA chunks (12 for 3-bit, else 16), CPR chunks per row, each chunk
// landing in a 16-byte LDS slot.
template <int BITS> struct CodeLayout {
    static constexpr int RB = 8 * BITS;              // bytes per row per step
    static constexpr int CS = BITS == 3 ? 12 : 16;   // DMA chunk bytes
    static constexpr int CPR = RB / CS;              // chunks per row
    static constexpr int SLOT_ROW = 16 * CPR;        // LDS bytes per row
};
template <int BITS, int BN, int WAVES> struct CodeStage {
    static constexpr int INSTR =
        (BN * CodeLayout<BITS>::CPR + 64 * WAVES - 1) / (64 * WAVES);       // per wave
    static constexpr int STAGE = INSTR * WAVES * 1024;                        // bytes
};

// Scales / biases of one step: one dword per tile row for the scales, then
// one per row for the biases (the aligned dword holding the row's first
// group of the step; with 32-wide groups, both groups of the step).
template <int BN> struct SbStage {
    static constexpr int STAGE = 8 * BN;        // bytes
    static constexpr int INSTR = 2 * BN / 64;   // dword DMA instructions per block
};

// LDS bytes of one block: A[NA] | B[2] | C[NC] | SB[NC].
template <int BITS, int BM, int BN, int THREADS, int NA, int NC>
constexpr int lds_bytes()
{
    return (NA * BM + 2 * BN) * ROW_BYTES + NC * (CodeStage<BITS, BN, THREADS / 64>::STAGE +
                                                  SbStage<BN>::STAGE);
}

// s_waitcnt immediate: at most `vm` vector-memory operations outstanding and
// no LDS operation (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8).
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

// Pipeline (NA activation stages, NC code / scale stages, two dequantized
// weight stages). Step kt issues the activation DMA of step kt + NA - 1 and
// the code and scale DMA of step kt + NC, runs the MFMAs of step kt and
// dequantizes step kt + 1 between them; it then waits only for what step
// kt + 1 needs (activations of kt + 1, codes and scales of kt + 2), so code
// loads get NC - 2 whole steps to arrive and the DMA of the newest steps stays
// in flight across the barrier.
template <int BITS, int DT, int BM, int BN, int THREADS, int NMAT, bool ROUTED, int NA, int NC>
__global__ __launch_bounds__(THREADS) void qgemm_tile_kernel(GemmArgs ga)
{
    using T = MfmaTraits<DT>;
    using frag_t = typename T::frag_t;
    using CL = CodeLayout<BITS>;
    constexpr int WAVES = THREADS / 64;
    constexpr int WGN = WAVES / 2;               // waves: 2 along M x WGN along N
    constexpr int WM = BM / 2, WN = BN / WGN;    // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;    // 32 x 32 MFMA tiles per wave
    constexpr int UPT = 2 * BN / THREADS;        // weight units per thread per step
    constexpr int BNO = BN / NMAT;               // output columns per tile
    constexpr int FNO = FN / NMAT;               // fragments per matrix per wave
    static_assert(BN == THREADS || BN == THREADS / 2, "a weight row per one or two threads");
    static_assert(FM >= 1 && FN >= NMAT && FN % NMAT == 0, "wave tile");
    static_assert(!ROUTED || NMAT == 1 || (BNO % 64 == 0 && (BNO * CL::CPR) % 64 == 0),
                  "each wave's rows and each DMA instruction within one matrix");
    static_assert(NMAT == 1 || ROUTED, "the fused form is routed");
    static_assert(NA >= 2 && NA <= 3 && NC >= 3, "pipeline depth");
    constexpr int A_STAGE = BM * ROW_BYTES, B_STAGE = BN * ROW_BYTES;
    constexpr int A_INSTR = A_STAGE / 1024 / WAVES;        // 1 KB DMA instructions per wave
    static_assert(A_INSTR * 1024 * WAVES == A_STAGE, "activation stage in whole DMA blocks");
    constexpr int C_INSTR = CodeStage<BITS, BN, WAVES>::INSTR;   // per wave (64 chunks each)
    // Every DMA instruction writes 64 x 16 bytes, so a codes stage spans whole
    // 1 KB blocks (chunks past the tile read zeros into the spare slots).
    constexpr int C_STAGE = CodeStage<BITS, BN, WAVES>::STAGE;
    constexpr int SB_STAGE = SbStage<BN>::STAGE;
    constexpr int SB_INSTR = SbStage<BN>::INSTR / WAVES;   // per wave
    static_assert(SB_INSTR * WAVES == SbStage<BN>::INSTR, "scale DMA split over waves");
    // Vector-memory operations a wave issues per step, and how many of them
    // may still be in flight when a step ends (the newest ones; everything
    // older, up to the activations of the next step and the codes and scales
    // of the one after, has landed).
    constexpr int STEP_OPS = A_INSTR + C_INSTR + SB_INSTR;
    // Step kt needs the activations of step kt + 1 (the first DMA of step
    // kt + 2 - NA) and the codes / scales of step kt + 2 (the last DMA of step
    // kt + 2 - NC); what was issued after the later of the two may be in flight.
    constexpr int IN_FLIGHT = NC > NA ? (C_INSTR + SB_INSTR) + (NA - 2) * STEP_OPS
                                      : (NC - 2) * STEP_OPS;
    static_assert(IN_FLIGHT < 64, "vmcnt range");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char* const a_st = lds;
    char* const b_st = a_st + NA * A_STAGE;
    char* const c_st = b_st + 2 * B_STAGE;
    char* const sb_st = c_st + NC * C_STAGE;

    const int K = ga.K, N = ga.N;
    const uint32_t xrow_bytes = (uint32_t)K * 2;
    const uint32_t wrow_bytes = (uint32_t)K * BITS / 8;
    const uint32_t groups = (uint32_t)(K / ga.gs);

    // Tile of this block, XCD by XCD.
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    int m0 = 0, n0, expert = 0, start = 0, count = 0;
    if constexpr (ROUTED) {
        // The grid covers the largest possible tile list; the real one is
        // spread evenly over the XCDs and the remaining blocks exit.
        const int work = *ga.n_tiles * ga.tiles_n;
        const int per_xcd = (work + 7) / 8;
        if (local >= per_xcd)
            return;
        const int w = xcd * per_xcd + local;
        if (w >= work)
            return;
        const TileDesc d = ga.tdesc[w / ga.tiles_n];
        expert = d.expert;
        start = d.start;
        count = d.count;
        n0 = (w % ga.tiles_n) * BNO;
    } else {
        if (local >= ga.per_xcd)
            return;
        const int tile = xcd * ga.per_xcd + local;
        if (tile >= ga.tiles)
            return;
        m0 = (tile / ga.tiles_n) * BM;
        n0 = (tile % ga.tiles_n) * BN;
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;

    const __amdgpu_buffer_rsrc_t rx = rsrc(ga.x, ga.x_bytes);
    // Weight operands of matrix t: this tile's expert in the stack.
    const size_t wmat_bytes = (size_t)N * wrow_bytes;
    auto rw_of = [&](int t) {
        return rsrc(reinterpret_cast<const char*>(ga.wq[t]) + (size_t)expert * wmat_bytes,
                    (uint32_t)wmat_bytes);
    };
    // Scales / biases: the whole array (all experts), read as aligned dwords.
    auto rsb_of = [&](int t, bool bias) {
        return rsrc(bias ? ga.biases[t] : ga.scales[t], ga.sb_bytes);
    };
    const uint32_t e_groups = (uint32_t)expert * (uint32_t)N * groups;

    // DMA plan. Activations: wave w's instruction i moves rows 8g..8g+7 of the
    // tile (g = A_INSTR * w + i) into 1 KB of LDS; lane l lands in slot l
    // = (row 8g + l/8, physical chunk l%8), so it reads logical chunk
    // (l%8) ^ swz(row) of that row. Rows past the tile read zeros.
    uint32_t a_goff[A_INSTR];
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
        const int g = wave * A_INSTR + i, r = 8 * g + (lane >> 3);
        const uint32_t c16 = (uint32_t)(((lane & 7) ^ swz(r)) * 16);
        if constexpr (ROUTED) {
            uint32_t off = OOB;
            if (r < count) {
                const int p = ga.perm[start + r];
                off = (uint32_t)(p / ga.top_k) * ga.outer_b + (uint32_t)(p % ga.top_k) * ga.inner_b +
                      c16;
            }
            a_goff[i] = off;
        } else {
            a_goff[i] = m0 + r < ga.M ? (uint32_t)(m0 + r) * xrow_bytes + c16 : OOB;
        }
    }
    // Codes: flat chunk q = 64 * (wave * C_INSTR + i) + lane -> tile row
    // q / CPR, part q % CPR; LDS slot q. Tile row r is row n0 + r % BNO of
    // matrix r / BNO; one DMA instruction stays within one matrix.
    uint32_t c_goff[C_INSTR];
    __amdgpu_buffer_rsrc_t rw[C_INSTR];
#pragma unroll
    for (int i = 0; i < C_INSTR; ++i) {
        const int q = 64 * (wave * C_INSTR + i) + lane;
        const int r = q / CL::CPR, part = q % CL::CPR;
        const int row = n0 + r % BNO;
        c_goff[i] = (q < BN * CL::CPR && row < N)
            ? (uint32_t)row * wrow_bytes + part * CL::CS : OOB;
        int t = 64 * (wave * C_INSTR + i) / (BNO * CL::CPR);
        t = t < NMAT ? t : NMAT - 1;
        rw[i] = rw_of(t);
    }
    // Scales / biases: instruction j = wave * SB_INSTR + i moves the dwords of
    // tile rows 64 (j % (BN / 64)) + lane, scales for j < BN / 64, else biases.
    uint32_t sb_row[SB_INSTR];
    __amdgpu_buffer_rsrc_t rsb[SB_INSTR];
#pragma unroll
    for (int i = 0; i < SB_INSTR; ++i) {
        const int j = wave * SB_INSTR + i;
        const int r = 64 * (j % (BN / 64)) + lane;
        const int row = n0 + r % BNO;
        sb_row[i] = row < N ? e_groups + (uint32_t)row * groups : 0x40000000u;
        rsb[i] = rsb_of(NMAT == 1 ? 0 : (r / BNO), j >= BN / 64);
    }
    const uint32_t gshift = (uint32_t)__builtin_ctz((unsigned)ga.gs);
    auto dma_a = [&](int kt, int stage) {
#pragma unroll
        for (int i = 0; i < A_INSTR; ++i)
            dma16(rx, a_st + stage * A_STAGE + (wave * A_INSTR + i) * 1024,
                  a_goff[i] + (uint32_t)kt * BK * 2);
    };
    auto dma_c = [&](int kt, int stage) {
#pragma unroll
        for (int i = 0; i < C_INSTR; ++i) {
            char* dst = c_st + stage * C_STAGE + (wave * C_INSTR + i) * 1024;
            const uint32_t off = c_goff[i] + (uint32_t)kt * CL::RB;
            if constexpr (CL::CS == 12)
                dma12(rw[i], dst, off);
            else
                dma16(rw[i], dst, off);
        }
        const uint32_t g0 = ((uint32_t)kt * BK) >> gshift;
#pragma unroll
        for (int i = 0; i < SB_INSTR; ++i) {
            // Rows past N: an offset past the end (reads zeros).
            const uint32_t off = sb_row[i] < 0x40000000u ? ((sb_row[i] + g0) * 2) & ~3u : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsb[i],
                (__attribute__((address_space(3))) void*)(sb_st + stage * SB_STAGE +
                                                          (wave * SB_INSTR + i) * 256),
                4, off, 0, 0, 0);
        }
    };

    // Dequantization work of this thread: tile row b_r, units [u0, u0 + UPT).
    const int b_r = tid % BN;
    const int u0 = (tid / BN) * UPT;
    const int b_row = n0 + b_r % BNO;
    const uint32_t b_gbase = e_groups + (uint32_t)(b_row < N ? b_row : 0) * groups;
    // Codes of step kt (C stage kt % NC) -> activation-typed weights in B stage
    // kt % 2, in slices: slice `part` (0..3) writes 16-byte chunk `part` of each
    // of this thread's units, so the work can be spread over the MFMA phases.
    using CB = CodeBytes<BITS>;
    uint32_t wcode[UPT][CB::NBW];
    float s_u[UPT], b_u[UPT];
    auto load_codes = [&](int kt, int stage) {
        const char* crow = c_st + stage * C_STAGE + b_r * CL::SLOT_ROW;
        static_for<UPT>([&](auto U) {
            const char* src = crow + (BITS == 3 ? (u0 + U) * 16 : (u0 + U) * 4 * BITS);
            uint32_t w[BITS];
#pragma unroll
            for (int i = 0; i < BITS; ++i)
                w[i] = reinterpret_cast<const uint32_t*>(src)[i];
            CB::split(w, wcode[U]);
        });
        // The scale / bias dword holds elements (base & ~1) and (base & ~1) + 1
        // of the array, base = this row's element of the step's first group:
        // with 32-wide groups (base even) both groups of the step, else the
        // step's one group in half base & 1.
        const char* sbp = sb_st + stage * SB_STAGE + b_r * 4;
        const uint32_t sd = *reinterpret_cast<const uint32_t*>(sbp);
        const uint32_t bd = *reinterpret_cast<const uint32_t*>(sbp + 4 * BN);
        const uint32_t base = b_gbase + (((uint32_t)kt * BK) >> gshift);
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const uint32_t g = b_gbase + (((uint32_t)kt * BK + (u0 + u) * 32) >> gshift);
            const uint32_t sh = (g - (base & ~1u)) * 16;
            s_u[u] = Elem<DT>::to_f32((uint16_t)(sd >> sh));
            b_u[u] = Elem<DT>::to_f32((uint16_t)(bd >> sh));
        }
    };
    auto dequant_part = [&](int stage, auto PART) {
        char* brow = b_st + stage * B_STAGE;
        static_for<UPT>([&](auto U) {
            const float s = s_u[U], b = b_u[U];
            uint32_t packed[4];
            static_for<4>([&](auto P) {
                constexpr int k0 = decltype(PART)::value * 8 + 2 * P;
                const float w0 = __builtin_fmaf(CB::template code<k0>(wcode[U]), s, b);
                const float w1 = __builtin_fmaf(CB::template code<k0 + 1>(wcode[U]), s, b);
                packed[P] = T::pack2(w0, w1);
            });
            *reinterpret_cast<u32x4_t*>(brow + lds_off(b_r, (u0 + U) * 4 + decltype(PART)::value)) =
                u32x4_t{packed[0], packed[1], packed[2], packed[3]};
        });
    };
    // End of a step: at most `vm` of this wave's DMAs in flight, its LDS
    // accesses done, then the block barrier. (A fence here would wait for
    // every DMA, so the barrier is issued bare, with compiler barriers around
    // it for the LDS accesses of this thread.)
    auto step_barrier = [&](auto VM) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(decltype(VM)::value));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x16_t{};

    // Tile row of B fragment j of this wave: NMAT = 1, WN consecutive rows;
    // NMAT = 2, the wave's WN / 2 gate rows then the same up rows.
    auto b_frag_row = [&](int j) {
        if constexpr (NMAT == 1)
            return wn * WN + j * 32;
        else
            return (j / FNO) * BNO + wn * (WN / 2) + (j % FNO) * 32;
    };

    // Prologue: the DMA of steps -NC .. -1 of the loop below (activations of
    // steps 0 .. NA-2, codes / scales of steps 0 .. NC-1, in the loop's order,
    // so the loop's in-flight counts hold from its first step), then B of
    // step 0 from the first codes.
    const int KT = K / BK;
#pragma unroll
    for (int s = -NC; s < 0; ++s) {
        if (s + NA - 1 >= 0)
            dma_a(s + NA - 1, s + NA - 1);
        dma_c(s + NC, s + NC);
    }
    // Codes / scales of step 0 have landed: everything after them may not.
    step_barrier(std::integral_constant<int, (NC - 1) * (C_INSTR + SB_INSTR) + (NA - 1) * A_INSTR>{});
    load_codes(0, 0);
    static_for<4>([&](auto PART) { dequant_part(0, PART); });
    // Step 0 needs A(0) (the first DMA of step 1 - NA) and the codes / scales
    // of step 1 (the last DMA of step 1 - NC).
    constexpr int IN_FLIGHT0 = NC > NA ? (C_INSTR + SB_INSTR) + (NA - 2) * STEP_OPS
                                       : (NC - 2) * STEP_OPS;
    step_barrier(std::integral_constant<int, IN_FLIGHT0>{});

    int a_cur = 0, c_nxt = 1;          // A stage of step kt, C stage of step kt + 1
    for (int kt = 0; kt < KT; ++kt) {
        const int b_cur = kt & 1;
        // In flight during this step: activations of kt + NA - 1, codes and
        // scales of kt + NC (reads past the last step are harmless: in-range
        // bytes that are never used, or zeros).
        const int a_new = a_cur + NA - 1 >= NA ? a_cur - 1 : a_cur + NA - 1;
        const int c_new = c_nxt == 0 ? NC - 1 : c_nxt - 1;   // stage of step kt + NC
        dma_a(kt + NA - 1, a_new);
        dma_c(kt + NC, c_new);
        // MFMAs on A stage a_cur / B stage b_cur, fragments double-buffered
        // across the four k16 sub-steps; after each sub-step's MFMAs, a quarter
        // of the weights of step kt + 1 is dequantized.
        const char* abase = a_st + a_cur * A_STAGE;
        const char* bbase = b_st + b_cur * B_STAGE;
        frag_t af[2][FM], bfr[2][FN];
        auto load_frags = [&](int kk, frag_t (&fa)[FM], frag_t (&fb)[FN]) {
            const int chunk = 2 * kk + (lane >> 5);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const frag_t*>(
                    abase + lds_off(wm * WM + i * 32 + (lane & 31), chunk));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[j] = *reinterpret_cast<const frag_t*>(
                    bbase + lds_off(b_frag_row(j) + (lane & 31), chunk));
        };
        load_frags(0, af[0], bfr[0]);
        load_codes(kt + 1, c_nxt);
        static_for<BK / 16>([&](auto KK) {
            constexpr int kk = decltype(KK)::value;
            if constexpr (kk + 1 < BK / 16)
                load_frags(kk + 1, af[(kk + 1) & 1], bfr[(kk + 1) & 1]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = T::mfma(af[kk & 1][i], bfr[kk & 1][j], acc[i][j]);
            dequant_part(b_cur ^ 1, KK);
        });
        step_barrier(std::integral_constant<int, IN_FLIGHT>{});
        a_cur = a_cur + 1 == NA ? 0 : a_cur + 1;
        c_nxt = c_nxt + 1 == NC ? 0 : c_nxt + 1;
    }
    // No DMA may still be writing this block's LDS when the block ends.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

    // Epilogue: lane l, register r of a 32 x 32 tile holds
    // row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32.
    const __amdgpu_buffer_rsrc_t ry = rsrc(ga.y, ga.y_bytes);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        // Output row (dense) or pair (routed) of each register's tile row.
        int orow[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if constexpr (ROUTED)
                orow[r] = row < count ? ga.perm[start + row] : -1;
            else
                orow[r] = m0 + row < ga.M ? m0 + row : -1;
        }
#pragma unroll
        for (int j = 0; j < FNO; ++j) {
            const int col = n0 + (NMAT == 1 ? wn * WN + j * 32 : wn * (WN / 2) + j * 32) + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float v = acc[i][j][r];
                if constexpr (NMAT == 2)
                    v = silu_f32(v) * acc[i][j + FNO][r];
                const uint32_t off = (orow[r] >= 0 && col < N)
                    ? ((uint32_t)orow[r] * (uint32_t)N + (uint32_t)col) * 2 : OOB;
                __builtin_amdgcn_raw_buffer_store_b16(Elem<DT>::from_f32(v), ry, off, 0, 0);
            }
        }
    }
}

} // namespace gemm

} // namespace qp
