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
//    waves in WMW x (WAVES / WMW), each wave a (BM/WMW) x (BN/(WAVES/WMW))
//    tile of v_mfma_f32_32x32x16 instructions accumulating in fp32;
//  - each step, the block stages its activation tile [BM][64], the weight
//    codes of its BN rows and their scales / biases in LDS by DMA; each lane
//    then builds its MFMA B fragments in registers: it reads the 32 codes of
//    one unit of its weight row (emily `dequantize_defn/1` layout), converts
//    them exactly to fp32 (FP8 / FP4 pair conversions of code bytes or
//    nibbles, or byte conversions), applies q * s' + b' in fp32 and rounds to
//    the activation type. The contraction over the step's 64 k
//    is taken in the order the units give: MFMA kk pairs k = 8 kk + i (lanes
//    0-31) with k = 32 + 8 kk + i (lanes 32-63), and the activation fragments
//    are read in the same order;
//  - NA activation stages and NC code / scale stages: the DMA of later steps
//    stays in flight across the per-step barrier, and each step's first
//    fragments (activations and B) are prepared during the step before;
//  - LDS rows of activations are 128 bytes (64 x 16-bit); 16-byte chunks are
//    XOR-swizzled by (row / 2) % 8, and the 16-byte code chunks of a row by a
//    row-dependent XOR, so the rows one phase of a fragment read touches hit
//    distinct banks;
//  - all global accesses are raw buffer accesses: rows past the tile read
//    zeros and their stores drop, so ragged shapes need no branches;
//  - blocks are mapped to tiles XCD by XCD (block b runs on XCD b % 8), each
//    XCD taking a contiguous run of tiles, so blocks that share an activation
//    strip share an L2.
// Fused gate / up (NMAT = 2): the weight tile holds BN / 2 gate rows then the
// same BN / 2 up rows; each wave's fragments pair a gate column with its up
// column in the same lane, and the epilogue writes SiLU(gate) * up.
#pragma once

#include "codepair.hpp"
#include "common.hpp"
#include "mx.hpp"

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
// group of the step; with 32-wide groups, both groups of the step). The
// microscaled modes (MODE > 0) have no biases, and their one-byte scales of a
// step (two of 32-wide groups, four of 16-wide) share one aligned dword.
// Every wave issues the same number of these DMAs (its wait counts assume
// it), so with fewer instructions than waves the spare waves load zeros into
// spare slots.
template <int BN, int WAVES, int MODE = 0> struct SbStage {
    static constexpr int ARRAYS = MODE == 0 ? 2 : 1;
    static constexpr int INSTR = ARRAYS * BN / 64;                  // useful dword DMAs per block
    static constexpr int PER_WAVE = (INSTR + WAVES - 1) / WAVES;    // issued by every wave
    static constexpr int STAGE = PER_WAVE * WAVES * 256;            // bytes
};

// LDS bytes of one block: A[NA] | C[NC] | SB[NC].
template <int BITS, int BM, int BN, int THREADS, int NA, int NC, int MODE = 0>
constexpr int lds_bytes()
{
    return NA * BM * ROW_BYTES + NC * (CodeStage<BITS, BN, THREADS / 64>::STAGE +
                                       SbStage<BN, THREADS / 64, MODE>::STAGE);
}

// Logical 16-byte code chunk c of tile row r sits in slot r * CPR + (c ^
// code_swz(r)): the rows one 16-lane phase of a unit read touches (16
// consecutive rows, one chunk each) then cover all 16 bank groups.
template <int BITS> __device__ __forceinline__ int code_swz(int r)
{
    constexpr int CPR = CodeLayout<BITS>::CPR;
    if constexpr (CPR == 2)
        return (r >> 3) & 1;
    else if constexpr (CPR == 4)
        return (r >> 2) & 3;
    else
        return 0;
}

// s_waitcnt immediate: at most `vm` vector-memory operations outstanding and
// no LDS operation (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8).
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

// Pipeline: step kt issues the activation DMA of step kt + NA - 1 and the code
// and scale DMA of step kt + NC - 1, then runs the MFMAs of step kt; during
// its last two sub-steps it reads the codes, scales and first activation
// fragments of step kt + 1 and builds that step's first B fragments, so the
// next step's MFMAs can start right after the barrier. At its end it waits
// only for what step kt + 1 reads early (the activations and codes / scales
// of kt + 2): activation loads get NA - 2 steps to arrive and code loads
// NC - 2, and the newest DMA stays in flight across the barrier.
// Exact codes 8 kk .. 8 kk + 7 of a unit, in order, as fp32. 4- and 3-bit
// codes go to bytes (a mask; for 3-bit the spreading of codepair.hpp) and
// 2-bit codes to nibbles, and each FP8 / FP4 pair conversion (scale 2^9 / 2,
// powers of two, so the values are the codes exactly) yields two of them;
// 6- and 8-bit codes take one byte conversion each.
template <int BITS> struct GemmCodes {
    using CB = CodeBytes<BITS>;
    static constexpr int NW = BITS == 4 ? 8 : BITS == 2 ? 4 : BITS == 3 ? 3 : CB::NBW;
    static __device__ __forceinline__ void split(const uint32_t (&w)[BITS], uint32_t (&bw)[NW])
    {
        if constexpr (BITS == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bw[2 * i] = and_opaque(w[i], 0x0F0F0F0Fu);           // codes 8i + 0, 2, 4, 6
                bw[2 * i + 1] = and_opaque(w[i] >> 4, 0x0F0F0F0Fu);  // codes 8i + 1, 3, 5, 7
            }
        } else if constexpr (BITS == 2) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                bw[2 * i] = and_opaque(w[i], 0x33333333u);           // nibble n: code 16i + 2n
                bw[2 * i + 1] = and_opaque(w[i] >> 2, 0x33333333u);  // nibble n: code 16i + 2n + 1
            }
        } else if constexpr (BITS == 3) {
#pragma unroll
            for (int i = 0; i < 3; ++i) bw[i] = w[i];
        } else {
            CB::split(w, bw);
        }
    }
    template <int KK> static __device__ __forceinline__ void codes8(const uint32_t (&bw)[NW], float (&q)[8])
    {
        if constexpr (BITS == 4 || BITS == 3) {
            uint32_t even, odd;   // codes 0, 2, 4, 6 and 1, 3, 5, 7 of the eight, one per byte
            if constexpr (BITS == 4) {
                even = bw[2 * KK];
                odd = bw[2 * KK + 1];
            } else {
                const uint32_t sl = KK == 0 ? bw[0]
                                  : KK == 1 ? __builtin_amdgcn_alignbyte(bw[1], bw[0], 3)
                                  : KK == 2 ? __builtin_amdgcn_alignbyte(bw[2], bw[1], 2)
                                            : bw[2] >> 8;
                code_bytes3(sl, 0u, even, odd);
            }
            const f32x2_t e01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(even, 512.0f, false);
            const f32x2_t e23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(even, 512.0f, true);
            const f32x2_t o01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(odd, 512.0f, false);
            const f32x2_t o23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(odd, 512.0f, true);
            q[0] = e01.x; q[1] = o01.x; q[2] = e01.y; q[3] = o01.y;
            q[4] = e23.x; q[5] = o23.x; q[6] = e23.y; q[7] = o23.y;
        } else if constexpr (BITS == 2) {
            constexpr int i = KK / 2;
            static_for<2>([&](auto BB) {
                constexpr int bb = decltype(BB)::value, b = 2 * (KK % 2) + bb;
                const f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(bw[2 * i], 2.0f, b);
                const f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(bw[2 * i + 1], 2.0f, b);
                q[4 * bb] = lo.x; q[4 * bb + 1] = hi.x; q[4 * bb + 2] = lo.y; q[4 * bb + 3] = hi.y;
            });
        } else {
            static_for<8>([&](auto C) { q[decltype(C)::value] = CB::template code<8 * KK + decltype(C)::value>(bw); });
        }
    }
};

template <int BITS, int DT, int BM, int BN, int THREADS, int WMW, int NMAT, bool ROUTED, int NA,
          int NC, int MODE = 0>
__global__ __launch_bounds__(THREADS) void qgemm_tile_kernel(GemmArgs ga)
{
    static_assert(MODE == 0 || (MxFmt<MODE>::BITS == BITS && NMAT == 1 && !ROUTED),
                  "microscaled modes: dense single-matrix tiles");
    using T = MfmaTraits<DT>;
    using frag_t = typename T::frag_t;
    using CL = CodeLayout<BITS>;
    using GC = GemmCodes<BITS>;
    constexpr int WAVES = THREADS / 64;
    constexpr int WGN = WAVES / WMW;             // waves: WMW along M x WGN along N
    constexpr int WM = BM / WMW, WN = BN / WGN;  // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;    // 32 x 32 MFMA tiles per wave
    constexpr int BNO = BN / NMAT;               // output columns per tile
    constexpr int FNO = FN / NMAT;               // fragments per matrix per wave
    static_assert(WAVES % WMW == 0 && FM >= 1 && FM * 32 * WMW == BM, "wave rows");
    static_assert(FN >= NMAT && FN % NMAT == 0 && FN * 32 * WGN == BN, "wave columns");
    static_assert(NMAT == 1 || (BNO % 64 == 0 && (BNO * CL::CPR) % 64 == 0),
                  "each DMA instruction within one matrix");
    static_assert(NMAT == 1 || ROUTED, "the fused form is routed");
    constexpr int A_STAGE = BM * ROW_BYTES;
    constexpr int A_INSTR = A_STAGE / 1024 / WAVES;        // 1 KB DMA instructions per wave
    static_assert(A_INSTR * 1024 * WAVES == A_STAGE, "activation stage in whole DMA blocks");
    constexpr int C_INSTR = CodeStage<BITS, BN, WAVES>::INSTR;   // per wave (64 chunks each)
    // Every DMA instruction writes 64 x 16 bytes, so a codes stage spans whole
    // 1 KB blocks (chunks past the tile read zeros into the spare slots).
    constexpr int C_STAGE = CodeStage<BITS, BN, WAVES>::STAGE;
    using SBS = SbStage<BN, WAVES, MODE>;
    constexpr int SB_STAGE = SBS::STAGE;
    constexpr int SB_INSTR = SBS::PER_WAVE;        // per wave
    // Vector-memory operations a wave issues per step, and how many of them
    // may still be in flight when a step ends. Step kt + 1 reads the
    // activations and codes / scales of step kt + 2: the first DMA of step
    // kt + 3 - NA and the last DMA of step kt + 3 - NC; what was issued after
    // the later of the two may be in flight.
    constexpr int STEP_OPS = A_INSTR + C_INSTR + SB_INSTR;
    static_assert(NA >= 3 && NC >= 4, "prefetch pipeline depth");
    constexpr int IN_FLIGHT = NC > NA ? (C_INSTR + SB_INSTR) + (NA - 3) * STEP_OPS
                                      : (NC - 3) * STEP_OPS;
    static_assert(IN_FLIGHT < 64, "vmcnt range");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char* const a_st = lds;
    char* const c_st = a_st + NA * A_STAGE;
    char* const sb_st = c_st + NC * C_STAGE;

    const int K = ga.K, N = ga.N;
    const uint32_t xrow_bytes = (uint32_t)K * 2;
    const uint32_t wrow_bytes = (uint32_t)K * BITS / 8;
    const uint32_t groups = (uint32_t)(K / ga.gs);

    // Tile of this block, XCD by XCD. The routed form is persistent: its
    // grid is at most what the GPU holds at once, and block l of XCD x takes
    // the items x * per_xcd + l, + B, + 2B, ... of the device-written work
    // list (B = blocks per XCD), so each XCD runs one contiguous stretch of
    // the list (an expert's row blocks side by side). The dense form takes
    // one tile per block.
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    for (int iter = 0;; ++iter) { // the tile loop, through the epilogue below
    int m0 = 0, n0, expert = 0, start = 0, count = 0;
    if constexpr (ROUTED) {
        const int work = *ga.n_tiles * ga.tiles_n;
        const int per_xcd = (work + 7) / 8;
        const int l = local + iter * (int)(gridDim.x / 8);
        if (l >= per_xcd)
            return;
        const int w = xcd * per_xcd + l;
        if (w >= work)
            return;
        const TileDesc d = ga.tdesc[w / ga.tiles_n];
        expert = d.expert;
        start = d.start;
        count = d.count;
        n0 = (w % ga.tiles_n) * BNO;
    } else {
        if (iter > 0 || local >= ga.per_xcd)
            return;
        const int tile = xcd * ga.per_xcd + local;
        if (tile >= ga.tiles)
            return;
        m0 = (tile / ga.tiles_n) * BM;
        n0 = (tile % ga.tiles_n) * BN;
    }

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;

    const __amdgpu_buffer_rsrc_t rx = rsrc(ga.x, ga.x_bytes);
    // Weight codes of matrix t: this tile's expert in the stack.
    const size_t wmat_bytes = (size_t)N * wrow_bytes;
    auto rw_of = [&](int t) {
        return rsrc(reinterpret_cast<const char*>(ga.wq[t]) + (size_t)expert * wmat_bytes,
                    (uint32_t)wmat_bytes);
    };
    // Scales / biases: the whole array (all experts), read as aligned dwords
    // (the array is 4-byte aligned; with an odd element count the last dword
    // reaches 2 bytes past its end, inside the same aligned word and so the
    // same page, and those bytes are never used).
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
    // Codes: flat slot q = 64 * (wave * C_INSTR + i) + lane -> tile row
    // r = q / CPR, physical part q % CPR, holding logical chunk
    // (q % CPR) ^ code_swz(r). Tile row r is row n0 + r % BNO of matrix r / BNO;
    // one DMA instruction stays within one matrix.
    uint32_t c_goff[C_INSTR];
    __amdgpu_buffer_rsrc_t rw[C_INSTR];
#pragma unroll
    for (int i = 0; i < C_INSTR; ++i) {
        const int q = 64 * (wave * C_INSTR + i) + lane;
        const int r = q / CL::CPR, part = (q % CL::CPR) ^ code_swz<BITS>(r);
        const int row = n0 + r % BNO;
        c_goff[i] = (q < BN * CL::CPR && row < N)
            ? (uint32_t)row * wrow_bytes + part * CL::CS : OOB;
        int t = 64 * (wave * C_INSTR + i) / (BNO * CL::CPR);
        t = t < NMAT ? t : NMAT - 1;
        rw[i] = rw_of(t);
    }
    // Scales / biases: instruction j = wave * SB_INSTR + i moves the dwords of
    // tile rows 64 (j % (BN / 64)) + lane, scales for j < BN / 64, else biases;
    // instructions j >= SBS::INSTR read zeros into spare slots.
    uint32_t sb_row[SB_INSTR];
    __amdgpu_buffer_rsrc_t rsb[SB_INSTR];
#pragma unroll
    for (int i = 0; i < SB_INSTR; ++i) {
        const int j = wave * SB_INSTR + i;
        const int r = 64 * (j % (BN / 64)) + lane;
        const int row = n0 + r % BNO;
        sb_row[i] = row < N && j < SBS::INSTR ? e_groups + (uint32_t)row * groups : 0x40000000u;
        rsb[i] = rsb_of(NMAT == 1 ? 0 : (r / BNO), MODE == 0 && j >= BN / 64);
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
            constexpr uint32_t ES = MODE == 0 ? 2 : 1;   // bytes per scale
            const uint32_t off = sb_row[i] < 0x40000000u ? ((sb_row[i] + g0) * ES) & ~3u : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsb[i],
                (__attribute__((address_space(3))) void*)(sb_st + stage * SB_STAGE +
                                                          (wave * SB_INSTR + i) * 256),
                4, off, 0, 0, 0);
        }
    };

    // B fragments of this lane: column block j is tile row bt[j] (its weight
    // row n0 + bt[j] % BNO of matrix bt[j] / BNO); the lane takes unit `half`
    // (codes 32 half .. 32 half + 31 of the step) of that row.
    int bt[FN];
    uint32_t b_gbase[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        if constexpr (NMAT == 1)
            bt[j] = wn * WN + j * 32 + (lane & 31);
        else
            bt[j] = (j / FNO) * BNO + wn * (WN / 2) + (j % FNO) * 32 + (lane & 31);
        const int row = n0 + bt[j] % BNO;
        b_gbase[j] = e_groups + (uint32_t)(row < N ? row : 0) * groups;
    }
    uint32_t wcode[FN][GC::NW];
    float s_u[FN], b_u[FN];
    // Microscaled modes: the unit's raw code words, and its scale bytes (one,
    // or two for 16-wide groups).
    constexpr int MX_SPU = MODE == 0 ? 1 : 32 / MxFmt<MODE == 0 ? 1 : MODE>::GS;
    uint32_t mx_w[FN][BITS];
    uint32_t mx_sb[FN][MX_SPU];
    // The unit's BITS words from C stage `stage`.
    auto read_unit = [&](int stage, int r, uint32_t (&w)[BITS]) {
        const char* row = c_st + stage * C_STAGE + r * CL::SLOT_ROW;
        const int sw = code_swz<BITS>(r);
        if constexpr (BITS == 4 || BITS == 3) {        // chunk `half` (16 or 12 bytes)
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + ((half ^ sw) << 4));
#pragma unroll
            for (int i = 0; i < BITS; ++i) w[i] = v[i];
        } else if constexpr (BITS == 8) {               // chunks 2 half, 2 half + 1
            const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(row + (((2 * half) ^ sw) << 4));
            const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(row + (((2 * half + 1) ^ sw) << 4));
#pragma unroll
            for (int i = 0; i < 4; ++i) { w[i] = v0[i]; w[4 + i] = v1[i]; }
        } else {                                        // 2-bit: 8 bytes; 6-bit: 24 bytes
#pragma unroll
            for (int i = 0; i < BITS / 2; ++i) {
                const u32x2_t v = *reinterpret_cast<const u32x2_t*>(row + half * 4 * BITS + 8 * i);
                w[2 * i] = v[0];
                w[2 * i + 1] = v[1];
            }
        }
    };
    // Codes and scale / bias of step kt (C / SB stage `stage`) for every
    // column block. The scale / bias dword holds elements (base & ~1) and
    // (base & ~1) + 1 of the array, base = the row's element of the step's
    // first group: with 32-wide groups (base even) both groups of the step,
    // else the step's one group in half base & 1.
    auto load_units = [&](int kt, int stage) {
        const uint32_t g0 = ((uint32_t)kt * BK) >> gshift;
        const uint32_t gu = ((uint32_t)kt * BK + half * 32) >> gshift;
        if constexpr (MODE != 0) {
            // The row's scale bytes of the step sit in one aligned dword, from
            // byte (b_gbase + g0) & 3 on; the lane's unit takes byte gu - g0
            // (and the next, for 16-wide groups) of the step's.
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                read_unit(stage, bt[j], mx_w[j]);
                const uint32_t sd = *reinterpret_cast<const uint32_t*>(sb_st + stage * SB_STAGE +
                                                                       bt[j] * 4);
                const uint32_t sh = ((b_gbase[j] + g0) & 3u) * 8 + (gu - g0) * 8;
#pragma unroll
                for (int g = 0; g < MX_SPU; ++g)
                    mx_sb[j][g] = (sd >> (sh + 8 * g)) & 0xFFu;
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            uint32_t w[BITS];
            read_unit(stage, bt[j], w);
            GC::split(w, wcode[j]);
            const char* sbp = sb_st + stage * SB_STAGE + bt[j] * 4;
            const uint32_t sd = *reinterpret_cast<const uint32_t*>(sbp);
            const uint32_t bd = *reinterpret_cast<const uint32_t*>(sbp + 4 * BN);
            const uint32_t sh = ((b_gbase[j] + gu) - ((b_gbase[j] + g0) & ~1u)) * 16;
            s_u[j] = Elem<DT>::to_f32((uint16_t)(sd >> sh));
            b_u[j] = Elem<DT>::to_f32((uint16_t)(bd >> sh));
        }
    };
    // B fragment of column block j for sub-step kk: codes 8 kk .. 8 kk + 7 of
    // the lane's unit, dequantized.
    auto make_bfrag = [&](auto J, auto KK) {
        constexpr int j = decltype(J)::value, kk = decltype(KK)::value;
        uint32_t packed[4];
        if constexpr (MODE != 0) {
            // Codes 8 kk .. 8 kk + 7 of the unit, converted exactly to fp32,
            // scaled by their group's scale (exact), rounded to the
            // activation type.
            constexpr int MXG = MODE == 0 ? 1 : MxFmt<MODE == 0 ? 1 : MODE>::GS;
            const uint32_t sbyte = mx_sb[j][(8 * kk) / MXG];
            float v[8];
            if constexpr (BITS == 4) {
                const uint32_t w = mx_w[j][kk];
                static_for<4>([&](auto B) {
                    constexpr int b = decltype(B)::value;
                    const f32x2_t p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, b);
                    v[2 * b] = p.x;
                    v[2 * b + 1] = p.y;
                });
            } else {
                static_for<2>([&](auto H) {
                    constexpr int h = decltype(H)::value;
                    const uint32_t w = mx_w[j][2 * kk + h];
                    const f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
                    const f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
                    v[4 * h] = lo.x; v[4 * h + 1] = lo.y; v[4 * h + 2] = hi.x; v[4 * h + 3] = hi.y;
                    // 0x7F / 0xFF convert to NaN; the pages' E4M3 reads +-480
                    // (fp32 0x43F00000, with the code's sign).
                    if (__builtin_expect((((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u) != 0u, 0)) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const float fix = __uint_as_float(0x43F00000u | ((w << (24 - 8 * c)) & 0x80000000u));
                            v[4 * h + c] = v[4 * h + c] != v[4 * h + c] ? fix : v[4 * h + c];
                        }
                    }
                });
            }
            static_for<4>([&](auto P) {
                constexpr int p = decltype(P)::value;
                packed[p] = T::pack2(mx_scaled<MODE == 0 ? 1 : MODE>(v[2 * p], sbyte),
                                     mx_scaled<MODE == 0 ? 1 : MODE>(v[2 * p + 1], sbyte));
            });
            return __builtin_bit_cast(frag_t, u32x4_t{packed[0], packed[1], packed[2], packed[3]});
        }
        float q[8];
        GC::template codes8<kk>(wcode[j], q);
        static_for<4>([&](auto P) {
            constexpr int p = decltype(P)::value;
            const float w0 = __builtin_fmaf(q[2 * p], s_u[j], b_u[j]);
            const float w1 = __builtin_fmaf(q[2 * p + 1], s_u[j], b_u[j]);
            packed[p] = T::pack2(w0, w1);
        });
        return __builtin_bit_cast(frag_t, u32x4_t{packed[0], packed[1], packed[2], packed[3]});
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

    // Prologue: the DMA of steps 1 - NC .. -1 of the loop below (activations
    // of steps 0 .. NA-2, codes / scales of steps 0 .. NC-2, in the loop's
    // order, so the loop's in-flight counts hold from its first step).
    const int KT = K / BK;
#pragma unroll
    for (int s = 1 - NC; s < 0; ++s) {
        if (s + NA - 1 >= 0)
            dma_a(s + NA - 1, s + NA - 1);
        dma_c(s + NC - 1, s + NC - 1);
    }
    step_barrier(std::integral_constant<int, IN_FLIGHT>{});

    frag_t af[2][FM], bfr[2][FN];
    auto load_afrags = [&](int stage, int kk, frag_t (&fa)[FM]) {
        const char* abase = a_st + stage * A_STAGE;
        const int chunk = kk + 4 * half;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            fa[i] = *reinterpret_cast<const frag_t*>(
                abase + lds_off(wm * WM + i * 32 + (lane & 31), chunk));
    };
    load_units(0, 0);
    load_afrags(0, 0, af[0]);
    static_for<FN>([&](auto J) { bfr[0][J] = make_bfrag(J, std::integral_constant<int, 0>{}); });

    int a_cur = 0, c_cur = 0;          // A and C stages of step kt
    for (int kt = 0; kt < KT; ++kt) {
        const int a_new = a_cur == 0 ? NA - 1 : a_cur - 1;
        const int c_new = c_cur == 0 ? NC - 1 : c_cur - 1;
        const int a_nxt = a_cur + 1 == NA ? 0 : a_cur + 1;
        const int c_nxt = c_cur + 1 == NC ? 0 : c_cur + 1;
        dma_a(kt + NA - 1, a_new);
        dma_c(kt + NC - 1, c_new);
        static_for<BK / 16>([&](auto KK) {
            constexpr int kk = decltype(KK)::value;
            if constexpr (kk + 1 < BK / 16)
                load_afrags(a_cur, kk + 1, af[(kk + 1) & 1]);
            else
                load_afrags(a_nxt, 0, af[0]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = T::mfma(af[kk & 1][i], bfr[kk & 1][j], acc[i][j]);
            if constexpr (kk + 1 < BK / 16) {
                static_for<FN>([&](auto J) {
                    bfr[(kk + 1) & 1][J] = make_bfrag(J, std::integral_constant<int, kk + 1>{});
                });
                if constexpr (kk + 2 == BK / 16)
                    load_units(kt + 1, c_nxt);
            } else {
                static_for<FN>([&](auto J) {
                    bfr[0][J] = make_bfrag(J, std::integral_constant<int, 0>{});
                });
            }
        });
        step_barrier(std::integral_constant<int, IN_FLIGHT>{});
        a_cur = a_nxt;
        c_cur = c_nxt;
    }
    // No DMA of this tile may still be writing the block's LDS when the
    // block ends or its next tile's DMA starts.
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
            const int row = wm * WM + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
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
    // Every wave leaves the tile before any starts the next one's DMA.
    __builtin_amdgcn_s_barrier();
    } // the tile loop (its body is left at the kernel's indentation)
}

} // namespace gemm

} // namespace qp
