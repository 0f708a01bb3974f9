// qgemm.hip — prefill path (M > 16): y = x @ dequant(W)^T on the matrix cores.
//
// The product is the one of emily lib/emily/quantization.ex, `quantized_matmul/2`
// (x [M, K] times the packed [N, K] weight, transposed); at M in the hundreds
// or thousands it is a dense contraction (2048 x 14336 x 4096 is 240 GFLOP over
// 33 MB of weights), so it runs on bf16 / fp16 MFMA:
//  - block tile BM x BN x 64 (two 32-code units of every weight row per step),
//    four waves in 2 x 2, each wave a (BM/2) x (BN/2) tile of
//    v_mfma_f32_32x32x16 instructions accumulating in fp32;
//  - each step, the block stages its activation tile [BM][64] and its weight
//    tile [BN][64] in LDS: weight codes are unpacked (emily `dequantize_defn/1`
//    layout) and dequantized in fp32 (q * s' + b') then rounded to the
//    activation type, so every weight is dequantized once per block row;
//  - two LDS stages (128 KB at 256 x 256): the next step's global loads are
//    issued before the current step's MFMAs and written to the other stage
//    interleaved with them (one barrier per step, no branch in the loop body);
//  - LDS rows are 128 bytes (64 x 16-bit); 16-byte chunks are XOR-swizzled by
//    (row / 2) % 8 so that the 16 rows one 16-lane phase of a fragment read
//    touches at one chunk hit distinct banks;
//  - all global accesses are raw buffer accesses: rows past M or N read zeros
//    and their stores drop, so ragged shapes need no branches;
//  - blocks are mapped to tiles XCD by XCD (block b runs on XCD b % 8), each
//    XCD taking a contiguous run of tiles in row-major tile order, so blocks
//    that share an activation strip share an L2.
#include "common.hpp"
#include "launch.hpp"

namespace qp {

namespace {

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

template <int BITS, int DT, int BM, int BN, int THREADS>
__global__ __launch_bounds__(THREADS) void qgemm_kernel(const void* __restrict__ x,
                                                        const uint32_t* __restrict__ wq,
                                                        const void* __restrict__ scales,
                                                        const void* __restrict__ biases,
                                                        void* __restrict__ y, int M, int N, int K,
                                                        int gs, int tiles_n, int tiles,
                                                        int per_xcd)
{
    using T = MfmaTraits<DT>;
    using frag_t = typename T::frag_t;
    constexpr int WAVES = THREADS / 64;
    struct CL : CodeLayout<BITS>, CodeStage<BITS, BN, WAVES> {};
    constexpr int WGN = WAVES / 2;               // waves: 2 along M x WGN along N
    constexpr int WM = BM / 2, WN = BN / WGN;    // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;    // 32 x 32 MFMA tiles per wave
    constexpr int UPT = 2 * BN / THREADS;        // weight units per thread per step
    static_assert(BN == THREADS || BN == THREADS / 2, "a weight row per one or two threads");
    constexpr int A_STAGE = BM * ROW_BYTES, B_STAGE = BN * ROW_BYTES;
    constexpr int A_INSTR = A_STAGE / 1024 / WAVES;        // 1 KB DMA instructions per wave
    constexpr int C_INSTR = CL::INSTR;                      // per wave (64 chunks each)
    // Every DMA instruction writes 64 x 16 bytes, so a codes stage spans whole
    // 4 KB blocks (chunks past the tile read zeros into the spare slots).
    constexpr int C_STAGE = CL::STAGE;
    // LDS: A[2] | B[2] | C[2]
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char* const a_st = lds;
    char* const b_st = lds + 2 * A_STAGE;
    char* const c_st = b_st + 2 * B_STAGE;

    // Tile of this block, XCD by XCD.
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    if (local >= per_xcd)
        return;
    const int tile = xcd * per_xcd + local;
    if (tile >= tiles)
        return;
    const int tm = tile / tiles_n, tn = tile % tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    const uint32_t xrow_bytes = (uint32_t)K * 2;
    const uint32_t wrow_bytes = (uint32_t)K * BITS / 8;
    const uint32_t groups = (uint32_t)(K / gs);
    const __amdgpu_buffer_rsrc_t rx = rsrc(x, (uint32_t)M * xrow_bytes);
    const __amdgpu_buffer_rsrc_t rw = rsrc(wq, (uint32_t)N * wrow_bytes);
    const __amdgpu_buffer_rsrc_t rs = rsrc(scales, (uint32_t)N * groups * 2);
    const __amdgpu_buffer_rsrc_t rb = rsrc(biases, (uint32_t)N * groups * 2);

    // DMA plan. Activations: wave w's instruction i moves rows 8g..8g+7 of the
    // tile (g = 8w + i for BM = 256) into 1 KB of LDS; lane l lands in slot l
    // = (row 8g + l/8, physical chunk l%8), so it reads logical chunk
    // (l%8) ^ swz(row) of that row. Rows past M read zeros.
    uint32_t a_goff[A_INSTR];
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
        const int g = wave * A_INSTR + i, r = 8 * g + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        a_goff[i] = m0 + r < M ? (uint32_t)(m0 + r) * xrow_bytes + c * 16 : 0x80000000u;
    }
    // Codes: flat chunk q = 64 * (wave * C_INSTR + i) + lane -> row q / CPR,
    // part q % CPR; LDS slot q.
    uint32_t c_goff[C_INSTR];
#pragma unroll
    for (int i = 0; i < C_INSTR; ++i) {
        const int q = 64 * (wave * C_INSTR + i) + lane;
        const int r = q / CL::CPR, part = q % CL::CPR;
        c_goff[i] = (q < BN * CL::CPR && n0 + r < N)
            ? (uint32_t)(n0 + r) * wrow_bytes + part * CL::CS : 0x80000000u;
    }
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
                dma12(rw, dst, off);
            else
                dma16(rw, dst, off);
        }
    };

    // Dequantization work of this thread: row b_r, units [u0, u0 + UPT).
    const int b_r = tid % BN;
    const int u0 = (tid / BN) * UPT;
    const uint32_t b_soff = n0 + b_r < N ? (uint32_t)(n0 + b_r) * groups * 2 : 0x80000000u;
    const uint32_t gshift = (uint32_t)__builtin_ctz((unsigned)gs);
    uint16_t s_next[UPT], b_next[UPT];
    auto load_sb = [&](int kt) {
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const uint32_t g = (uint32_t)(kt * BK + (u0 + u) * 32) >> gshift;
            s_next[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, b_soff + g * 2, 0, 0);
            b_next[u] = __builtin_amdgcn_raw_buffer_load_b16(rb, b_soff + g * 2, 0, 0);
        }
    };
    // Codes of step kt (C stage kt % 2) -> activation-typed weights in B stage
    // kt % 2, in slices: slice `part` (0..3) writes 16-byte chunk `part` of each
    // of this thread's units, so the work can be spread over the MFMA phases.
    using CB = CodeBytes<BITS>;
    uint32_t wcode[UPT][CB::NBW];
    auto load_codes = [&](int stage) {
        const char* crow = c_st + stage * C_STAGE + b_r * CL::SLOT_ROW;
        static_for<UPT>([&](auto U) {
            const char* src = crow + (BITS == 3 ? (u0 + U) * 16 : (u0 + U) * 4 * BITS);
            uint32_t w[BITS];
#pragma unroll
            for (int i = 0; i < BITS; ++i)
                w[i] = reinterpret_cast<const uint32_t*>(src)[i];
            CB::split(w, wcode[U]);
        });
    };
    auto dequant_part = [&](int stage, auto PART, const uint16_t (&sv)[UPT],
                            const uint16_t (&bv)[UPT]) {
        char* brow = b_st + stage * B_STAGE;
        static_for<UPT>([&](auto U) {
            const float s = Elem<DT>::to_f32(sv[U]), b = Elem<DT>::to_f32(bv[U]);
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
    auto dequant = [&](int stage, const uint16_t (&sv)[UPT], const uint16_t (&bv)[UPT]) {
        load_codes(stage);
        static_for<4>([&](auto PART) { dequant_part(stage, PART, sv, bv); });
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x16_t{};

    // Prologue: codes of steps 0 and 1, activations of step 0, B of step 0.
    const int KT = K / BK;
    uint16_t s_cur[UPT], b_cur[UPT];
    dma_c(0, 0);
    dma_c(1, 1);
    dma_a(0, 0);
    load_sb(0);
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int u = 0; u < UPT; ++u) { s_cur[u] = s_next[u]; b_cur[u] = b_next[u]; }
    __syncthreads();
    dequant(0, s_cur, b_cur);
    load_sb(1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1, nxt = cur ^ 1;
        // In flight during this step: activations of kt + 1, codes of kt + 2,
        // scales / biases of kt + 2 (reads past the last step are harmless:
        // in-range bytes that are never used, or zeros).
#pragma unroll
        for (int u = 0; u < UPT; ++u) { s_cur[u] = s_next[u]; b_cur[u] = b_next[u]; }
        dma_a(kt + 1, nxt);
        dma_c(kt + 2, cur);
        load_sb(kt + 2);
        // MFMAs on stage cur, fragments double-buffered across the four k16
        // sub-steps; after each sub-step's MFMAs, a quarter of the weights of
        // step kt + 1 is dequantized (from codes that arrived during the
        // previous step).
        const char* abase = a_st + cur * A_STAGE;
        const char* bbase = b_st + cur * B_STAGE;
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
                    bbase + lds_off(wn * WN + j * 32 + (lane & 31), chunk));
        };
        load_frags(0, af[0], bfr[0]);
        load_codes(nxt);
        static_for<BK / 16>([&](auto KK) {
            constexpr int kk = decltype(KK)::value;
            if constexpr (kk + 1 < BK / 16)
                load_frags(kk + 1, af[(kk + 1) & 1], bfr[(kk + 1) & 1]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = T::mfma(af[kk & 1][i], bfr[kk & 1][j], acc[i][j]);
            dequant_part(nxt, KK, s_cur, b_cur);
        });
        __builtin_amdgcn_s_waitcnt(0); // this step's DMA and loads have landed
        __syncthreads();
    }

    // Epilogue: lane l, register r of a 32 x 32 tile holds
    // row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32.
    const __amdgpu_buffer_rsrc_t ry = rsrc(y, (uint32_t)M * (uint32_t)N * 2);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WN + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const uint32_t off = (row < M && col < N)
                    ? ((uint32_t)row * (uint32_t)N + (uint32_t)col) * 2 : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b16(Elem<DT>::from_f32(acc[i][j][r]), ry, off,
                                                      0, 0);
            }
        }
}

template <int BITS, int DT, int BM, int BN, int NT>
hipError_t run_gemm(const GemvArgs& a, hipStream_t st)
{
    constexpr int LDS = 2 * (BM + BN) * ROW_BYTES + 2 * CodeStage<BITS, BN, NT / 64>::STAGE;
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static bool attr_set = false; // per instantiation; set before its first launch
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&qgemm_kernel<BITS, DT, BM, BN, NT>),
            hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    const int tiles_m = (int)((a.M + BM - 1) / BM), tiles_n = (int)((a.N + BN - 1) / BN);
    const int tiles = tiles_m * tiles_n;
    const int per_xcd = (tiles + 7) / 8;
    hipLaunchKernelGGL((qgemm_kernel<BITS, DT, BM, BN, NT>), dim3(per_xcd * 8), dim3(NT), LDS, st,
                       a.x, a.wq, a.scales, a.biases, a.y, (int)a.M, (int)a.N, (int)a.K, a.gs,
                       tiles_n, tiles, per_xcd);
    return hipGetLastError();
}

template <int DT>
hipError_t run_gemm_dt(const GemvArgs& a, hipStream_t st)
{
    // Wide tiles (eight waves, two per SIMD) when there are enough of them to
    // fill the 256 CUs; otherwise 256 x 128 tiles with four waves.
    const bool wide = ((a.M + 255) / 256) * ((a.N + 255) / 256) >= 384;
    switch (a.bits) {
    case 2: return wide ? run_gemm<2, DT, 256, 256, 512>(a, st) : run_gemm<2, DT, 256, 128, 256>(a, st);
    case 3: return wide ? run_gemm<3, DT, 256, 256, 512>(a, st) : run_gemm<3, DT, 256, 128, 256>(a, st);
    case 4: return wide ? run_gemm<4, DT, 256, 256, 512>(a, st) : run_gemm<4, DT, 256, 128, 256>(a, st);
    case 6: return wide ? run_gemm<6, DT, 256, 256, 512>(a, st) : run_gemm<6, DT, 256, 128, 256>(a, st);
    case 8: return wide ? run_gemm<8, DT, 256, 256, 512>(a, st) : run_gemm<8, DT, 256, 128, 256>(a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_qgemm(const GemvArgs& a, hipStream_t stream)
{
    // 32-bit buffer offsets: every operand below 2 GB, and whole 64-wide k
    // steps; otherwise the GEMV path (in chunks of activation rows) covers
    // the shape.
    const bool fits = a.K % BK == 0 && a.M * a.K * 2 < (int64_t(1) << 31) &&
                      a.N * (a.K * a.bits / 8) < (int64_t(1) << 31) &&
                      a.M * a.N * 2 < (int64_t(1) << 31) && a.K < (int64_t(1) << 30);
    if (!fits)
        return launch_qgemv(a, stream);
    if (a.dt == DT_BF16)
        return run_gemm_dt<DT_BF16>(a, stream);
    if (a.dt == DT_F16)
        return run_gemm_dt<DT_F16>(a, stream);
    return launch_qgemv(a, stream);
}

} // namespace qp
