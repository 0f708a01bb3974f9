// launch.hpp — host-side launchers implemented by the kernel files and
// called by the C ABI layer (api.cpp). Arguments are validated by the caller;
// every launcher returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace qp {

// Compute units of the current device, asked of the runtime once per device
// and kept (persistent grids are sized from it).
inline hipError_t device_cu_count(int* cus)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    if (cached) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return hipSuccess;
        }
    }
    e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess && cached && *cus > 0)
        cache[dev].store(*cus, std::memory_order_relaxed);
    return e;
}

struct GemvArgs {
    const void* x;          // [M, K] activations
    int dt;                 // element type of x, scales, biases and y
    int64_t M, K, N;
    const uint32_t* wq;     // [N, K*bits/32]
    const void* scales;     // [N, K/gs]
    const void* biases;     // [N, K/gs]
    int bits, gs;
    void* y;                // [M, N]
};

#define QP_CAT_(a, b) a##b
#define QP_CAT(a, b) QP_CAT_(a, b)

// Decode GEMV (M <= 16): weights streamed once per launch group. One entry
// point per bit width (each in its own translation unit), plus a dispatcher.
hipError_t launch_qgemv_b2(const GemvArgs& a, hipStream_t stream);
hipError_t launch_qgemv_b3(const GemvArgs& a, hipStream_t stream);
hipError_t launch_qgemv_b4(const GemvArgs& a, hipStream_t stream);
hipError_t launch_qgemv_b6(const GemvArgs& a, hipStream_t stream);
hipError_t launch_qgemv_b8(const GemvArgs& a, hipStream_t stream);
hipError_t launch_qgemv(const GemvArgs& a, hipStream_t stream);

// Prefill GEMM (M > 16, 16-bit activations): bf16/f16 MFMA.
hipError_t launch_qgemm(const GemvArgs& a, hipStream_t stream);

// Writes zeros to `n` elements of `dt` (used for K == 0).
hipError_t launch_fill_zero(void* p, int dt, int64_t n, hipStream_t stream);

struct QuantizeArgs {
    const float* w;         // [N, K]
    int64_t N, K;
    int bits, gs, dt;       // dt: storage type of scales / biases
    uint32_t* wq;
    void* scales;
    void* biases;
};
hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream);

struct DequantArgs {
    const uint32_t* wq;     // [N, K*bits/32]
    const void* scales;     // [N, K/gs] of sdt
    const void* biases;
    int sdt, odt;           // scales' type; output type (DT_F32, or sdt)
    int64_t N, K;
    int bits, gs;
    void* out;              // [N, K] of odt
};
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t stream);

// Microscaled modes (mode 1 mxfp4, 2 mxfp8, 3 nvfp4; see mx.hpp).
struct DequantMxArgs {
    const uint32_t* wq;     // [N, K*bits/32]
    const uint8_t* scales;  // [N, K/gs]
    int mode, odt;
    int64_t N, K;
    void* out;              // [N, K] of odt
};
hipError_t launch_dequantize_mx(const DequantMxArgs& a, hipStream_t stream);

struct GemvMxArgs {
    const void* x;          // [M, K] of dt
    int dt, mode;
    int64_t M, K, N;
    const uint32_t* wq;     // [N, K*bits/32]
    const uint8_t* scales;  // [N, K/gs]
    void* y;                // [M, N] of dt
};
hipError_t launch_qmatmul_mx(const GemvMxArgs& a, hipStream_t stream);
// Prefill tiles for the microscaled modes (qgemm.hip): 16-bit activations,
// K a multiple of 64, 4-byte aligned scales, operands below 2 GB.
bool qgemm_mx_fits(const GemvMxArgs& a);
hipError_t launch_qgemm_mx(const GemvMxArgs& a, hipStream_t stream);

struct MoeArgs {
    const void* a;          // activations
    int dt;
    const int32_t* ids;     // [P]
    int64_t n_tokens, top_k, a_outer, a_inner;
    const uint32_t* wq[2];  // expert stacks: [E, n_rows, n_cols*bits/32]; [1] = up (fused)
    const void* scales[2];
    const void* biases[2];
    int64_t E, n_rows, n_cols;
    int bits, gs;
    bool fused_silu;        // out = SiLU(gate) * up
    void* out;              // [P, n_rows]
    void* workspace;
    size_t ws_bytes;
};
size_t moe_workspace_bytes(int64_t n_pairs, int64_t num_experts);
// Routing (moe.hip) and the per-(bits, fused) compute entry points
// (moe_compute.hip, one translation unit each).
struct MoeRouting {
    const int32_t* n_tiles; // device tile count (null: pair t is tile t, see moe.hip)
    const int32_t* perm;    // pair indices in expert order
    const void* tiles;      // TileDesc list
    int mt;                 // tile height
    int64_t max_tiles;      // upper bound of the tile count
    int nb;                 // > 0: matrix-core tiles of 16 * nb pairs (mt == 16 * nb)
    int gemm_bm;            // > 0: routed GEMM tiles of gemm_bm pairs (mt == gemm_bm)
    int rowmfma;            // > 0: four-row matrix-instruction tiles of mt <= 8 pairs
    int rowstream;          // > 0: one-pair tiles on the dot-product row kernel (mt == 1)
};
hipError_t launch_moe_route(const MoeArgs& a, int mt, MoeRouting* r, hipStream_t stream);
int moe_tile_height(int64_t n_pairs, int64_t num_experts, int bits, int dt);
// Column blocks of 16 pairs per matrix-core tile for this call, or 0 when the
// streaming kernel takes it (fp32 activations, few pairs per expert, or
// operands the 16-byte / 32-bit-offset accesses cannot cover).
int moe_mfma_nb(const MoeArgs& a);
// Tile height (8) when the routed tiles go to the four-row matrix-instruction
// kernel (the fused gate + up form, 2-, 4- and 8-bit codes, 16-bit
// activations, K <= 2048, two to four pairs per expert), else 0.
int moe_rowmfma_mt(const MoeArgs& a);
// True when one-pair tiles go to the dot-product row kernel (2-, 4- and 8-bit
// codes, 16-bit activations, K <= 4096, one tile per pair, few pairs per
// expert).
bool moe_rowstream_ok(const MoeArgs& a, int mt);
// Pairs per routed-GEMM tile for this call, or 0 when the GEMV kernels take
// it (fp32 activations, few pairs per expert, K not a multiple of 64, or
// operands the 16-byte / 32-bit-offset accesses cannot cover).
int moe_gemm_bm(const MoeArgs& a);
#define QP_MOE_DECL(B)                                                                          \
    hipError_t launch_moe_b##B##_n1(const MoeArgs& a, const MoeRouting& r, hipStream_t stream); \
    hipError_t launch_moe_b##B##_n2(const MoeArgs& a, const MoeRouting& r, hipStream_t stream);
QP_MOE_DECL(2)
QP_MOE_DECL(3)
QP_MOE_DECL(4)
QP_MOE_DECL(6)
QP_MOE_DECL(8)
#undef QP_MOE_DECL
hipError_t launch_moe(const MoeArgs& a, hipStream_t stream);
// Two MoE calls over the same ids, pairs and experts, in stream order (the
// FFN block's gate + up, then down): one routing pass when both take the same
// tile height, two otherwise. Both use a's workspace for the tables.
hipError_t launch_moe_pair(const MoeArgs& a, const MoeArgs& b, hipStream_t stream);

// The transpose = false product (qgemv_t.hip): W stored [K, N], grouped along
// N; fp32 partial sums of the K splits in `workspace`.
struct QgemvTArgs {
    const void* x;          // [M, K] of dt
    int dt;
    int64_t M, K, N;
    const uint32_t* wq;     // [K, N*bits/32]
    const void* scales;     // [K, N/gs] of dt
    const void* biases;
    int bits, gs;
    void* y;                // [M, N] of dt
    float* workspace;       // >= qgemv_t_plan(...).workspace_bytes
};
struct QgemvTPlan {
    int splits, rows_per_split;
    size_t workspace_bytes;
};
// Activation rows per pass over the weights (the LDS of the split reduction
// holds 3 x rows x columns-per-lane x 64 floats).
constexpr int qgemv_t_rows(int bits) { return (bits == 3 || bits == 6) ? 2 : 4; }
QgemvTPlan qgemv_t_plan(int64_t m, int64_t k, int64_t n, int bits);
hipError_t launch_qgemv_t(const QgemvTArgs& a, hipStream_t stream);

// Per-tensor dynamic-range int8 (int8_tensor.hip). `range` is the device
// pair [lo, hi]; the quantizer uses it as scratch for its reduction keys.
hipError_t launch_quantize_int8_tensor(const float* w, int64_t count, int8_t* q, float* range,
                                       hipStream_t stream);
hipError_t launch_dequantize_int8_tensor(const int8_t* q, int64_t count, const float* range,
                                         int odt, void* out, hipStream_t stream);
struct Int8TensorArgs {
    const void* x;          // [M, K] of dt
    int dt;
    int64_t M, K, N;
    const int8_t* q;        // [N, K]
    const float* range;     // [2] device
    void* y;                // [M, N] of dt
};
hipError_t launch_qmatmul_int8_tensor(const Int8TensorArgs& a, hipStream_t stream);

// Weighted slot sum closing an MoE FFN block (moe_ffn.hip).
struct MoeCombineArgs {
    const void* o;          // [n_tokens * top_k, d_model] of dt
    const int32_t* ids;     // [n_tokens * top_k]
    const float* rw;        // [n_tokens * top_k] router weights
    int64_t n_tokens, top_k, d_model, E;
    int dt;
    void* out;              // [n_tokens, d_model] of dt
};
hipError_t launch_moe_combine(const MoeCombineArgs& a, hipStream_t stream);

// The down projection of an MoE block fused with the slot combine, for few
// tokens (one pair per tile; moe_rows.hpp, `qgemv_moe_rowcombine_kernel`):
// out[t, r] = sum_j rw[t*top_k + j] * round(h[t*top_k + j] . W[ids][r]), the
// same result as launch_moe on `dn` followed by launch_moe_combine. `dn` is the
// plain (not fused) down call; out is [n_tokens, dn.n_rows] of dn.dt.
constexpr int kMoeCombineMaxTopK = 8;
bool moe_down_combine_ok(const MoeArgs& dn);
hipError_t launch_moe_down_combine(const MoeArgs& dn, const float* rw, void* out, hipStream_t stream);
#define QP_MOE_DC_DECL(B) \
    hipError_t launch_moe_b##B##_dc(const MoeArgs& a, const float* rw, void* out, hipStream_t stream);
QP_MOE_DC_DECL(2)
QP_MOE_DC_DECL(4)
QP_MOE_DC_DECL(8)
#undef QP_MOE_DC_DECL

} // namespace qp
