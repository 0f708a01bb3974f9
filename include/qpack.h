/*
 * qpack.h — C ABI of libqpack.so: weight-only quantized linear layers on
 * MI355X (gfx950).
 *
 *   y = x @ dequant(W)^T,   dequant(W)[n, k] = q[n, k] * scale[n, g] + bias[n, g],
 *   g = k / group_size,
 *
 * with W stored as packed b-bit codes (b in {2, 3, 4, 6, 8}) and one scale and
 * one bias per group of `group_size` consecutive elements along K.
 *
 * Sources (the surveyed pages):
 *  - emily lib/emily/quantization.ex, `quantized_matmul/2` docs: the product
 *    x @ W^T with W packed row-major [N, K] ("transpose = true"), and the rule
 *    that the input dtype must equal the scales dtype (affine mode).
 *  - same page, `dequantize_defn/1` docs and its unpack helpers: lane i of a
 *    row sits at bit offset i*bits of the row's little-endian u32 stream,
 *    masked to `bits` bits; 3- and 6-bit lanes may straddle two words; the
 *    packed length must satisfy K*bits % 32 == 0; groups run along the last
 *    axis (K % group_size == 0).
 *  - ollama x/create/client/quantize.go, `quantizeParams` and
 *    `loadAndQuantizeArray`: quantize(w, group_size, bits, mode) returns
 *    (codes, scales, biases); int4 = {64, 4, affine}, int8 = {64, 8, affine}.
 *  - ferrum-kernels src/stacked_expert.rs, `StackedExpertGgufLinear` docs:
 *    the MoE calls `gemv_moe_id` / `gemv_moe_id_batched` (pair p reads
 *    a[(p/top_k)*outer + (p%top_k)*inner] and expert ids[p]) and
 *    `gemv_moe_id_gate_up_silu` (SiLU(gate) * up in one dispatch).
 *
 * Conventions for every call:
 *  - Pointers marked "device" are HIP device (or managed) memory; the caller
 *    allocates and frees every buffer. The library never allocates device
 *    memory.
 *  - Calls are asynchronous on `stream` (0 = the null stream): they validate
 *    on the host, enqueue kernels and return. There is no host synchronisation
 *    and no device-to-host copy.
 *  - Errors are returned as qp_status; nothing is thrown. On an error no work
 *    is enqueued and qpack_last_error() (thread-local) describes it. Argument
 *    checks run before any HIP call, so they work without a GPU.
 *  - All arrays are row-major and densely packed (no row strides except the
 *    MoE activation strides).
 *  - Element types: QP_F32, QP_F16 (IEEE binary16), QP_BF16. 16-bit outputs
 *    are rounded to nearest even from an fp32 accumulator.
 */
#ifndef QPACK_H
#define QPACK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums are int-sized in C and C++ alike; in C++ they have int as their
 * fixed underlying type, so that any int a caller passes (an out-of-range
 * one included, which the calls reject) is a valid value of the type. */
#ifdef __cplusplus
#define QP_ENUM(name) enum name : int
#else
#define QP_ENUM(name) enum name
#endif

typedef QP_ENUM(qp_status) {
    QP_OK = 0,
    QP_ERR_INVALID_ARG = 1,    /* null pointer, negative size, size overflow */
    QP_ERR_UNSUPPORTED = 2,    /* bits not in {2,3,4,6,8}, group_size not in {32,64,128} */
    QP_ERR_DTYPE_MISMATCH = 3, /* activation dtype != scales dtype */
    QP_ERR_SHAPE = 4,          /* K % group_size != 0, K*bits % 32 != 0, gate/up mismatch */
    QP_ERR_ALIGN = 5,          /* a pointer not aligned to its element size */
    QP_ERR_WORKSPACE = 6,      /* MoE workspace too small */
    QP_ERR_HIP = 7             /* a HIP launch failed */
} qp_status;

typedef QP_ENUM(qp_dtype) { QP_F32 = 0, QP_F16 = 1, QP_BF16 = 2 } qp_dtype;

/* Microscaled modes (emily "Defn-native dequantize", the mxfp4 / mxfp8 /
 * nvfp4 implementations; group sizes as in ollama quantize.go
 * `quantizeParams`): no biases, one scale byte per group of lanes.
 *   QP_MXFP4: 4-bit FP4-E2M1 lanes, groups of 32, FP8-E8M0 scales 2^(s-127);
 *   QP_MXFP8: 8-bit FP8-E4M3 lanes, groups of 32, FP8-E8M0 scales;
 *   QP_NVFP4: 4-bit FP4-E2M1 lanes, groups of 16, FP8-E4M3 scales.
 * FP8-E4M3 is decoded as MLX decodes it: bias 7, subnormals, and no NaN
 * (0x7F / 0xFF are +-480). Lanes are packed as in the affine mode. */
typedef QP_ENUM(qp_mode) { QP_MXFP4 = 1, QP_MXFP8 = 2, QP_NVFP4 = 3 } qp_mode;

/*
 * Affine group quantization (ollama quantize.go `loadAndQuantizeArray`,
 * emily `QuantizedWeight.from_dense/2`), computed on the device.
 *   w       device, fp32 [n, k]                       (input)
 *   wq      device, u32 [n, k*bits/32]                (output, packed codes)
 *   scales  device, sb_dtype [n, k/group_size]        (output)
 *   biases  device, sb_dtype [n, k/group_size]        (output)
 * Per row and group: mn/mx = group min/max; s = (mx - mn) / (2^bits - 1) in
 * fp32, floored at FLT_EPSILON; stored s' = RNE(s), b' = RNE(mn) (a zero bias
 * is stored as +0); q = clamp(round_half_away((w - b') / s'), 0, 2^bits - 1);
 * lane i of the row goes to bits [i*bits, i*bits + bits) of the row's u32
 * stream. Inputs must be finite; with fp16 storage, |scale| and |bias| must
 * stay below 65504. Deterministic: the output does not depend on the launch.
 * n == 0 or k == 0 is a no-op.
 */
qp_status qpack_quantize(const float* w, int64_t n, int64_t k, int32_t bits,
                         int32_t group_size, qp_dtype sb_dtype, uint32_t* wq,
                         void* scales, void* biases, hipStream_t stream);

/*
 * Dense weight (emily "Defn-native dequantize": `dequantize_defn/1` and its
 * affine `dequantize_impl`, the math of `QuantizedWeight.to_dense/1`):
 *   w[r, i] = q[r, i] * s'[r, i/gs] + b'[r, i/gs],  q = bits [i*bits, i*bits + bits)
 *   of row r's u32 stream
 *   wq      device, u32 [n, k*bits/32]
 *   scales, biases  device, sb_dtype [n, k/group_size]
 *   out     device, out_dtype [n, k] (output)
 * out_dtype QP_F32: fp32(q) * s' + b', a multiply and then an add in fp32
 * (the weight qmatmul's product is defined on). out_dtype == sb_dtype (16-bit):
 * the code cast to that type, then the product and the sum each rounded to
 * nearest-even in that type, as the pages' affine step computes in the
 * scales' type. Any other out_dtype is QP_ERR_DTYPE_MISMATCH; k above 2^33 is
 * QP_ERR_UNSUPPORTED. Deterministic
 * and exact to these definitions on any launch. n == 0 or k == 0 is a no-op.
 */
qp_status qpack_dequantize(const uint32_t* wq, const void* scales, const void* biases,
                           qp_dtype sb_dtype, int64_t n, int64_t k, int32_t bits,
                           int32_t group_size, qp_dtype out_dtype, void* out,
                           hipStream_t stream);

/*
 * Dense weight of a microscaled mode: w[r, i] = lane(q[r, i]) * scale(s[r, i/gs]),
 * exact in fp32 (every lane times every scale up to 2^127 is an fp32 value;
 * E8M0 byte 255 is 2^128 and gives +-inf, or 0 for a zero lane), rounded to
 * nearest even in out_dtype (QP_F32, QP_F16 or QP_BF16; the pages' output is
 * bf16).
 *   wq      device, u32 [n, k*bits/32]
 *   scales  device, u8 [n, k/gs]
 *   out     device, out_dtype [n, k] (output)
 * k must be a multiple of the mode's group size (QP_ERR_SHAPE). n == 0 or
 * k == 0 is a no-op.
 */
qp_status qpack_dequantize_mx(const uint32_t* wq, const uint8_t* scales, qp_mode mode,
                              int64_t n, int64_t k, qp_dtype out_dtype, void* out,
                              hipStream_t stream);

/*
 * Quantized linear in a microscaled mode (emily `quantized_matmul/2` with
 * mode mxfp4 / mxfp8 / nvfp4, transpose = true):
 *   y[m, n] = sum_k x[m, k] * lane(q[n, k]) * scale(s[n, k/gs])
 *   x       device, x_dtype [m, k] (any of QP_F32, QP_F16, QP_BF16)
 *   wq      device, u32 [n, k*bits/32];  scales  device, u8 [n, k/gs]
 *   y       device, x_dtype [m, n] (output)
 * fp32 accumulation; every dense weight must be finite in fp32. 16-bit x
 * with k a multiple of 32 up to 16384 and x 16-byte aligned runs the stream
 * kernel (codes converted by the gfx950 FP4 / FP8 instructions, dot2
 * products), one or two activation rows per pass over the weights; every
 * other call runs the generic kernel (one wave per output). k == 0 writes
 * zeros; m == 0 or n == 0 is a no-op.
 */
qp_status qmatmul_mx(const void* x, qp_dtype x_dtype, int64_t m, int64_t k,
                     const uint32_t* wq, const uint8_t* scales, qp_mode mode, int64_t n,
                     void* y, hipStream_t stream);

/*
 * Quantized linear (emily `quantized_matmul/2`, transpose = true):
 *   y[m, n] = sum_k x[m, k] * (q[n, k] * s'[n, k/gs] + b'[n, k/gs])
 *   x       device, x_dtype [m, k]
 *   wq      device, u32 [n, k*bits/32]
 *   scales, biases  device, sb_dtype [n, k/group_size]; sb_dtype must equal
 *           x_dtype (QP_ERR_DTYPE_MISMATCH otherwise)
 *   y       device, x_dtype [m, n] (output)
 * fp32 accumulation. m <= 16 runs the decode GEMV, weights streamed once
 * (dot products for m <= 2 and fp32; from 3 rows of 16-bit activations the
 * codes feed the matrix cores). m > 16 with 16-bit activations runs the MFMA
 * tile GEMM when k is a multiple of 64 and scales / biases are 4-byte
 * aligned, else the matrix-core GEMV once per 16 rows. k == 0 writes zeros;
 * m == 0 or n == 0 is a no-op.
 */
qp_status qmatmul(const void* x, qp_dtype x_dtype, int64_t m, int64_t k,
                  const uint32_t* wq, const void* scales, const void* biases,
                  qp_dtype sb_dtype, int64_t n, int32_t bits, int32_t group_size,
                  void* y, hipStream_t stream);

/*
 * Workspace (bytes) the MoE calls need for n_pairs = n_tokens * top_k pairs
 * over num_experts experts (routing tables, written by the device).
 */
size_t qgemv_moe_workspace_bytes(int64_t n_pairs, int64_t num_experts);

/*
 * MoE over stacked experts (ferrum-kernels stacked_expert.rs,
 * `gemv_moe_id` / `gemv_moe_id_batched`):
 *   for p in [0, n_tokens*top_k):  t = p / top_k, j = p % top_k,
 *     out[p, :] = a_row(p) @ dequant(W[ids[p]])^T,
 *     a_row(p) = a + t*a_outer_stride + j*a_inner_stride   (elements)
 *   a        device, a_dtype, rows of n_cols elements at the strides above
 *   ids      device, int32 [n_tokens*top_k], each in [0, num_experts)
 *   wq       device, u32 [num_experts, n_rows, n_cols*bits/32] (expert-major)
 *   scales, biases  device, sb_dtype [num_experts, n_rows, n_cols/group_size]
 *   out      device, a_dtype [n_tokens*top_k, n_rows] (output)
 *   workspace device, >= qgemv_moe_workspace_bytes(n_tokens*top_k, num_experts)
 * The single-token form of the page is n_tokens = 1, top_k = n_selected,
 * a_outer_stride = 0, a_inner_stride = src1_stride; its offset form is
 * pointer arithmetic on `a` and `ids`. Pairs are sorted by expert on the
 * device and grouped into tiles of one expert, so each expert's weights are
 * streamed once per tile (with at most one pair per expert on average every
 * pair is its own tile and the sort is skipped). A pair whose id is out of
 * range is skipped (its output row is left unwritten). When the pairs are
 * sorted, the workspace afterwards begins with two device-written int32: the
 * number of tiles and the number of pairs skipped for an out-of-range id
 * (read them once the stream has synchronised). The order of one expert's
 * pairs in the sort is not specified (they are scattered with atomics);
 * every pair's output row is computed on its own, so it changes no value.
 */
qp_status qgemv_moe_id(const void* a, qp_dtype a_dtype, const int32_t* ids,
                       int64_t n_tokens, int64_t top_k, int64_t a_outer_stride,
                       int64_t a_inner_stride, const uint32_t* wq, const void* scales,
                       const void* biases, qp_dtype sb_dtype, int64_t num_experts,
                       int64_t n_rows, int64_t n_cols, int32_t bits, int32_t group_size,
                       void* out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * Fused gate/up MoE product (ferrum-kernels stacked_expert.rs,
 * `gemv_moe_id_gate_up_silu` and its batched form): one launch computes,
 * for every pair p and row r,
 *   silu_out[p, r] = SiLU(g) * u,  g = a_row(p) . gate_W[ids[p], r, :],
 *                                  u = a_row(p) . up_W[ids[p], r, :],
 *   SiLU(z) = z / (1 + exp(-z)),
 * with both stacks of identical shape, bits and group size. Arguments as in
 * qgemv_moe_id; silu_out is a_dtype [n_tokens*top_k, n_rows].
 */
qp_status qgemv_moe_id_gate_up_silu(const void* a, qp_dtype a_dtype, const int32_t* ids,
                                    int64_t n_tokens, int64_t top_k,
                                    int64_t a_outer_stride, int64_t a_inner_stride,
                                    const uint32_t* gate_wq, const void* gate_scales,
                                    const void* gate_biases, const uint32_t* up_wq,
                                    const void* up_scales, const void* up_biases,
                                    qp_dtype sb_dtype, int64_t num_experts, int64_t n_rows,
                                    int64_t n_cols, int32_t bits, int32_t group_size,
                                    void* silu_out, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * Scratch bytes of qgemv_moe_id_noalloc on each GPU: room for the routing
 * tables of up to about 60,000 pairs over 4096 experts (qgemv_moe_workspace_bytes
 * of the call must not exceed it).
 */
#define QP_NOALLOC_SCRATCH_BYTES (2u << 20)

/*
 * qgemv_moe_id without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation, harnesses without an allocator). The routing tables go
 * to a library-owned device array of QP_NOALLOC_SCRATCH_BYTES bytes per GPU,
 * present from load to process end; the call itself allocates nothing (no
 * hipMalloc, hipFree or allocating library routine). Arguments, result and
 * errors as qgemv_moe_id; QP_ERR_WORKSPACE when
 * qgemv_moe_workspace_bytes(n_tokens*top_k, num_experts) exceeds
 * QP_NOALLOC_SCRATCH_BYTES. Every call on one GPU shares that GPU's array
 * and overwrites it (nothing in it needs clearing: each call's routing
 * writes every table entry it reads), so calls that overlap in time on one
 * GPU (on different streams) race; calls ordered on one stream do not.
 */
qp_status qgemv_moe_id_noalloc(const void* a, qp_dtype a_dtype, const int32_t* ids,
                               int64_t n_tokens, int64_t top_k, int64_t a_outer_stride,
                               int64_t a_inner_stride, const uint32_t* wq, const void* scales,
                               const void* biases, qp_dtype sb_dtype, int64_t num_experts,
                               int64_t n_rows, int64_t n_cols, int32_t bits, int32_t group_size,
                               void* out, hipStream_t stream);

/* Description of the calling thread's last error ("" if none). */
const char* qpack_last_error(void);

/* Library version string. */
const char* qpack_version(void);

/*
 * Quantized linear with transpose = false (emily `quantized_matmul/2`: the
 * packed weight read as already transposed, the AWQ convention):
 *   y[m, j] = sum_i x[m, i] * (q[i, j] * s'[i, j/gs] + b'[i, j/gs])
 *   x       device, x_dtype [m, k]
 *   wq      device, u32 [k, n*bits/32]   (W stored [k, n], packed along n)
 *   scales, biases  device, sb_dtype [k, n/group_size] (sb_dtype == x_dtype)
 *   y       device, x_dtype [m, n] (output)
 *   workspace device, >= qmatmul_t_workspace_bytes(m, k, n, bits), 4-byte
 *           aligned: fp32 partial sums of the k splits.
 * n must be a multiple of group_size and n*bits of 32. A lane owns a slice of
 * output columns and walks down the rows; blocks split k, and a second
 * kernel adds the splits in order (deterministic), rounding to x_dtype. Up to
 * 4 activation rows (2 at 3 and 6 bits) per pass over the weights. k == 0
 * writes zeros; m == 0 or n == 0 is a no-op.
 */
size_t qmatmul_t_workspace_bytes(int64_t m, int64_t k, int64_t n, int32_t bits);
qp_status qmatmul_t(const void* x, qp_dtype x_dtype, int64_t m, int64_t k, const uint32_t* wq,
                    const void* scales, const void* biases, qp_dtype sb_dtype, int64_t n,
                    int32_t bits, int32_t group_size, void* y, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * Per-tensor dynamic-range int8 (mlex src/quant.rs, `quantize_dynamic_int8`
 * and `dequantize_dynamic_int8`): one output range [lo, hi] for the whole
 * weight, held on the device as range[0] = lo, range[1] = hi (fp32), and
 *   w = (q + 128) * ((hi - lo) / 255) + lo     (fp32: add, multiply, add)
 * for the signed code q. The input range the page also records is not needed
 * for weight-only products and is not kept.
 *
 * qpack_quantize_int8_tensor: w device fp32 [count] -> q device int8 [count]
 * and range; lo / hi are the tensor's min / max, the step (hi - lo) / 255 is
 * floored at FLT_EPSILON, q = clamp(round_half_away((w - lo) / step) - 128,
 * -128, 127). Finite inputs; deterministic on any launch.
 */
qp_status qpack_quantize_int8_tensor(const float* w, int64_t count, int8_t* q, float* range,
                                     hipStream_t stream);

/* qpack_dequantize_int8_tensor: q device int8 [count], range device fp32 [2]
 * -> out device out_dtype [count] (w rounded to nearest even). */
qp_status qpack_dequantize_int8_tensor(const int8_t* q, int64_t count, const float* range,
                                       qp_dtype out_dtype, void* out, hipStream_t stream);

/*
 * y[m, n] = sum_k x[m, k] * w[n, k] for a per-tensor int8 weight q [n, k]
 * (row-major) and its device range. x: x_dtype [m, k]; y: x_dtype [m, n];
 * fp32 accumulation (computed as step * sum x (q + 128) + lo * sum x). 16-bit
 * x with k a multiple of 32 up to 16384 (16-byte aligned) runs the stream
 * kernel, one or two activation rows per pass; everything else the generic
 * kernel. k == 0 writes zeros; m == 0 or n == 0 is a no-op.
 */
qp_status qmatmul_int8_tensor(const void* x, qp_dtype x_dtype, int64_t m, int64_t k,
                              const int8_t* q, const float* range, int64_t n, void* y,
                              hipStream_t stream);

/*
 * Workspace (bytes) of qgemv_moe_ffn: the routing tables of n_tokens*top_k
 * pairs, then the intermediates h [P, d_ff] and o [P, d_model] in `dtype`.
 * 0 for invalid sizes.
 */
size_t qgemv_moe_ffn_workspace_bytes(int64_t n_tokens, int64_t top_k, int64_t num_experts,
                                     int64_t d_model, int64_t d_ff, qp_dtype dtype);

/*
 * One MoE feed-forward block over stacked experts, on the device with no
 * host round trip (ferrum-kernels stacked_expert.rs: the fused gate/up call
 * `gemv_moe_id_gate_up_silu`, then the down call `gemv_moe_id_batched` on its
 * output; the weighted sum over a token's slots, which the pages leave to
 * the caller, closes it):
 *   h[p] = SiLU(a_t Wg[e]^T) * (a_t Wu[e]^T),  o[p] = h[p] Wd[e]^T,
 *   out[t] = sum_j route_weights[t*top_k + j] * o[t*top_k + j],
 *   p = t*top_k + j, e = ids[p]; h and o are stored in a_dtype.
 *   a              device, a_dtype [n_tokens, d_model] (contiguous)
 *   ids            device, int32 [n_tokens*top_k]
 *   route_weights  device, fp32 [n_tokens*top_k]
 *   gate_*, up_*   device, expert stacks [E, d_ff, d_model*bits/32], s/b [E, d_ff, d_model/gs]
 *   down_*         device, expert stack [E, d_model, d_ff*bits/32], s/b [E, d_model, d_ff/gs]
 *   out            device, a_dtype [n_tokens, d_model] (output)
 *   workspace      device, >= qgemv_moe_ffn_workspace_bytes(...), 16-byte aligned
 * The slot sum is taken in fp32 in slot order; a slot whose id is outside
 * [0, E) adds nothing. Errors as for the MoE calls above. n_tokens == 0 or
 * d_model == 0 is a no-op; top_k == 0 or d_ff == 0 writes zeros.
 */
qp_status qgemv_moe_ffn(const void* a, qp_dtype a_dtype, const int32_t* ids,
                        const float* route_weights, int64_t n_tokens, int64_t top_k,
                        const uint32_t* gate_wq, const void* gate_scales, const void* gate_biases,
                        const uint32_t* up_wq, const void* up_scales, const void* up_biases,
                        const uint32_t* down_wq, const void* down_scales, const void* down_biases,
                        qp_dtype sb_dtype, int64_t num_experts, int64_t d_model, int64_t d_ff,
                        int32_t bits, int32_t group_size, void* out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* QPACK_H */
