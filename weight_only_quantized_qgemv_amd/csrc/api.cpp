// api.cpp — the C ABI of libqpack.so (declared in include/qpack.h): argument
// validation on the host, then kernel selection and launch on the caller's
// stream. Every check runs before any HIP call, so the error paths work on a
// machine without a GPU.
//
// Rules enforced, by source:
//  - bits in {2, 3, 4, 6, 8}: emily lib/emily/quantization.ex,
//    `defn_supported_bits/0` and `validate_defn_bits!`;
//  - K * bits % 32 == 0 and K % group_size == 0: same page,
//    `build_word_indices` (the packing invariant) and `group_last_axis`;
//  - activation dtype == scales dtype in affine mode: same page,
//    `validate_dtype_match!`;
//  - gate and up stacks of one shape: ferrum-kernels src/stacked_expert.rs,
//    `gemv_moe_id_gate_up_silu` docs ("must match shape").
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "../../include/qpack.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

qp_status fail(qp_status s, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

qp_status ok()
{
    g_last_error.clear();
    return QP_OK;
}

qp_status hip_result(hipError_t e, const char* what)
{
    if (e != hipSuccess)
        return fail(QP_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
    return ok();
}

bool bits_ok(int32_t b) { return b == 2 || b == 3 || b == 4 || b == 6 || b == 8; }
bool gs_ok(int32_t g) { return g == 32 || g == 64 || g == 128; }
bool dtype_ok(int d) { return d == QP_F32 || d == QP_F16 || d == QP_BF16; }
size_t esize(int d) { return d == QP_F32 ? 4 : 2; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a * b without int64 overflow (both non-negative).
bool mul_ok(int64_t a, int64_t b) { return a == 0 || b <= INT64_MAX / a; }

// Checks shared by every call: bits, group size, K divisibility.
qp_status check_layout(int64_t k, int32_t bits, int32_t gs)
{
    if (!bits_ok(bits))
        return fail(QP_ERR_UNSUPPORTED, "bits=%d not supported (2, 3, 4, 6, 8)", bits);
    if (!gs_ok(gs))
        return fail(QP_ERR_UNSUPPORTED, "group_size=%d not supported (32, 64, 128)", gs);
    if (k % gs != 0)
        return fail(QP_ERR_SHAPE, "K=%lld is not a multiple of group_size=%d", (long long)k, gs);
    if ((k * bits) % 32 != 0)
        return fail(QP_ERR_SHAPE, "K*bits=%lld is not a multiple of 32", (long long)(k * bits));
    return QP_OK;
}

} // namespace

extern "C" {

const char* qpack_last_error(void) { return g_last_error.c_str(); }

const char* qpack_version(void) { return "qpack 0.1.0 (gfx950)"; }

qp_status qpack_quantize(const float* w, int64_t n, int64_t k, int32_t bits, int32_t group_size,
                         qp_dtype sb_dtype, uint32_t* wq, void* scales, void* biases,
                         hipStream_t stream)
{
    if (n < 0 || k < 0)
        return fail(QP_ERR_INVALID_ARG, "negative size (n=%lld, k=%lld)", (long long)n,
                    (long long)k);
    if (!dtype_ok(sb_dtype))
        return fail(QP_ERR_INVALID_ARG, "unknown scales dtype %d", (int)sb_dtype);
    if (qp_status s = check_layout(k, bits, group_size); s != QP_OK)
        return s;
    if (!mul_ok(n, k))
        return fail(QP_ERR_INVALID_ARG, "n*k overflows");
    if (n == 0 || k == 0)
        return ok();
    if (!w || !wq || !scales || !biases)
        return fail(QP_ERR_INVALID_ARG, "null pointer");
    if (!aligned(w, 4) || !aligned(wq, 4) || !aligned(scales, esize(sb_dtype)) ||
        !aligned(biases, esize(sb_dtype)))
        return fail(QP_ERR_ALIGN, "pointer not aligned to its element size");
    qp::QuantizeArgs a{w, n, k, bits, group_size, (int)sb_dtype, wq, scales, biases};
    return hip_result(qp::launch_quantize(a, stream), "qpack_quantize");
}

qp_status qpack_dequantize(const uint32_t* wq, const void* scales, const void* biases,
                           qp_dtype sb_dtype, int64_t n, int64_t k, int32_t bits,
                           int32_t group_size, qp_dtype out_dtype, void* out, hipStream_t stream)
{
    if (n < 0 || k < 0)
        return fail(QP_ERR_INVALID_ARG, "negative size (n=%lld, k=%lld)", (long long)n,
                    (long long)k);
    if (!dtype_ok(sb_dtype) || !dtype_ok(out_dtype))
        return fail(QP_ERR_INVALID_ARG, "unknown dtype (scales=%d, out=%d)", (int)sb_dtype,
                    (int)out_dtype);
    if (qp_status s = check_layout(k, bits, group_size); s != QP_OK)
        return s;
    if (k > (int64_t(1) << 33))
        return fail(QP_ERR_UNSUPPORTED, "k=%lld above 2^33", (long long)k);
    if (out_dtype != QP_F32 && out_dtype != sb_dtype)
        return fail(QP_ERR_DTYPE_MISMATCH,
                    "output dtype %d must be fp32 or the scales dtype %d", (int)out_dtype,
                    (int)sb_dtype);
    if (!mul_ok(n, k))
        return fail(QP_ERR_INVALID_ARG, "n*k overflows");
    if (n == 0 || k == 0)
        return ok();
    if (!wq || !scales || !biases || !out)
        return fail(QP_ERR_INVALID_ARG, "null pointer");
    if (!aligned(wq, 4) || !aligned(scales, esize(sb_dtype)) || !aligned(biases, esize(sb_dtype)) ||
        !aligned(out, esize(out_dtype)))
        return fail(QP_ERR_ALIGN, "pointer not aligned to its element size");
    qp::DequantArgs a{wq, scales, biases, (int)sb_dtype, (int)out_dtype, n, k, bits, group_size,
                      out};
    return hip_result(qp::launch_dequantize(a, stream), "qpack_dequantize");
}

static qp_status mx_layout(int mode, int64_t k, int* bits, int* gs)
{
    switch (mode) {
    case QP_MXFP4: *bits = 4; *gs = 32; break;
    case QP_MXFP8: *bits = 8; *gs = 32; break;
    case QP_NVFP4: *bits = 4; *gs = 16; break;
    default: return fail(QP_ERR_UNSUPPORTED, "mode=%d not supported (1 mxfp4, 2 mxfp8, 3 nvfp4)",
                         mode);
    }
    if (k % *gs != 0)
        return fail(QP_ERR_SHAPE, "K=%lld is not a multiple of the mode's group size %d",
                    (long long)k, *gs);
    return QP_OK;
}

qp_status qpack_dequantize_mx(const uint32_t* wq, const uint8_t* scales, qp_mode mode, int64_t n,
                              int64_t k, qp_dtype out_dtype, void* out, hipStream_t stream)
{
    if (n < 0 || k < 0)
        return fail(QP_ERR_INVALID_ARG, "negative size (n=%lld, k=%lld)", (long long)n,
                    (long long)k);
    if (!dtype_ok(out_dtype))
        return fail(QP_ERR_INVALID_ARG, "unknown output dtype %d", (int)out_dtype);
    int bits, gs;
    if (qp_status s = mx_layout(mode, k, &bits, &gs); s != QP_OK)
        return s;
    if (k > (int64_t(1) << 33))
        return fail(QP_ERR_UNSUPPORTED, "k=%lld above 2^33", (long long)k);
    if (!mul_ok(n, k))
        return fail(QP_ERR_INVALID_ARG, "n*k overflows");
    if (n == 0 || k == 0)
        return ok();
    if (!wq || !scales || !out)
        return fail(QP_ERR_INVALID_ARG, "null pointer");
    if (!aligned(wq, 4) || !aligned(out, esize(out_dtype)))
        return fail(QP_ERR_ALIGN, "pointer not aligned to its element size");
    qp::DequantMxArgs a{wq, scales, (int)mode, (int)out_dtype, n, k, out};
    return hip_result(qp::launch_dequantize_mx(a, stream), "qpack_dequantize_mx");
}

qp_status qmatmul_mx(const void* x, qp_dtype x_dtype, int64_t m, int64_t k, const uint32_t* wq,
                     const uint8_t* scales, qp_mode mode, int64_t n, void* y, hipStream_t stream)
{
    if (m < 0 || k < 0 || n < 0)
        return fail(QP_ERR_INVALID_ARG, "negative size (m=%lld, k=%lld, n=%lld)", (long long)m,
                    (long long)k, (long long)n);
    if (!dtype_ok(x_dtype))
        return fail(QP_ERR_INVALID_ARG, "unknown dtype %d", (int)x_dtype);
    int bits, gs;
    if (qp_status s = mx_layout(mode, k, &bits, &gs); s != QP_OK)
        return s;
    if (!mul_ok(m, k) || !mul_ok(n, k) || !mul_ok(m, n) || k >= (int64_t(1) << 31) ||
        n >= (int64_t(1) << 31) || m >= (int64_t(1) << 31))
        return fail(QP_ERR_INVALID_ARG, "size too large");
    if (m == 0 || n == 0)
        return ok();
    if (!y)
        return fail(QP_ERR_INVALID_ARG, "null output pointer");
    const size_t es = esize(x_dtype);
    if (!aligned(y, es))
        return fail(QP_ERR_ALIGN, "y not aligned to its element size");
    if (k == 0)
        return hip_result(qp::launch_fill_zero(y, (int)x_dtype, m * n, stream), "qmatmul_mx");
    if (!x || !wq || !scales)
        return fail(QP_ERR_INVALID_ARG, "null pointer");
    if (!aligned(x, es) || !aligned(wq, 4))
        return fail(QP_ERR_ALIGN, "pointer not aligned to its element size");
    qp::GemvMxArgs a{x, (int)x_dtype, (int)mode, m, k, n, wq, scales, y};
    if (m > 16 && qp::qgemm_mx_fits(a))
        return hip_result(qp::launch_qgemm_mx(a, stream), "qmatmul_mx");
    return hip_result(qp::launch_qmatmul_mx(a, stream), "qmatmul_mx");
}

qp_status qmatmul(const void* x, qp_dtype x_dtype, int64_t m, int64_t k, const uint32_t* wq,
                  const void* scales, const void* biases, qp_dtype sb_dtype, int64_t n,
                  int32_t bits, int32_t group_size, void* y, hipStream_t stream)
{
    if (m < 0 || k < 0 || n < 0)
        return fail(QP_ERR_INVALID_ARG, "negative size (m=%lld, k=%lld, n=%lld)", (long long)m,
                    (long long)k, (long long)n);
    if (!dtype_ok(x_dtype) || !dtype_ok(sb_dtype))
        return fail(QP_ERR_INVALID_ARG, "unknown dtype (x=%d, scales=%d)", (int)x_dtype,
                    (int)sb_dtype);
    if (qp_status s = check_layout(k, bits, group_size); s != QP_OK)
        return s;
    if (x_dtype != sb_dtype)
        return fail(QP_ERR_DTYPE_MISMATCH,
                    "input dtype %d must match scales dtype %d (affine mode)", (int)x_dtype,
                    (int)sb_dtype);
    if (!mul_ok(m, k) || !mul_ok(n, k) || !mul_ok(m, n))
        return fail(QP_ERR_INVALID_ARG, "size product overflows");
    if (m == 0 || n == 0)
        return ok();
    if (!y)
        return fail(QP_ERR_INVALID_ARG, "null output pointer");
    const size_t es = esize(x_dtype);
    if (!aligned(y, es))
        return fail(QP_ERR_ALIGN, "y not aligned to its element size");
    if (k == 0)
        return hip_result(qp::launch_fill_zero(y, (int)x_dtype, m * n, stream), "qmatmul");
    if (!x || !wq || !scales || !biases)
        return fail(QP_ERR_INVALID_ARG, "null pointer");
    if (!aligned(x, es) || !aligned(wq, 4) || !aligned(scales, es) || !aligned(biases, es))
        return fail(QP_ERR_ALIGN, "pointer not aligned to its element size");
    qp::GemvArgs a{x, (int)x_dtype, m, k, n, wq, scales, biases, bits, group_size, y};
    if (m <= 16 || x_dtype == QP_F32)
        return hip_result(qp::launch_qgemv(a, stream), "qmatmul");
    return hip_result(qp::launch_qgemm(a, stream), "qmatmul");
}

size_t qgemv_moe_workspace_bytes(int64_t n_pairs, int64_t num_experts)
{
    if (n_pairs < 0 || num_experts < 0)
        return 0;
    return qp::moe_workspace_bytes(n_pairs, num_experts);
}

// check_ws: the caller brings the workspace (pointer, size and alignment are
// checked); false for the allocation-free call, whose scratch is the
// library's own.
static qp_status moe_common(const qp::MoeArgs& a, const char* what, bool check_ws = true)
{
    if (a.n_tokens < 0 || a.top_k < 0 || a.E < 0 || a.n_rows < 0 || a.n_cols < 0 ||
        a.a_outer < 0 || a.a_inner < 0)
        return fail(QP_ERR_INVALID_ARG, "%s: negative size or stride", what);
    if (!dtype_ok(a.dt))
        return fail(QP_ERR_INVALID_ARG, "%s: unknown dtype", what);
    if (qp_status s = check_layout(a.n_cols, a.bits, a.gs); s != QP_OK)
        return s;
    if (a.E > 4096)
        return fail(QP_ERR_UNSUPPORTED, "%s: num_experts=%lld above 4096", what, (long long)a.E);
    if (!mul_ok(a.n_tokens, a.top_k) || a.n_tokens * a.top_k > (int64_t)INT32_MAX / 2)
        return fail(QP_ERR_INVALID_ARG, "%s: too many pairs", what);
    const int64_t P = a.n_tokens * a.top_k;
    if (!mul_ok(a.E, a.n_rows) || !mul_ok(a.E * a.n_rows, a.n_cols) || !mul_ok(P, a.n_rows))
        return fail(QP_ERR_INVALID_ARG, "%s: size product overflows", what);
    if (P == 0 || a.n_rows == 0)
        return QP_OK;
    if (a.E == 0)
        return fail(QP_ERR_INVALID_ARG, "%s: no experts for %lld pairs", what, (long long)P);
    if (!a.ids || !a.out || (check_ws && !a.workspace))
        return fail(QP_ERR_INVALID_ARG, "%s: null pointer", what);
    if (a.ws_bytes < qp::moe_workspace_bytes(P, a.E))
        return fail(QP_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", what, a.ws_bytes,
                    qp::moe_workspace_bytes(P, a.E));
    const size_t es = esize(a.dt);
    if (!aligned(a.out, es) || !aligned(a.ids, 4) || (check_ws && !aligned(a.workspace, 16)))
        return fail(QP_ERR_ALIGN, "%s: pointer not aligned", what);
    if (a.n_cols > 0) {
        if (!a.a)
            return fail(QP_ERR_INVALID_ARG, "%s: null activation pointer", what);
        if (!aligned(a.a, es))
            return fail(QP_ERR_ALIGN, "%s: activations not aligned", what);
        for (int t = 0; t < (a.fused_silu ? 2 : 1); ++t) {
            if (!a.wq[t] || !a.scales[t] || !a.biases[t])
                return fail(QP_ERR_INVALID_ARG, "%s: null weight pointer", what);
            if (!aligned(a.wq[t], 4) || !aligned(a.scales[t], es) || !aligned(a.biases[t], es))
                return fail(QP_ERR_ALIGN, "%s: weight pointer not aligned", what);
        }
    }
    return QP_OK;
}

} // extern "C"

static qp_status scratch_address(void** out, const char* what);

// qgemv_moe_id with the caller's workspace, or (scratch) with the library's
// own scratch array in its place.
static qp_status moe_id_run(const void* a, qp_dtype a_dtype, const int32_t* ids, int64_t n_tokens,
                            int64_t top_k, int64_t a_outer_stride, int64_t a_inner_stride,
                            const uint32_t* wq, const void* scales, const void* biases,
                            qp_dtype sb_dtype, int64_t num_experts, int64_t n_rows,
                            int64_t n_cols, int32_t bits, int32_t group_size, void* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream,
                            bool scratch, const char* what)
{
    if (dtype_ok(a_dtype) && dtype_ok(sb_dtype) && a_dtype != sb_dtype)
        return fail(QP_ERR_DTYPE_MISMATCH, "%s: input dtype must match scales dtype", what);
    qp::MoeArgs m{};
    m.a = a; m.dt = (int)a_dtype; m.ids = ids;
    m.n_tokens = n_tokens; m.top_k = top_k; m.a_outer = a_outer_stride; m.a_inner = a_inner_stride;
    m.wq[0] = m.wq[1] = wq; m.scales[0] = m.scales[1] = scales; m.biases[0] = m.biases[1] = biases;
    m.E = num_experts; m.n_rows = n_rows; m.n_cols = n_cols; m.bits = bits; m.gs = group_size;
    m.fused_silu = false; m.out = out; m.workspace = workspace; m.ws_bytes = workspace_bytes;
    if (qp_status s = moe_common(m, what, !scratch); s != QP_OK)
        return s;
    const int64_t P = n_tokens * top_k;
    if (P == 0 || n_rows == 0)
        return ok();
    if (n_cols == 0)
        return hip_result(qp::launch_fill_zero(out, (int)a_dtype, P * n_rows, stream), what);
    if (scratch) {
        if (qp_status s = scratch_address(&m.workspace, what); s != QP_OK)
            return s;
    }
    return hip_result(qp::launch_moe(m, stream), what);
}

extern "C" {

qp_status qgemv_moe_id(const void* a, qp_dtype a_dtype, const int32_t* ids, int64_t n_tokens,
                       int64_t top_k, int64_t a_outer_stride, int64_t a_inner_stride,
                       const uint32_t* wq, const void* scales, const void* biases,
                       qp_dtype sb_dtype, int64_t num_experts, int64_t n_rows, int64_t n_cols,
                       int32_t bits, int32_t group_size, void* out, void* workspace,
                       size_t workspace_bytes, hipStream_t stream)
{
    return moe_id_run(a, a_dtype, ids, n_tokens, top_k, a_outer_stride, a_inner_stride, wq,
                      scales, biases, sb_dtype, num_experts, n_rows, n_cols, bits, group_size, out,
                      workspace, workspace_bytes, stream, false, "qgemv_moe_id");
}

} // extern "C"

// Routing tables of qgemv_moe_id_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends. Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol); it
// resolves the array's device address once per device with the device
// current and passes that address as the workspace.
static __device__ __align__(256) unsigned char scratch[QP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

} // namespace

static qp_status scratch_address(void** out, const char* what)
{
    int dev = -1;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
        return hip_result(e, what);
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(QP_ERR_UNSUPPORTED, "%s: device %d above the %d the scratch table covers", what,
                    dev, kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess)
            return hip_result(e, what);
        if (p == nullptr)
            return fail(QP_ERR_HIP, "%s: no device address for the scratch array", what);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QP_OK;
}

extern "C" {

qp_status qgemv_moe_id_noalloc(const void* a, qp_dtype a_dtype, const int32_t* ids,
                               int64_t n_tokens, int64_t top_k, int64_t a_outer_stride,
                               int64_t a_inner_stride, const uint32_t* wq, const void* scales,
                               const void* biases, qp_dtype sb_dtype, int64_t num_experts,
                               int64_t n_rows, int64_t n_cols, int32_t bits, int32_t group_size,
                               void* out, hipStream_t stream)
{
    const char* what = "qgemv_moe_id_noalloc";
    if (n_tokens >= 0 && top_k >= 0 && num_experts >= 0 && num_experts <= 4096 &&
        mul_ok(n_tokens, top_k) && n_tokens * top_k <= (int64_t)INT32_MAX / 2) {
        const size_t need = qp::moe_workspace_bytes(n_tokens * top_k, num_experts);
        if (need > QP_NOALLOC_SCRATCH_BYTES)
            return fail(QP_ERR_WORKSPACE,
                        "%s: %lld pairs over %lld experts need %zu bytes of scratch, above the "
                        "%u-byte maximum", what, (long long)(n_tokens * top_k),
                        (long long)num_experts, need, (unsigned)QP_NOALLOC_SCRATCH_BYTES);
    }
    return moe_id_run(a, a_dtype, ids, n_tokens, top_k, a_outer_stride, a_inner_stride, wq,
                      scales, biases, sb_dtype, num_experts, n_rows, n_cols, bits, group_size, out,
                      nullptr, QP_NOALLOC_SCRATCH_BYTES, stream, true, what);
}

qp_status qgemv_moe_id_gate_up_silu(const void* a, qp_dtype a_dtype, const int32_t* ids,
                                    int64_t n_tokens, int64_t top_k, int64_t a_outer_stride,
                                    int64_t a_inner_stride, const uint32_t* gate_wq,
                                    const void* gate_scales, const void* gate_biases,
                                    const uint32_t* up_wq, const void* up_scales,
                                    const void* up_biases, qp_dtype sb_dtype,
                                    int64_t num_experts, int64_t n_rows, int64_t n_cols,
                                    int32_t bits, int32_t group_size, void* silu_out,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (dtype_ok(a_dtype) && dtype_ok(sb_dtype) && a_dtype != sb_dtype)
        return fail(QP_ERR_DTYPE_MISMATCH,
                    "qgemv_moe_id_gate_up_silu: input dtype must match scales dtype");
    qp::MoeArgs m{};
    m.a = a; m.dt = (int)a_dtype; m.ids = ids;
    m.n_tokens = n_tokens; m.top_k = top_k; m.a_outer = a_outer_stride; m.a_inner = a_inner_stride;
    m.wq[0] = gate_wq; m.scales[0] = gate_scales; m.biases[0] = gate_biases;
    m.wq[1] = up_wq; m.scales[1] = up_scales; m.biases[1] = up_biases;
    m.E = num_experts; m.n_rows = n_rows; m.n_cols = n_cols; m.bits = bits; m.gs = group_size;
    m.fused_silu = true; m.out = silu_out; m.workspace = workspace; m.ws_bytes = workspace_bytes;
    if (qp_status s = moe_common(m, "qgemv_moe_id_gate_up_silu"); s != QP_OK)
        return s;
    const int64_t P = n_tokens * top_k;
    if (P == 0 || n_rows == 0)
        return ok();
    if (n_cols == 0) // g = u = 0, SiLU(0) * 0 = 0
        return hip_result(qp::launch_fill_zero(silu_out, (int)a_dtype, P * n_rows, stream),
                          "qgemv_moe_id_gate_up_silu");
    return hip_result(qp::launch_moe(m, stream), "qgemv_moe_id_gate_up_silu");
}

qp_status qpack_quantize_int8_tensor(const float* w, int64_t count, int8_t* q, float* range,
                                     hipStream_t stream)
{
    if (count < 0)
        return fail(QP_ERR_INVALID_ARG, "negative size %lld", (long long)count);
    if (count == 0)
        return ok();
    if (!w || !q || !range)
        return fail(QP_ERR_INVALID_ARG, "null pointer");
    if (!aligned(w, 4) || !aligned(range, 4))
        return fail(QP_ERR_ALIGN, "pointer not aligned to its element size");
    return hip_result(qp::launch_quantize_int8_tensor(w, count, q, range, stream),
                      "qpack_quantize_int8_tensor");
}

qp_status qpack_dequantize_int8_tensor(const int8_t* q, int64_t count, const float* range,
                                       qp_dtype out_dtype, void* out, hipStream_t stream)
{
    if (count < 0)
        return fail(QP_ERR_INVALID_ARG, "negative size %lld", (long long)count);
    if (!dtype_ok(out_dtype))
        return fail(QP_ERR_INVALID_ARG, "unknown output dtype %d", (int)out_dtype);
    if (count == 0)
        return ok();
    if (!q || !range || !out)
        return fail(QP_ERR_INVALID_ARG, "null pointer");
    if (!aligned(range, 4) || !aligned(out, esize(out_dtype)))
        return fail(QP_ERR_ALIGN, "pointer not aligned to its element size");
    return hip_result(qp::launch_dequantize_int8_tensor(q, count, range, (int)out_dtype, out,
                                                        stream),
                      "qpack_dequantize_int8_tensor");
}

qp_status qmatmul_int8_tensor(const void* x, qp_dtype x_dtype, int64_t m, int64_t k,
                              const int8_t* q, const float* range, int64_t n, void* y,
                              hipStream_t stream)
{
    if (m < 0 || k < 0 || n < 0)
        return fail(QP_ERR_INVALID_ARG, "negative size (m=%lld, k=%lld, n=%lld)", (long long)m,
                    (long long)k, (long long)n);
    if (!dtype_ok(x_dtype))
        return fail(QP_ERR_INVALID_ARG, "unknown dtype %d", (int)x_dtype);
    if (!mul_ok(m, k) || !mul_ok(n, k) || !mul_ok(m, n) || k >= (int64_t(1) << 31) ||
        n >= (int64_t(1) << 31) || m >= (int64_t(1) << 31))
        return fail(QP_ERR_INVALID_ARG, "size too large");
    if (m == 0 || n == 0)
        return ok();
    if (!y)
        return fail(QP_ERR_INVALID_ARG, "null output pointer");
    const size_t es = esize(x_dtype);
    if (!aligned(y, es))
        return fail(QP_ERR_ALIGN, "y not aligned to its element size");
    if (k == 0)
        return hip_result(qp::launch_fill_zero(y, (int)x_dtype, m * n, stream),
                          "qmatmul_int8_tensor");
    if (!x || !q || !range)
        return fail(QP_ERR_INVALID_ARG, "null pointer");
    if (!aligned(x, es) || !aligned(range, 4))
        return fail(QP_ERR_ALIGN, "pointer not aligned to its element size");
    qp::Int8TensorArgs a{x, (int)x_dtype, m, k, n, q, range, y};
    return hip_result(qp::launch_qmatmul_int8_tensor(a, stream), "qmatmul_int8_tensor");
}

size_t qmatmul_t_workspace_bytes(int64_t m, int64_t k, int64_t n, int32_t bits)
{
    if (m <= 0 || k <= 0 || n <= 0 || !bits_ok(bits) || !mul_ok(m, n) || !mul_ok(k, n))
        return 0;
    return qp::qgemv_t_plan(m, k, n, bits).workspace_bytes;
}

qp_status qmatmul_t(const void* x, qp_dtype x_dtype, int64_t m, int64_t k, const uint32_t* wq,
                    const void* scales, const void* biases, qp_dtype sb_dtype, int64_t n,
                    int32_t bits, int32_t group_size, void* y, void* workspace,
                    size_t workspace_bytes, hipStream_t stream)
{
    const char* what = "qmatmul_t";
    if (m < 0 || k < 0 || n < 0)
        return fail(QP_ERR_INVALID_ARG, "%s: negative size", what);
    if (!dtype_ok(x_dtype) || !dtype_ok(sb_dtype))
        return fail(QP_ERR_INVALID_ARG, "%s: unknown dtype", what);
    if (qp_status s = check_layout(n, bits, group_size); s != QP_OK)   // groups run along n
        return s;
    if (x_dtype != sb_dtype)
        return fail(QP_ERR_DTYPE_MISMATCH, "%s: input dtype must match scales dtype", what);
    if (!mul_ok(m, k) || !mul_ok(n, k) || !mul_ok(m, n) || k >= (int64_t(1) << 31) ||
        n >= (int64_t(1) << 31))
        return fail(QP_ERR_INVALID_ARG, "%s: size too large", what);
    if (m == 0 || n == 0)
        return ok();
    if (!y)
        return fail(QP_ERR_INVALID_ARG, "%s: null output pointer", what);
    const size_t es = esize(x_dtype);
    if (!aligned(y, es))
        return fail(QP_ERR_ALIGN, "%s: y not aligned", what);
    if (k == 0)
        return hip_result(qp::launch_fill_zero(y, (int)x_dtype, m * n, stream), what);
    if (!x || !wq || !scales || !biases || !workspace)
        return fail(QP_ERR_INVALID_ARG, "%s: null pointer", what);
    const size_t need = qmatmul_t_workspace_bytes(m, k, n, bits);
    if (workspace_bytes < need)
        return fail(QP_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", what,
                    workspace_bytes, need);
    if (!aligned(x, es) || !aligned(wq, 4) || !aligned(scales, es) || !aligned(biases, es) ||
        !aligned(workspace, 4))
        return fail(QP_ERR_ALIGN, "%s: pointer not aligned", what);
    qp::QgemvTArgs a{x, (int)x_dtype, m, k, n, wq, scales, biases, bits, group_size, y,
                     static_cast<float*>(workspace)};
    return hip_result(qp::launch_qgemv_t(a, stream), what);
}

static size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

size_t qgemv_moe_ffn_workspace_bytes(int64_t n_tokens, int64_t top_k, int64_t num_experts,
                                     int64_t d_model, int64_t d_ff, qp_dtype dtype)
{
    if (n_tokens < 0 || top_k < 0 || num_experts < 0 || d_model < 0 || d_ff < 0 ||
        !dtype_ok(dtype) || !mul_ok(n_tokens, top_k))
        return 0;
    const int64_t P = n_tokens * top_k;
    if (!mul_ok(P, d_ff) || !mul_ok(P, d_model))
        return 0;
    const size_t es = esize(dtype);
    return round256(qp::moe_workspace_bytes(P, num_experts)) + round256((size_t)(P * d_ff) * es) +
           (size_t)(P * d_model) * es;
}

qp_status qgemv_moe_ffn(const void* a, qp_dtype a_dtype, const int32_t* ids,
                        const float* route_weights, int64_t n_tokens, int64_t top_k,
                        const uint32_t* gate_wq, const void* gate_scales, const void* gate_biases,
                        const uint32_t* up_wq, const void* up_scales, const void* up_biases,
                        const uint32_t* down_wq, const void* down_scales, const void* down_biases,
                        qp_dtype sb_dtype, int64_t num_experts, int64_t d_model, int64_t d_ff,
                        int32_t bits, int32_t group_size, void* out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream)
{
    const char* what = "qgemv_moe_ffn";
    if (dtype_ok(a_dtype) && dtype_ok(sb_dtype) && a_dtype != sb_dtype)
        return fail(QP_ERR_DTYPE_MISMATCH, "%s: input dtype must match scales dtype", what);
    if (n_tokens < 0 || top_k < 0 || num_experts < 0 || d_model < 0 || d_ff < 0)
        return fail(QP_ERR_INVALID_ARG, "%s: negative size", what);
    if (!dtype_ok(a_dtype))
        return fail(QP_ERR_INVALID_ARG, "%s: unknown dtype", what);
    if (qp_status s = check_layout(d_model, bits, group_size); s != QP_OK)
        return s;
    if (qp_status s = check_layout(d_ff, bits, group_size); s != QP_OK)
        return s;
    if (!mul_ok(n_tokens, top_k) || n_tokens * top_k > (int64_t)INT32_MAX / 2 ||
        !mul_ok(n_tokens, d_model))
        return fail(QP_ERR_INVALID_ARG, "%s: too many pairs", what);
    const int64_t P = n_tokens * top_k;
    if (n_tokens == 0 || d_model == 0)
        return ok();
    if (!out)
        return fail(QP_ERR_INVALID_ARG, "%s: null output pointer", what);
    if (!aligned(out, esize(a_dtype)))
        return fail(QP_ERR_ALIGN, "%s: output not aligned", what);
    if (P == 0 || d_ff == 0) // empty slot sums, or h = 0 and so o = 0
        return hip_result(qp::launch_fill_zero(out, (int)a_dtype, n_tokens * d_model, stream), what);
    const size_t need = qgemv_moe_ffn_workspace_bytes(n_tokens, top_k, num_experts, d_model, d_ff,
                                                      a_dtype);
    if (!workspace || !route_weights)
        return fail(QP_ERR_INVALID_ARG, "%s: null pointer", what);
    if (workspace_bytes < need)
        return fail(QP_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", what,
                    workspace_bytes, need);
    if (!aligned(route_weights, 4))
        return fail(QP_ERR_ALIGN, "%s: router weights not aligned", what);
    const size_t es = esize(a_dtype);
    const size_t route_bytes = round256(qp::moe_workspace_bytes(P, num_experts));
    char* h = static_cast<char*>(workspace) + route_bytes;
    char* o = h + round256((size_t)(P * d_ff) * es);

    qp::MoeArgs gu{};
    gu.a = a; gu.dt = (int)a_dtype; gu.ids = ids;
    gu.n_tokens = n_tokens; gu.top_k = top_k; gu.a_outer = d_model; gu.a_inner = 0;
    gu.wq[0] = gate_wq; gu.scales[0] = gate_scales; gu.biases[0] = gate_biases;
    gu.wq[1] = up_wq; gu.scales[1] = up_scales; gu.biases[1] = up_biases;
    gu.E = num_experts; gu.n_rows = d_ff; gu.n_cols = d_model; gu.bits = bits; gu.gs = group_size;
    gu.fused_silu = true; gu.out = h; gu.workspace = workspace; gu.ws_bytes = route_bytes;
    qp::MoeArgs dn{};
    dn.a = h; dn.dt = (int)a_dtype; dn.ids = ids;
    dn.n_tokens = n_tokens; dn.top_k = top_k; dn.a_outer = top_k * d_ff; dn.a_inner = d_ff;
    dn.wq[0] = dn.wq[1] = down_wq; dn.scales[0] = dn.scales[1] = down_scales;
    dn.biases[0] = dn.biases[1] = down_biases;
    dn.E = num_experts; dn.n_rows = d_model; dn.n_cols = d_ff; dn.bits = bits; dn.gs = group_size;
    dn.fused_silu = false; dn.out = o; dn.workspace = workspace; dn.ws_bytes = route_bytes;
    if (qp_status s = moe_common(gu, what); s != QP_OK)
        return s;
    if (qp_status s = moe_common(dn, what); s != QP_OK)
        return s;
    if (qp::moe_down_combine_ok(dn)) {
        // Few tokens: the down projection and the slot combine in one launch,
        // straight into `out` (the same values as the two launches below).
        if (hipError_t e = qp::launch_moe(gu, stream); e != hipSuccess)
            return hip_result(e, what);
        return hip_result(qp::launch_moe_down_combine(dn, route_weights, out, stream), what);
    }
    if (hipError_t e = qp::launch_moe_pair(gu, dn, stream); e != hipSuccess)
        return hip_result(e, what);
    qp::MoeCombineArgs c{o, ids, route_weights, n_tokens, top_k, d_model, num_experts,
                         (int)a_dtype, out};
    return hip_result(qp::launch_moe_combine(c, stream), what);
}

} // extern "C"

namespace qp {

hipError_t launch_qgemv(const GemvArgs& a, hipStream_t stream)
{
    switch (a.bits) {
    case 2: return launch_qgemv_b2(a, stream);
    case 3: return launch_qgemv_b3(a, stream);
    case 4: return launch_qgemv_b4(a, stream);
    case 6: return launch_qgemv_b6(a, stream);
    case 8: return launch_qgemv_b8(a, stream);
    }
    return hipErrorInvalidValue;
}

} // namespace qp
