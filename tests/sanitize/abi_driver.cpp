// abi_driver.cpp — calls every C-ABI entry point with argument errors (each
// must return its status and launch nothing) and with valid shapes (each
// must reach a launcher), against the stub launchers of abi_stubs.cpp. Built
// with the host side under AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_sanitize_host.py; no GPU is touched.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/qpack.h"

extern "C" int g_stub_launches;

static int failures = 0;

static void expect(const char* what, qp_status got, qp_status want, int launches)
{
    if (got != want) {
        std::fprintf(stderr, "FAIL %s: status %d, want %d (%s)\n", what, (int)got, (int)want,
                     qpack_last_error());
        ++failures;
    }
    if (want != QP_OK && launches != 0) {
        std::fprintf(stderr, "FAIL %s: an argument error launched %d kernels\n", what, launches);
        ++failures;
    }
    if (want != QP_OK && std::strlen(qpack_last_error()) == 0) {
        std::fprintf(stderr, "FAIL %s: no error message\n", what);
        ++failures;
    }
}

#define RUN(what, call, want)                                                                      \
    do {                                                                                           \
        const int l0 = g_stub_launches;                                                            \
        const qp_status s = (call);                                                                \
        expect(what, s, want, g_stub_launches - l0);                                               \
    } while (0)

int main()
{
    // Stand-in device addresses: aligned and misaligned, never dereferenced.
    void* A = reinterpret_cast<void*>(0x10000);
    void* ODD = reinterpret_cast<void*>(0x10001);
    const uint32_t* WQ = static_cast<const uint32_t*>(A);
    const int32_t* IDS = static_cast<const int32_t*>(A);
    const float* FP = static_cast<const float*>(A);
    const qp_dtype BF = QP_BF16, F16 = QP_F16, F32 = QP_F32;

    // qmatmul
    RUN("qmatmul ok", qmatmul(A, BF, 2, 128, WQ, A, A, BF, 8, 4, 64, A, nullptr), QP_OK);
    RUN("qmatmul bits 5", qmatmul(A, BF, 2, 128, WQ, A, A, BF, 8, 5, 64, A, nullptr), QP_ERR_UNSUPPORTED);
    RUN("qmatmul gs 16", qmatmul(A, BF, 2, 128, WQ, A, A, BF, 8, 4, 16, A, nullptr), QP_ERR_UNSUPPORTED);
    RUN("qmatmul k%gs", qmatmul(A, BF, 2, 96, WQ, A, A, BF, 8, 4, 64, A, nullptr), QP_ERR_SHAPE);
    RUN("qmatmul dtype", qmatmul(A, F16, 2, 128, WQ, A, A, BF, 8, 4, 64, A, nullptr), QP_ERR_DTYPE_MISMATCH);
    RUN("qmatmul m<0", qmatmul(A, BF, -1, 128, WQ, A, A, BF, 8, 4, 64, A, nullptr), QP_ERR_INVALID_ARG);
    RUN("qmatmul null x", qmatmul(nullptr, BF, 2, 128, WQ, A, A, BF, 8, 4, 64, A, nullptr), QP_ERR_INVALID_ARG);
    RUN("qmatmul null y", qmatmul(A, BF, 2, 128, WQ, A, A, BF, 8, 4, 64, nullptr, nullptr), QP_ERR_INVALID_ARG);
    RUN("qmatmul odd y", qmatmul(A, BF, 2, 128, WQ, A, A, BF, 8, 4, 64, ODD, nullptr), QP_ERR_ALIGN);
    RUN("qmatmul odd wq", qmatmul(A, BF, 2, 128, static_cast<const uint32_t*>(ODD), A, A, BF, 8, 4, 64, A, nullptr), QP_ERR_ALIGN);
    RUN("qmatmul overflow", qmatmul(A, BF, int64_t(1) << 62, 128, WQ, A, A, BF, int64_t(1) << 62, 4, 64, A, nullptr), QP_ERR_INVALID_ARG);
    RUN("qmatmul dtype 9", qmatmul(A, (qp_dtype)9, 2, 128, WQ, A, A, BF, 8, 4, 64, A, nullptr), QP_ERR_INVALID_ARG);

    // quantize / dequantize
    RUN("quantize ok", qpack_quantize(FP, 4, 128, 4, 64, BF, static_cast<uint32_t*>(A), A, A, nullptr), QP_OK);
    RUN("quantize null", qpack_quantize(nullptr, 4, 128, 4, 64, BF, static_cast<uint32_t*>(A), A, A, nullptr), QP_ERR_INVALID_ARG);
    RUN("quantize bits 7", qpack_quantize(FP, 4, 128, 7, 64, BF, static_cast<uint32_t*>(A), A, A, nullptr), QP_ERR_UNSUPPORTED);
    RUN("quantize odd", qpack_quantize(FP, 4, 128, 4, 64, BF, static_cast<uint32_t*>(ODD), A, A, nullptr), QP_ERR_ALIGN);
    RUN("dequantize ok", qpack_dequantize(WQ, A, A, BF, 4, 128, 3, 32, F32, A, nullptr), QP_OK);
    RUN("dequantize shape", qpack_dequantize(WQ, A, A, BF, 4, 100, 3, 32, F32, A, nullptr), QP_ERR_SHAPE);
    RUN("dequantize null", qpack_dequantize(WQ, nullptr, A, BF, 4, 128, 3, 32, F32, A, nullptr), QP_ERR_INVALID_ARG);
    RUN("dequantize_mx ok", qpack_dequantize_mx(WQ, static_cast<const uint8_t*>(A), QP_MXFP4, 4, 64, BF, A, nullptr), QP_OK);
    RUN("dequantize_mx mode", qpack_dequantize_mx(WQ, static_cast<const uint8_t*>(A), (qp_mode)7, 4, 64, BF, A, nullptr), QP_ERR_UNSUPPORTED);
    RUN("qmatmul_mx ok", qmatmul_mx(A, BF, 2, 64, WQ, static_cast<const uint8_t*>(A), QP_NVFP4, 8, A, nullptr), QP_OK);
    RUN("qmatmul_mx null", qmatmul_mx(A, BF, 2, 64, nullptr, static_cast<const uint8_t*>(A), QP_NVFP4, 8, A, nullptr), QP_ERR_INVALID_ARG);

    // MoE
    const size_t ws = qgemv_moe_workspace_bytes(6, 4);
    RUN("moe ok", qgemv_moe_id(A, BF, IDS, 3, 2, 128, 0, WQ, A, A, BF, 4, 16, 128, 4, 64, A, A, ws, nullptr), QP_OK);
    RUN("moe workspace", qgemv_moe_id(A, BF, IDS, 3, 2, 128, 0, WQ, A, A, BF, 4, 16, 128, 4, 64, A, A, ws - 1, nullptr), QP_ERR_WORKSPACE);
    RUN("moe odd ids", qgemv_moe_id(A, BF, static_cast<const int32_t*>(reinterpret_cast<void*>(0x10002)), 3, 2, 128, 0, WQ, A, A, BF, 4, 16, 128, 4, 64, A, A, ws, nullptr), QP_ERR_ALIGN);
    RUN("moe experts", qgemv_moe_id(A, BF, IDS, 3, 2, 128, 0, WQ, A, A, BF, 0, 16, 128, 4, 64, A, A, ws, nullptr), QP_ERR_INVALID_ARG);
    RUN("moe gate_up ok", qgemv_moe_id_gate_up_silu(A, BF, IDS, 3, 2, 128, 0, WQ, A, A, WQ, A, A, BF, 4, 16, 128, 4, 64, A, A, ws, nullptr), QP_OK);
    RUN("moe gate_up null", qgemv_moe_id_gate_up_silu(A, BF, IDS, 3, 2, 128, 0, WQ, A, A, nullptr, A, A, BF, 4, 16, 128, 4, 64, A, A, ws, nullptr), QP_ERR_INVALID_ARG);
    RUN("moe noalloc limit", qgemv_moe_id_noalloc(A, BF, IDS, 1 << 20, 8, 128, 0, WQ, A, A, BF, 4, 16, 128, 4, 64, A, nullptr), QP_ERR_WORKSPACE);
    RUN("moe noalloc null", qgemv_moe_id_noalloc(nullptr, BF, IDS, 3, 2, 128, 0, WQ, A, A, BF, 4, 16, 128, 4, 64, A, nullptr), QP_ERR_INVALID_ARG);
    const size_t fws = qgemv_moe_ffn_workspace_bytes(3, 2, 4, 128, 64, BF);
    RUN("ffn ok", qgemv_moe_ffn(A, BF, IDS, FP, 3, 2, WQ, A, A, WQ, A, A, WQ, A, A, BF, 4, 128, 64, 4, 64, A, A, fws, nullptr), QP_OK);
    RUN("ffn workspace", qgemv_moe_ffn(A, BF, IDS, FP, 3, 2, WQ, A, A, WQ, A, A, WQ, A, A, BF, 4, 128, 64, 4, 64, A, A, 0, nullptr), QP_ERR_WORKSPACE);

    // Transposed product, int8 tensor.
    const size_t tws = qmatmul_t_workspace_bytes(2, 128, 64, 4);
    RUN("qmatmul_t ok", qmatmul_t(A, BF, 2, 128, WQ, A, A, BF, 64, 4, 64, A, A, tws, nullptr), QP_OK);
    RUN("qmatmul_t workspace", qmatmul_t(A, BF, 2, 128, WQ, A, A, BF, 64, 4, 64, A, A, 0, nullptr), QP_ERR_WORKSPACE);
    RUN("int8 quantize ok", qpack_quantize_int8_tensor(FP, 64, static_cast<int8_t*>(A), static_cast<float*>(A), nullptr), QP_OK);
    RUN("int8 quantize null", qpack_quantize_int8_tensor(nullptr, 64, static_cast<int8_t*>(A), static_cast<float*>(A), nullptr), QP_ERR_INVALID_ARG);
    RUN("int8 dequantize ok", qpack_dequantize_int8_tensor(static_cast<const int8_t*>(A), 64, FP, F16, A, nullptr), QP_OK);
    RUN("int8 qmatmul ok", qmatmul_int8_tensor(A, BF, 2, 64, static_cast<const int8_t*>(A), FP, 8, A, nullptr), QP_OK);
    RUN("int8 qmatmul odd", qmatmul_int8_tensor(A, BF, 2, 64, static_cast<const int8_t*>(A), FP, 8, ODD, nullptr), QP_ERR_ALIGN);

    if (std::strstr(qpack_version(), "gfx950") == nullptr) {
        std::fprintf(stderr, "FAIL version string\n");
        ++failures;
    }
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("abi driver: all calls clean (%d stub launches)\n", g_stub_launches);
    return 0;
}
