// abi_stubs.cpp — stand-ins for the library's launchers, so that the host
// side of the C ABI (api.cpp) can be built alone with sanitizers and run
// without a GPU. Every launcher counts its calls and succeeds without
// touching memory; the driver checks that argument errors launch nothing.
#include "../../weight_only_quantized_qgemv_amd/csrc/launch.hpp"

extern "C" int g_stub_launches = 0;

namespace qp {

#define STUB(decl)                                                                                 \
    decl                                                                                           \
    {                                                                                              \
        ++g_stub_launches;                                                                         \
        return hipSuccess;                                                                         \
    }
STUB(hipError_t launch_qgemv_b2(const GemvArgs&, hipStream_t))
STUB(hipError_t launch_qgemv_b3(const GemvArgs&, hipStream_t))
STUB(hipError_t launch_qgemv_b4(const GemvArgs&, hipStream_t))
STUB(hipError_t launch_qgemv_b6(const GemvArgs&, hipStream_t))
STUB(hipError_t launch_qgemv_b8(const GemvArgs&, hipStream_t))
STUB(hipError_t launch_qgemm(const GemvArgs&, hipStream_t))
STUB(hipError_t launch_fill_zero(void*, int, int64_t, hipStream_t))
STUB(hipError_t launch_quantize(const QuantizeArgs&, hipStream_t))
STUB(hipError_t launch_dequantize(const DequantArgs&, hipStream_t))
STUB(hipError_t launch_dequantize_mx(const DequantMxArgs&, hipStream_t))
STUB(hipError_t launch_qmatmul_mx(const GemvMxArgs&, hipStream_t))
STUB(hipError_t launch_qgemm_mx(const GemvMxArgs&, hipStream_t))
STUB(hipError_t launch_moe(const MoeArgs&, hipStream_t))
STUB(hipError_t launch_moe_pair(const MoeArgs&, const MoeArgs&, hipStream_t))
STUB(hipError_t launch_qgemv_t(const QgemvTArgs&, hipStream_t))
STUB(hipError_t launch_quantize_int8_tensor(const float*, int64_t, int8_t*, float*, hipStream_t))
STUB(hipError_t launch_dequantize_int8_tensor(const int8_t*, int64_t, const float*, int, void*,
                                              hipStream_t))
STUB(hipError_t launch_qmatmul_int8_tensor(const Int8TensorArgs&, hipStream_t))
STUB(hipError_t launch_moe_combine(const MoeCombineArgs&, hipStream_t))
STUB(hipError_t launch_moe_down_combine(const MoeArgs&, const float*, void*, hipStream_t))
#undef STUB

// The FFN block takes its two-launch close in this build.
bool moe_down_combine_ok(const MoeArgs&) { return false; }

bool qgemm_mx_fits(const GemvMxArgs&) { return false; }
// Sizes only need to be positive and grow with the problem here.
size_t moe_workspace_bytes(int64_t n_pairs, int64_t num_experts)
{
    return 1024 + (size_t)(n_pairs > 0 ? n_pairs : 1) * 16 + (size_t)num_experts * 12;
}
QgemvTPlan qgemv_t_plan(int64_t m, int64_t, int64_t n, int)
{
    return QgemvTPlan{1, (int)m, (size_t)(m * n * 4)};
}

} // namespace qp
