// gate.hip -- gate preparation: beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias).
//
// Megatron-Core API docs, "core.ssm.ops.gdp.decode_prepare": the module
// introduction gives both formulas; the "softplus" entry fixes softplus as
// log1p(exp(x)) in fp32, the identity once x exceeds 20, with log1p keeping
// the far-negative tail.
//
// An elementwise map over [R, H]; one thread per element, fp32 math with the
// accurate device exp / log1p and IEEE division. At the workloads' sizes
// (<= 2M elements, <= 25 MB) it is launch-bound; the decode path fuses the
// same formulas into its kernel instead of calling this one.
#include "gdn_common.hpp"

namespace gdn {

template <typename T>
__global__ __launch_bounds__(256) void gate_prepare_kernel(
    const T* __restrict__ a, int64_t asr, const T* __restrict__ b, int64_t bsr,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    float* __restrict__ g, float* __restrict__ beta, int R, int H)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)R * H) return;
    const int64_t r = i / H;
    const int h = (int)(i - r * H);
    const float av = to_f32(a[r * asr + h]);
    const float bv = to_f32(b[r * bsr + h]);
    beta[i] = gate_beta(bv);
    g[i] = gate_g(av, A_log[h], dt_bias[h]);
}

hipError_t launch_gate_prepare(const void* a, int64_t asr, const void* b, int64_t bsr,
                               const float* A_log, const float* dt_bias, float* g, float* beta,
                               int R, int H, bool bf16_in, hipStream_t stream)
{
    const int64_t n = (int64_t)R * H;
    dim3 grid((unsigned)((n + 255) / 256));
    if (bf16_in)
        hipLaunchKernelGGL(gate_prepare_kernel<bf16>, grid, dim3(256), 0, stream,
                           (const bf16*)a, asr, (const bf16*)b, bsr, A_log, dt_bias, g, beta, R, H);
    else
        hipLaunchKernelGGL(gate_prepare_kernel<float>, grid, dim3(256), 0, stream,
                           (const float*)a, asr, (const float*)b, bsr, A_log, dt_bias, g, beta, R, H);
    return hipGetLastError();
}

}  // namespace gdn
