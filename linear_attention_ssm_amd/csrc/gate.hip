// gate.hip -- gate preparation: beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias).
//
// Megatron-Core API docs, "core.ssm.ops.gdp.decode_prepare": the module
// introduction gives both formulas; the "softplus" entry fixes softplus as
// log1p(exp(x)) in fp32, the identity once x exceeds 20, with log1p keeping
// the far-negative tail.
//
// An elementwise map over [R, H], fp32 math with the accurate device exp /
// log1p and IEEE division. When H is a multiple of 4 and the rows allow it,
// a thread takes four consecutive heads of one row (one 8- or 16-byte load
// per input, one 16-byte store per output; 32-bit index arithmetic), else one
// element. At the workloads' sizes (<= 2M elements, <= 25 MB) it is close to
// launch-bound; the decode path fuses the same formulas into its kernel
// instead of calling this one.
#include <climits>
#include <cstdint>

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

// four heads of one row per thread (H % 4 == 0, aligned rows)
template <typename T>
__global__ __launch_bounds__(256) void gate_prepare4_kernel(
    const T* __restrict__ a, int asr, const T* __restrict__ b, int bsr,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    float* __restrict__ g, float* __restrict__ beta, int R, int H4)
{
    typedef T T4 __attribute__((ext_vector_type(4)));
    const int i = blockIdx.x * 256 + threadIdx.x;   // (row, group of 4 heads)
    if (i >= R * H4) return;
    const int r = i / H4;
    const int h = 4 * (i - r * H4);
    const T4 av = *reinterpret_cast<const T4*>(a + (int64_t)r * asr + h);
    const T4 bv = *reinterpret_cast<const T4*>(b + (int64_t)r * bsr + h);
    const f32x4 Al = *reinterpret_cast<const f32x4*>(A_log + h);
    const f32x4 db = *reinterpret_cast<const f32x4*>(dt_bias + h);
    f32x4 go, bo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bo[e] = gate_beta(to_f32(bv[e]));
        go[e] = gate_g(to_f32(av[e]), Al[e], db[e]);
    }
    *reinterpret_cast<f32x4*>(beta + 4 * (int64_t)i) = bo;
    *reinterpret_cast<f32x4*>(g + 4 * (int64_t)i) = go;
}

hipError_t launch_gate_prepare(const void* a, int64_t asr, const void* b, int64_t bsr,
                               const float* A_log, const float* dt_bias, float* g, float* beta,
                               int R, int H, bool bf16_in, hipStream_t stream)
{
    const int64_t n = (int64_t)R * H;
    const int es = bf16_in ? 2 : 4;
    const auto al = [](const void* p, int bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; };
    if (H % 4 == 0 && n / 4 < INT_MAX && asr < INT_MAX && bsr < INT_MAX && (asr * es) % (4 * es) == 0 &&
        (bsr * es) % (4 * es) == 0 && al(a, 4 * es) && al(b, 4 * es) && al(A_log, 16) &&
        al(dt_bias, 16) && al(g, 16) && al(beta, 16)) {
        const int m = (int)(n / 4);
        dim3 grid((unsigned)((m + 255) / 256));
        if (bf16_in)
            hipLaunchKernelGGL(gate_prepare4_kernel<bf16>, grid, dim3(256), 0, stream, (const bf16*)a,
                               (int)asr, (const bf16*)b, (int)bsr, A_log, dt_bias, g, beta, R, H / 4);
        else
            hipLaunchKernelGGL(gate_prepare4_kernel<float>, grid, dim3(256), 0, stream, (const float*)a,
                               (int)asr, (const float*)b, (int)bsr, A_log, dt_bias, g, beta, R, H / 4);
        return hipGetLastError();
    }
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
