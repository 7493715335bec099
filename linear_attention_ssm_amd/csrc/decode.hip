// decode.hip -- one decode token of a Gated DeltaProduct layer, fused:
// split + gate + L2 norm + M Householder sub-steps + readout, state in place.
//
// Megatron-Core API docs, "core.ssm.ops.gdp.decode_prepare": the module
// introduction describes the preparation (split value/key/query, expand q/k
// groups to heads, interleave the Householder copies with the query on the
// last copy and the decay on the first, gate ba into beta and g); the
// "gdp_decode_prepare" Returns list says the recurrent kernel then runs an
// M-length sequence per request. The preparation is launch-bound on its own,
// which is why it is fused here rather than written out.
//
// Design for CDNA4: the op streams the fp32 state (64 KiB per request and
// head at N = P = 128) once in and once out, so it is HBM bound. One
// 256-thread workgroup owns one (request, head) state: thread (rg, cg) holds
// columns 4cg..4cg+3 of rows rg, rg+RG, rg+2RG, ... in registers, loaded with
// 16-byte loads (a wave reads whole 512-byte rows: coalesced). Each sub-step
// needs h^T k (a reduction over rows): per-thread partial sums, then one LDS
// exchange across the RG row groups (double-buffered, one barrier per
// sub-step). The state never leaves registers between the M sub-steps, so it
// is read once and written once per token.
#include "gdn_common.hpp"

namespace gdn {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeMaxM = 4;

template <typename T, int NK, int PV>
__global__ __launch_bounds__(kDecodeThreads) void gdp_decode_kernel(
    const T* __restrict__ x, int64_t xs, const T* __restrict__ ba, int64_t bas,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    float* __restrict__ state, T* __restrict__ o,
    int M, int H, int G, float scale, int l2norm)
{
    constexpr int CG = PV / 4;               // column groups of 4
    constexpr int RG = kDecodeThreads / CG;  // row groups
    constexpr int RPT = NK / RG;             // rows per thread
    static_assert(RPT * RG == NK && CG * RG == kDecodeThreads, "tile shape");

    __shared__ float kv[kDecodeMaxM][NK];
    __shared__ float qv[kDecodeThreads > NK ? kDecodeThreads : NK];   // (staged past NK, unread)
    __shared__ float vv[kDecodeMaxM][PV];
    __shared__ __align__(16) float red[2][RG][PV];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int r = blockIdx.x / H;
    const int h = blockIdx.x - r * H;
    const int grp = h / (H / G);
    const T* xr = x + (int64_t)r * xs;
    const T* br = ba + (int64_t)r * bas;
    const int64_t k_base = (int64_t)M * H * PV;
    const int64_t q_base = k_base + (int64_t)M * G * NK;

    // --- the token's inputs, all requested at once (one memory round trip):
    // this head's value slices, its group's keys and query, b per copy and a
    constexpr int VPT = (kDecodeMaxM * PV + kDecodeThreads - 1) / kDecodeThreads;
    constexpr int KPT = (kDecodeMaxM * NK + kDecodeThreads - 1) / kDecodeThreads;
    constexpr int QPT = (NK + kDecodeThreads - 1) / kDecodeThreads;
    // (unpredicated loads of clamped indices, masked when staged: a predicated
    // load would get a wait of its own)
    T vin[VPT], kin[KPT], qin[QPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int e0 = tid + i * kDecodeThreads, e = e0 < M * PV ? e0 : 0;
        const int m = e / PV, p = e - m * PV;
        vin[i] = xr[((int64_t)m * H + h) * PV + p];
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int e0 = tid + i * kDecodeThreads, e = e0 < M * NK ? e0 : 0;
        const int m = e / NK, c = e - m * NK;
        kin[i] = xr[k_base + ((int64_t)m * G + grp) * NK + c];
    }
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int c0 = tid + i * kDecodeThreads, c = c0 < NK ? c0 : 0;
        qin[i] = xr[q_base + (int64_t)grp * NK + c];
    }
    // gate inputs, read by every thread (uniform addresses: one request each)
    T bin[kDecodeMaxM];
#pragma unroll
    for (int m = 0; m < kDecodeMaxM; ++m) bin[m] = br[(int64_t)(m < M ? m : 0) * H + h];
    const T ain = br[(int64_t)M * H + h];

    // --- then the state: the bulk of the traffic, in flight while the inputs
    // are staged and normalised
    const int cg = tid % CG;
    const int rg = tid / CG;
    float* st = state + ((int64_t)r * H + h) * NK * PV;
    f32x4 S[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j)
        S[j] = *reinterpret_cast<const f32x4*>(st + (int64_t)(rg + RG * j) * PV + 4 * cg);

    // (staged unconditionally: slots of copies >= M and query slots >= NK take
    // stand-in values nothing reads, and no load waits behind a branch)
    static_assert(VPT * kDecodeThreads <= kDecodeMaxM * PV && KPT * kDecodeThreads <= kDecodeMaxM * NK,
                  "staging stays inside the arrays");
#pragma unroll
    for (int i = 0; i < VPT; ++i) (&vv[0][0])[tid + i * kDecodeThreads] = to_f32(vin[i]);
#pragma unroll
    for (int i = 0; i < KPT; ++i) (&kv[0][0])[tid + i * kDecodeThreads] = to_f32(kin[i]);
#pragma unroll
    for (int i = 0; i < QPT; ++i) qv[tid + i * kDecodeThreads] = to_f32(qin[i]);
    // --- gates: beta per copy, the decay on copy 0 only (formed in every
    // thread's registers)
    float beta_r[kDecodeMaxM];
#pragma unroll
    for (int m = 0; m < kDecodeMaxM; ++m) beta_r[m] = gate_beta(to_f32(bin[m]));
    const float alpha = expf(gate_g(to_f32(ain), A_log[h], dt_bias[h]));
    __syncthreads();

    // --- L2 normalisation of k_0..k_{M-1} and q, one wave per vector
    if (l2norm) {
        for (int vec = wave; vec <= M; vec += kDecodeThreads / kWave) {
            float* z = (vec < M) ? kv[vec] : qv;
            float ss = 0.f;
            for (int i = lane; i < NK; i += kWave) ss += z[i] * z[i];
            ss = wave_sum(ss);
            float inv = 1.f / sqrtf(ss + 1e-6f);
            for (int i = lane; i < NK; i += kWave) z[i] *= inv;
        }
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < RPT; ++j) S[j] *= alpha;

    // --- M sub-steps: u = beta (v - h^T k); h += k u^T
#pragma unroll
    for (int m = 0; m < kDecodeMaxM; ++m) {
        if (m >= M) break;
        f32x4 part = zero4();
#pragma unroll
        for (int j = 0; j < RPT; ++j) part += S[j] * kv[m][rg + RG * j];
        *reinterpret_cast<f32x4*>(&red[m & 1][rg][4 * cg]) = part;
        __syncthreads();
        f32x4 hk = zero4();
#pragma unroll
        for (int a = 0; a < RG; ++a) hk += *reinterpret_cast<const f32x4*>(&red[m & 1][a][4 * cg]);
        const f32x4 vm = *reinterpret_cast<const f32x4*>(&vv[m][4 * cg]);
        const f32x4 u = beta_r[m] * (vm - hk);
#pragma unroll
        for (int j = 0; j < RPT; ++j) S[j] += kv[m][rg + RG * j] * u;
    }

    // --- readout of the last copy: o = scale * h^T q
    {
        f32x4 part = zero4();
#pragma unroll
        for (int j = 0; j < RPT; ++j) part += S[j] * qv[rg + RG * j];
        *reinterpret_cast<f32x4*>(&red[M & 1][rg][4 * cg]) = part;
        __syncthreads();
        if (rg == 0) {
            f32x4 acc = zero4();
#pragma unroll
            for (int a = 0; a < RG; ++a) acc += *reinterpret_cast<const f32x4*>(&red[M & 1][a][4 * cg]);
            T* orow = o + ((int64_t)r * H + h) * PV + 4 * cg;
#pragma unroll
            for (int e = 0; e < 4; ++e) orow[e] = from_f32<T>(scale * acc[e]);
        }
    }

    // the updated state streams out: nothing reads it back within this launch,
    // and non-temporal writes keep it from displacing other data on its way out
#pragma unroll
    for (int j = 0; j < RPT; ++j)
        __builtin_nontemporal_store(S[j], reinterpret_cast<f32x4*>(st + (int64_t)(rg + RG * j) * PV + 4 * cg));
}

template <typename T, int NK, int PV>
static void launch_decode_nkpv(const void* x, int64_t xs, const void* ba, int64_t bas,
                               const float* A_log, const float* dt_bias, float* state, void* o,
                               int n, int M, int H, int G, float scale, int l2norm,
                               hipStream_t stream)
{
    hipLaunchKernelGGL((gdp_decode_kernel<T, NK, PV>), dim3((unsigned)((int64_t)n * H)),
                       dim3(kDecodeThreads), 0, stream, (const T*)x, xs, (const T*)ba, bas,
                       A_log, dt_bias, state, (T*)o, M, H, G, scale, l2norm);
}

template <typename T>
static void launch_decode_t(const void* x, int64_t xs, const void* ba, int64_t bas,
                            const float* A_log, const float* dt_bias, float* state, void* o,
                            int n, int M, int H, int G, int P, int N, float scale, int l2norm,
                            hipStream_t stream)
{
    if (N == 128 && P == 128)
        launch_decode_nkpv<T, 128, 128>(x, xs, ba, bas, A_log, dt_bias, state, o, n, M, H, G, scale, l2norm, stream);
    else if (N == 128 && P == 64)
        launch_decode_nkpv<T, 128, 64>(x, xs, ba, bas, A_log, dt_bias, state, o, n, M, H, G, scale, l2norm, stream);
    else if (N == 64 && P == 128)
        launch_decode_nkpv<T, 64, 128>(x, xs, ba, bas, A_log, dt_bias, state, o, n, M, H, G, scale, l2norm, stream);
    else
        launch_decode_nkpv<T, 64, 64>(x, xs, ba, bas, A_log, dt_bias, state, o, n, M, H, G, scale, l2norm, stream);
}

hipError_t launch_recurrent_decode(const void* x, int64_t xs, const void* ba, int64_t bas,
                                   const float* A_log, const float* dt_bias, float* state,
                                   void* o, int n, int M, int H, int G, int P, int N, float scale,
                                   int l2norm, bool bf16_io, hipStream_t stream)
{
    if (bf16_io)
        launch_decode_t<bf16>(x, xs, ba, bas, A_log, dt_bias, state, o, n, M, H, G, P, N, scale, l2norm, stream);
    else
        launch_decode_t<float>(x, xs, ba, bas, A_log, dt_bias, state, o, n, M, H, G, P, N, scale, l2norm, stream);
    return hipGetLastError();
}

}  // namespace gdn
