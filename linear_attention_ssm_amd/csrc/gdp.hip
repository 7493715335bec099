// gdp.hip -- the Gated DeltaProduct steps around the recurrent core.
//
// Megatron-Core API docs, "core.ssm.ops.gdp.decode_prepare":
//   * the module introduction places the preparation between the short-conv
//     update and the recurrent kernel: split the post-conv row into value,
//     key and query, GQA-expand query and key, interleave the M Householder
//     copies (query on the last copy, the decay on the first) and gate the ba
//     slice; a -1 slot zeroes the short-conv output of a padding request;
//   * "gdp_decode_prepare" returns query, key [n, M, H, N], value [n, M, H, P]
//     and beta, g [n, M, H] (fp32), the layouts of an M-length sequence per
//     request.
// Three kernels:
//   gdp_decode_prepare_kernel   that five-tensor export for one decode step
//                               (query / key / value plain copies, one thread
//                               per 16-byte output vector);
//   conv1d_update_kernel        the short-conv state update of one decode
//                               token per request (W - 1 past rows per slot);
//   gdp_prefill_prepare_kernel  the same interleave for a whole prefill: row
//                               t * M + m of an M*T-token sequence is copy m of
//                               token t, so the chunked forward runs a Gated
//                               DeltaProduct layer unchanged (the decay on copy
//                               0, the query on copy M - 1; the outputs of token
//                               t are row t * M + M - 1).
// All three move whole 16-byte vectors (a row of P or N elements is 128 or 256
// bytes) and form the gates with the shared formulas of gdn_common.hpp.
#include "gdn_common.hpp"

namespace gdn {

constexpr int kGdpThreads = 256;

// Copy `units` 16-byte vectors from src to dst (or write zeros), spread over the block.
template <typename V>
__device__ __forceinline__ void copy_units(V* __restrict__ dst, const V* __restrict__ src, int units,
                                           bool zero) {
    for (int i = threadIdx.x; i < units; i += kGdpThreads) dst[i] = zero ? V{} : src[i];
}

// One thread per 16-byte vector of the value, key and query outputs (in that
// order, output-major), then one per gate element: row r of x is
// v [M][H][P] | k [M][G][N] | q [G][N].
template <typename T>
__global__ __launch_bounds__(kGdpThreads) void gdp_decode_prepare_kernel(
    const T* __restrict__ x, int64_t xs, const T* __restrict__ ba, int64_t bas,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    T* __restrict__ qo, T* __restrict__ ko, T* __restrict__ vo, float* __restrict__ beta,
    float* __restrict__ g, int n, int M, int H, int G, int P, int N)
{
    typedef typename V16<T>::type V;
    constexpr int VN = V16<T>::n;
    // 32-bit index arithmetic (the entry point bounds the work); P / VN and
    // N / VN are powers of two
    const uint32_t psh = __builtin_ctz((uint32_t)(P / VN)), nsh = __builtin_ctz((uint32_t)(N / VN));
    const uint32_t MH = (uint32_t)(M * H);
    const uint32_t rows = (uint32_t)n * MH;             // (request, copy, head) rows
    const uint32_t nv = rows << psh, nk = rows << nsh;
    uint32_t i = blockIdx.x * kGdpThreads + threadIdx.x;
    const int64_t kbase = (int64_t)M * H * P, qbase = kbase + (int64_t)M * G * N;
    if (i < nv) {
        // value: output row (r, m, h) is x[r][(m H + h) P ..]
        const uint32_t o = i >> psh, u = i & ((1u << psh) - 1);
        const uint32_t r = o / MH, mh = o - r * MH;
        reinterpret_cast<V*>(vo)[i] = reinterpret_cast<const V*>(x + (int64_t)r * xs + (int64_t)mh * P)[u];
        return;
    }
    i -= nv;
    if (i < 2 * nk) {
        // key (i < nk) or query: head h reads group h / (H/G)
        const bool isq = i >= nk;
        const uint32_t j = isq ? i - nk : i;
        const uint32_t o = j >> nsh, u = j & ((1u << nsh) - 1);
        const uint32_t r = o / MH, mh = o - r * MH;
        const uint32_t m = mh / (uint32_t)H, h = mh - m * (uint32_t)H;
        const uint32_t grp = h / (uint32_t)(H / G);
        const T* src = x + (int64_t)r * xs + (isq ? qbase + (int64_t)grp * N : kbase + ((int64_t)m * G + grp) * N);
        const V val = isq && (int)m != M - 1 ? V{} : reinterpret_cast<const V*>(src)[u];
        reinterpret_cast<V*>(isq ? qo : ko)[j] = val;
        return;
    }
    i -= 2 * nk;
    if (i < rows) {
        // gates: beta per copy, the decay on copy 0 only
        const uint32_t r = i / MH, mh = i - r * MH;
        const uint32_t m = mh / (uint32_t)H, h = mh - m * (uint32_t)H;
        const T* br = ba + (int64_t)r * bas;
        beta[i] = gate_beta(to_f32(br[(int64_t)m * H + h]));
        g[i] = m == 0 ? gate_g(to_f32(br[(int64_t)M * H + h]), A_log[h], dt_bias[h]) : 0.f;
    }
}

// One thread per (request, 16-byte channel group). conv_state [S, W-1, C]:
// row j of a slot is x[t - (W - 1) + j] for the next token t.
template <typename T>
__global__ __launch_bounds__(kGdpThreads) void conv1d_update_kernel(
    const T* __restrict__ x, int64_t xs, T* __restrict__ state, const int32_t* __restrict__ slot,
    const T* __restrict__ w, const T* __restrict__ bias, T* __restrict__ y, int64_t ys,
    int n_slots, int C, int silu)
{
    typedef V16<T> VV;
    typedef typename VV::type V;
    constexpr int VN = VV::n;
    constexpr int W = 4;
    const int r = blockIdx.x;
    const int cg = blockIdx.y * kGdpThreads + threadIdx.x;
    if (cg * VN >= C) return;
    const int c0 = cg * VN;
    V* yr = reinterpret_cast<V*>(y + (int64_t)r * ys + c0);
    const int s = slot[r];
    if (s < 0 || s >= n_slots) {   // padding request (or a slot outside the pool): zero output
        *yr = V{};
        return;
    }
    V* st = reinterpret_cast<V*>(state + (int64_t)s * (W - 1) * C + c0);
    const int64_t srow = C / VN;    // 16-byte vectors per state row
    const V xr = *reinterpret_cast<const V*>(x + (int64_t)r * xs + c0);
    V raw[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) raw[j] = st[j * srow];
    typename VV::ftype bs{};
    if (bias) bs = VV::to_float(*reinterpret_cast<const V*>(bias + c0));
    typename VV::ftype out;
    // the same arithmetic as the prefill kernel: taps wt[j][e] multiply
    // x[t - (W-1) + j][c0 + e] (bf16: as they lie, two to a word)
    if constexpr (sizeof(T) == 2) {
        uint32_t wp[2 * VN];
#pragma unroll
        for (int i = 0; i < W; ++i) {
            const u32x4 u = __builtin_bit_cast(u32x4, *reinterpret_cast<const V*>(w + (int64_t)c0 * W + i * VN));
#pragma unroll
            for (int d = 0; d < 4; ++d) wp[4 * i + d] = u[d];
        }
        const u32x4 w0 = __builtin_bit_cast(u32x4, raw[0]), w1 = __builtin_bit_cast(u32x4, raw[1]);
        const u32x4 w2 = __builtin_bit_cast(u32x4, raw[2]), xw = __builtin_bit_cast(u32x4, xr);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float a0 = conv_taps4_bf16(wp[4 * d], wp[4 * d + 1], bias ? bs[2 * d] : 0.f,
                                             pair_lo(w0[d], w1[d]), pair_lo(w2[d], xw[d]));
            const float a1 = conv_taps4_bf16(wp[4 * d + 2], wp[4 * d + 3], bias ? bs[2 * d + 1] : 0.f,
                                             pair_hi(w0[d], w1[d]), pair_hi(w2[d], xw[d]));
            out[2 * d] = silu ? conv_silu(a0) : a0;
            out[2 * d + 1] = silu ? conv_silu(a1) : a1;
        }
    } else {
        const typename VV::ftype xf = VV::to_float(xr);
        typename VV::ftype win[W - 1];
#pragma unroll
        for (int j = 0; j < W - 1; ++j) win[j] = VV::to_float(raw[j]);
        float wt[W][VN];
#pragma unroll
        for (int i = 0; i < W; ++i) {
            const typename VV::ftype f = VV::to_float(*reinterpret_cast<const V*>(w + (int64_t)c0 * W + i * VN));
#pragma unroll
            for (int u = 0; u < VN; ++u) {
                const int flat = i * VN + u;
                wt[flat % W][flat / W] = f[u];
            }
        }
#pragma unroll
        for (int e = 0; e < VN; ++e) {
            const float acc = conv_taps4(wt[0][e], wt[1][e], wt[2][e], wt[3][e], bias ? bs[e] : 0.f,
                                         win[0][e], win[1][e], win[2][e], xf[e]);
            out[e] = silu ? conv_silu(acc) : acc;
        }
    }
    *yr = VV::from_float(out);
    // the window moves one token on
    st[0] = raw[1];
    st[srow] = raw[2];
    st[2 * srow] = xr;
}

// One block per (token row, copy m) of a prefill: output row p = row * M + m.
template <typename T>
__global__ __launch_bounds__(kGdpThreads) void gdp_prefill_prepare_kernel(
    const T* __restrict__ x, int64_t xs, const T* __restrict__ ba, int64_t bas,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    const int32_t* __restrict__ cu, int n_seqs, int32_t* __restrict__ cu_out,
    T* __restrict__ qo, T* __restrict__ ko, T* __restrict__ vo, float* __restrict__ g,
    float* __restrict__ beta, int M, int H, int G, int P, int N)
{
    typedef typename V16<T>::type V;
    constexpr int VN = V16<T>::n;
    const int64_t row = blockIdx.x / M;
    const int m = (int)(blockIdx.x - row * M);
    const int64_t p = row * M + m;
    const T* xr = x + row * xs;
    const int64_t kbase = (int64_t)M * H * P, qbase = kbase + (int64_t)M * G * N;
    copy_units(reinterpret_cast<V*>(vo + p * H * P), reinterpret_cast<const V*>(xr + (int64_t)m * H * P),
               H * P / VN, false);
    copy_units(reinterpret_cast<V*>(ko + p * G * N), reinterpret_cast<const V*>(xr + kbase + (int64_t)m * G * N),
               G * N / VN, false);
    copy_units(reinterpret_cast<V*>(qo + p * G * N), reinterpret_cast<const V*>(xr + qbase), G * N / VN,
               m != M - 1);
    const T* br = ba + row * bas;
    for (int h = threadIdx.x; h < H; h += kGdpThreads) {
        beta[p * H + h] = gate_beta(to_f32(br[(int64_t)m * H + h]));
        g[p * H + h] = m == 0 ? gate_g(to_f32(br[(int64_t)M * H + h]), A_log[h], dt_bias[h]) : 0.f;
    }
    if (cu && cu_out && blockIdx.x == 0)
        for (int i = threadIdx.x; i <= n_seqs; i += kGdpThreads) cu_out[i] = cu[i] * M;
}

hipError_t launch_decode_prepare(const void* x, int64_t xs, const void* ba, int64_t bas,
                                 const float* A_log, const float* dt_bias, void* q, void* k,
                                 void* v, float* beta, float* g, int n, int M, int H, int G, int P,
                                 int N, bool bf16_io, hipStream_t stream)
{
    const int vn = bf16_io ? 8 : 4;
    const int64_t rows = (int64_t)n * M * H;
    const int64_t work = rows * (P + 2 * N) / vn + rows;
    const dim3 grid((unsigned)((work + kGdpThreads - 1) / kGdpThreads));
    if (bf16_io)
        hipLaunchKernelGGL(gdp_decode_prepare_kernel<bf16>, grid, dim3(kGdpThreads), 0, stream,
                           (const bf16*)x, xs, (const bf16*)ba, bas, A_log, dt_bias, (bf16*)q,
                           (bf16*)k, (bf16*)v, beta, g, n, M, H, G, P, N);
    else
        hipLaunchKernelGGL(gdp_decode_prepare_kernel<float>, grid, dim3(kGdpThreads), 0, stream,
                           (const float*)x, xs, (const float*)ba, bas, A_log, dt_bias, (float*)q,
                           (float*)k, (float*)v, beta, g, n, M, H, G, P, N);
    return hipGetLastError();
}

hipError_t launch_conv1d_update(const void* x, int64_t xs, void* state, const int32_t* slot,
                                const void* w, const void* bias, void* y, int64_t ys, int n,
                                int n_slots, int C, int silu, bool bf16_io, hipStream_t stream)
{
    const int vn = bf16_io ? 8 : 4;
    const dim3 grid((unsigned)n, (unsigned)((C / vn + kGdpThreads - 1) / kGdpThreads));
    if (bf16_io)
        hipLaunchKernelGGL(conv1d_update_kernel<bf16>, grid, dim3(kGdpThreads), 0, stream,
                           (const bf16*)x, xs, (bf16*)state, slot, (const bf16*)w, (const bf16*)bias,
                           (bf16*)y, ys, n_slots, C, silu);
    else
        hipLaunchKernelGGL(conv1d_update_kernel<float>, grid, dim3(kGdpThreads), 0, stream,
                           (const float*)x, xs, (float*)state, slot, (const float*)w,
                           (const float*)bias, (float*)y, ys, n_slots, C, silu);
    return hipGetLastError();
}

hipError_t launch_gdp_prefill_prepare(const void* x, int64_t xs, const void* ba, int64_t bas,
                                      const float* A_log, const float* dt_bias, const int32_t* cu,
                                      int n_seqs, int32_t* cu_out, void* q, void* k, void* v,
                                      float* g, float* beta, int64_t rows, int M, int H, int G,
                                      int P, int N, bool bf16_io, hipStream_t stream)
{
    const dim3 grid((unsigned)(rows * M));
    if (bf16_io)
        hipLaunchKernelGGL(gdp_prefill_prepare_kernel<bf16>, grid, dim3(kGdpThreads), 0, stream,
                           (const bf16*)x, xs, (const bf16*)ba, bas, A_log, dt_bias, cu, n_seqs, cu_out,
                           (bf16*)q, (bf16*)k, (bf16*)v, g, beta, M, H, G, P, N);
    else
        hipLaunchKernelGGL(gdp_prefill_prepare_kernel<float>, grid, dim3(kGdpThreads), 0, stream,
                           (const float*)x, xs, (const float*)ba, bas, A_log, dt_bias, cu, n_seqs,
                           cu_out, (float*)q, (float*)k, (float*)v, g, beta, M, H, G, P, N);
    return hipGetLastError();
}

}  // namespace gdn
