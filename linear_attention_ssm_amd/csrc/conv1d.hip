// conv1d.hip -- depthwise causal convolution (W = 4) with optional SiLU.
//
// "ZzCompute" (PyTorch Helion Hackathon gallery), item 1 "Causal Conv1d":
// each channel is convolved with its own past; the width is a compile-time
// constant so the tap loop unrolls; out-of-range taps are masked to zero
// instead of padding on the host; the operation is memory bound.
//
// Design for CDNA4: the op streams [B, T, C] once in and once out, so it is
// bound by HBM. A thread owns one 16-byte group of channels (8 bf16 or 4
// fp32) for a run of RUN consecutive tokens: it issues all RUN row loads up
// front (RUN x 16 B in flight per lane), keeps the last W-1 inputs in
// registers as a sliding window, and writes each output row with one 16-byte
// store. A wave covers 64 adjacent channel groups (1 KiB of one token row),
// so every access is a fully coalesced 1 KiB segment. Taps before the start
// of a token's sequence read zero; with packed sequences the run tracks the
// next boundary and clears its window there.
#include <climits>

#include "gdn_common.hpp"

namespace gdn {

constexpr int kConvW = 4;
constexpr int kConvRun = 16;       // tokens per thread (default)
constexpr int kConvThreads = 256;  // threads per workgroup (default)

template <typename T, int RUN, int NTH>
__global__ __launch_bounds__(NTH) void conv1d_causal_kernel(
    const T* __restrict__ x, int64_t xsb, int64_t xst,
    const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ y, int64_t ysb, int64_t yst,
    const int32_t* __restrict__ cu, int n_seqs,
    int T_len, int C, int runs_per_row, int runs_total, int runs_pad, int silu)
{
    typedef V16<T> V;
    constexpr int VN = V::n;
    // XCD-aware block order: each XCD (blockIdx % 8) takes a contiguous range
    // of runs, so the W-1 rows before a run were just fetched into the same L2
    // by the run before it
    const int ncg = C / VN;
    const int per_xcd = runs_pad / 8;
    const int j = blockIdx.x >> 3;
    const int cgb = j / per_xcd;
    const int run = (blockIdx.x & 7) * per_xcd + (j - cgb * per_xcd);
    const int cg = cgb * NTH + threadIdx.x;
    if (cg >= ncg || run >= runs_total) return;
    const int b = run / runs_per_row;
    const int t0 = (run % runs_per_row) * RUN;
    const int c0 = cg * VN;

    // taps: wt[j][e] multiplies x[t - (W-1) + j][c0 + e]; the group's VN x W taps
    // are contiguous, read as W 16-byte vectors (bf16: kept as they lie, two
    // taps to a word: word 2 e holds (w0, w1) of channel e, word 2 e + 1 (w2, w3))
    float wt[kConvW][VN];
    uint32_t wp[2 * VN];
#pragma unroll
    for (int i = 0; i < kConvW; ++i) {
        const typename V::type raw_w = *reinterpret_cast<const typename V::type*>(w + (int64_t)c0 * kConvW + i * VN);
        if constexpr (sizeof(T) == 2) {
            const u32x4 u = __builtin_bit_cast(u32x4, raw_w);
#pragma unroll
            for (int d = 0; d < 4; ++d) wp[4 * i + d] = u[d];
        } else {
            const typename V::ftype f = V::to_float(raw_w);
#pragma unroll
            for (int u = 0; u < VN; ++u) {
                const int flat = i * VN + u;            // = e * W + j
                wt[flat % kConvW][flat / kConvW] = f[u];
            }
        }
    }
    float bs[VN];
    if (bias) {
        const typename V::ftype f = V::to_float(*reinterpret_cast<const typename V::type*>(bias + c0));
#pragma unroll
        for (int e = 0; e < VN; ++e) bs[e] = f[e];
    } else {
#pragma unroll
        for (int e = 0; e < VN; ++e) bs[e] = 0.f;
    }

    const T* xb = x + (int64_t)b * xsb + c0;
    T* yb = y + (int64_t)b * ysb + c0;

    // sequence bounds of the first token of the run
    int seq_start = 0, seq_end = T_len, si = 0;
    if (cu) {
        si = find_seq(cu, n_seqs, t0 < T_len ? t0 : T_len - 1);
        seq_start = cu[si];
        seq_end = cu[si + 1];
    }

    // issue every load of the run (window + RUN rows) before using any
    // (unpredicated loads of clamped rows, zeroed after: all stay in flight together)
    typename V::type raw[kConvW - 1 + RUN];
#pragma unroll
    for (int i = 0; i < kConvW - 1 + RUN; ++i) {
        const int t = t0 - (kConvW - 1) + i;
        const int tc = min(max(t, 0), T_len - 1);
        raw[i] = *reinterpret_cast<const typename V::type*>(xb + (int64_t)tc * xst);
        if (t < 0 || t >= T_len) raw[i] = typename V::type{};
    }

    if constexpr (sizeof(T) == 2) {
        // the window as raw words (two channels each): x[t-3], x[t-2], x[t-1]
        u32x4 win[kConvW - 1];
#pragma unroll
        for (int i = 0; i < kConvW - 1; ++i) {
            const int t = t0 - (kConvW - 1) + i;
            win[i] = t >= seq_start ? __builtin_bit_cast(u32x4, raw[i]) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < RUN; ++i) {
            const int t = t0 + i;
            if (t >= T_len) break;
            if (cu && t >= seq_end) {
                // crossed into a later sequence: its taps start from zero
                while (t >= seq_end) { ++si; seq_start = cu[si]; seq_end = cu[si + 1]; }
#pragma unroll
                for (int a = 0; a < kConvW - 1; ++a)
                    if (t - (kConvW - 1) + a < seq_start) win[a] = u32x4{0u, 0u, 0u, 0u};
            }
            const u32x4 xw = __builtin_bit_cast(u32x4, raw[kConvW - 1 + i]);
            typename V::ftype out;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const float a0 = conv_taps4_bf16(wp[4 * d], wp[4 * d + 1], bs[2 * d],
                                                 pair_lo(win[0][d], win[1][d]), pair_lo(win[2][d], xw[d]));
                const float a1 = conv_taps4_bf16(wp[4 * d + 2], wp[4 * d + 3], bs[2 * d + 1],
                                                 pair_hi(win[0][d], win[1][d]), pair_hi(win[2][d], xw[d]));
                out[2 * d] = silu ? conv_silu(a0) : a0;
                out[2 * d + 1] = silu ? conv_silu(a1) : a1;
            }
            win[0] = win[1];
            win[1] = win[2];
            win[2] = xw;
            *reinterpret_cast<typename V::type*>(yb + (int64_t)t * yst) = V::from_float(out);
        }
    } else {
        float win[kConvW - 1][VN];   // x[t-3], x[t-2], x[t-1]
#pragma unroll
        for (int i = 0; i < kConvW - 1; ++i) {
            int t = t0 - (kConvW - 1) + i;
            typename V::ftype f = V::to_float(raw[i]);
            bool live = (t >= seq_start);
#pragma unroll
            for (int e = 0; e < VN; ++e) win[i][e] = live ? f[e] : 0.f;
        }

#pragma unroll
        for (int i = 0; i < RUN; ++i) {
            const int t = t0 + i;
            if (t >= T_len) break;
            if (cu && t >= seq_end) {
                // crossed into a later sequence: its taps start from zero
                while (t >= seq_end) { ++si; seq_start = cu[si]; seq_end = cu[si + 1]; }
#pragma unroll
                for (int a = 0; a < kConvW - 1; ++a)
#pragma unroll
                    for (int e = 0; e < VN; ++e)
                        win[a][e] = (t - (kConvW - 1) + a >= seq_start) ? win[a][e] : 0.f;
            }
            typename V::ftype xf = V::to_float(raw[kConvW - 1 + i]);
            typename V::ftype out;
#pragma unroll
            for (int e = 0; e < VN; ++e) {
                const float acc = conv_taps4(wt[0][e], wt[1][e], wt[2][e], wt[3][e], bs[e],
                                             win[0][e], win[1][e], win[2][e], xf[e]);
                out[e] = silu ? conv_silu(acc) : acc;
                win[0][e] = win[1][e];
                win[1][e] = win[2][e];
                win[2][e] = xf[e];
            }
            *reinterpret_cast<typename V::type*>(yb + (int64_t)t * yst) = V::from_float(out);
        }
    }
}

template <typename T, int RUN, int NTH>
static hipError_t launch_conv1d_cfg(const void* x, int64_t xsb, int64_t xst, const void* w,
                                    const void* bias, void* y, int64_t ysb, int64_t yst,
                                    const int32_t* cu, int n_seqs, int B, int T_len, int C,
                                    int silu, hipStream_t stream)
{
    const int ncg = C / V16<T>::n;
    const int runs = (T_len + RUN - 1) / RUN;
    const int total = runs * B;
    const int pad = (total + 7) / 8 * 8;
    const int cgb = (ncg + NTH - 1) / NTH;
    hipLaunchKernelGGL((conv1d_causal_kernel<T, RUN, NTH>), dim3((unsigned)(pad * cgb)), dim3(NTH),
                       0, stream, (const T*)x, xsb, xst, (const T*)w, (const T*)bias, (T*)y, ysb,
                       yst, cu, n_seqs, T_len, C, runs, total, pad, silu);
    return hipGetLastError();
}

template <typename T, int RUN>
static hipError_t launch_conv1d_run(int nth, const void* x, int64_t xsb, int64_t xst,
                                    const void* w, const void* bias, void* y, int64_t ysb,
                                    int64_t yst, const int32_t* cu, int n_seqs, int B, int T_len,
                                    int C, int silu, hipStream_t stream)
{
    if (nth == 64)
        return launch_conv1d_cfg<T, RUN, 64>(x, xsb, xst, w, bias, y, ysb, yst, cu, n_seqs, B, T_len, C, silu, stream);
    if (nth == 128)
        return launch_conv1d_cfg<T, RUN, 128>(x, xsb, xst, w, bias, y, ysb, yst, cu, n_seqs, B, T_len, C, silu, stream);
    return launch_conv1d_cfg<T, RUN, 256>(x, xsb, xst, w, bias, y, ysb, yst, cu, n_seqs, B, T_len, C, silu, stream);
}

template <typename T>
hipError_t launch_conv1d_t(const void* x, int64_t xsb, int64_t xst, const void* w,
                           const void* bias, void* y, int64_t ysb, int64_t yst,
                           const int32_t* cu, int n_seqs, int B, int T_len, int C, int silu,
                           hipStream_t stream)
{
    // the tuned configuration, unless its grid would not fit (the default's is
    // checked by the entry point)
    int run = tune_knob[kTuneConvRun] ? tune_knob[kTuneConvRun] : kConvRun;
    int nth = tune_knob[kTuneConvThreads] ? tune_knob[kTuneConvThreads] : kConvThreads;
    const int64_t grid = ((int64_t)(T_len + run - 1) / run * B + 7) / 8 * 8 *
                         ((C / V16<T>::n + nth - 1) / nth);
    if (grid > INT_MAX) { run = kConvRun; nth = kConvThreads; }
    if (run == 8)
        return launch_conv1d_run<T, 8>(nth, x, xsb, xst, w, bias, y, ysb, yst, cu, n_seqs, B, T_len, C, silu, stream);
    if (run == 32)
        return launch_conv1d_run<T, 32>(nth, x, xsb, xst, w, bias, y, ysb, yst, cu, n_seqs, B, T_len, C, silu, stream);
    return launch_conv1d_run<T, 16>(nth, x, xsb, xst, w, bias, y, ysb, yst, cu, n_seqs, B, T_len, C, silu, stream);
}

hipError_t launch_conv1d(const void* x, int64_t xsb, int64_t xst, const void* w,
                         const void* bias, void* y, int64_t ysb, int64_t yst,
                         const int32_t* cu, int n_seqs, int B, int T_len, int C, int silu,
                         bool bf16_io, hipStream_t stream)
{
    if (bf16_io)
        return launch_conv1d_t<bf16>(x, xsb, xst, w, bias, y, ysb, yst, cu, n_seqs, B, T_len, C,
                                     silu, stream);
    return launch_conv1d_t<float>(x, xsb, xst, w, bias, y, ysb, yst, cu, n_seqs, B, T_len, C,
                                  silu, stream);
}

}  // namespace gdn
