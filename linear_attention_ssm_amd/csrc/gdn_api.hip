// gdn_api.hip -- the C ABI declared in include/gdn.h: argument validation,
// dtype / shape dispatch, workspace carving and launches on the caller's
// stream. Validation finishes before the first HIP call, so a rejected call
// has no side effect and the checks can be exercised without a GPU.
#include <climits>
#include <cstdint>
#include <mutex>

#include "../../include/gdn.h"
#include "gdn_common.hpp"

namespace gdn {
hipError_t launch_conv1d(const void* x, int64_t xsb, int64_t xst, const void* w, const void* bias,
                         void* y, int64_t ysb, int64_t yst, const int32_t* cu, int n_seqs, int B,
                         int T_len, int C, int silu, bool bf16_io, hipStream_t stream);
hipError_t launch_gate_prepare(const void* a, int64_t asr, const void* b, int64_t bsr,
                               const float* A_log, const float* dt_bias, float* g, float* beta,
                               int R, int H, bool bf16_in, hipStream_t stream);
size_t chunk_workspace_bytes(int B, int T_len, int H, int n_seqs, bool packed, bool bf16);
hipError_t launch_chunk_prepare(const void* q, const void* k, int64_t qks, const float* g,
                                const float* beta, const int32_t* cu, int n_seqs, int B, int T_len,
                                int H, int Hk, int K, float scale, int l2norm, bool use_bf16,
                                void* ws, hipStream_t stream);
hipError_t launch_chunk_scan(const void* q, const void* k, int64_t qks, const void* v, int64_t vs,
                             const float* S0, float* Sf, void* o, const int32_t* cu, int n_seqs,
                             int B, int T_len, int H, int Hk, int K, int V, bool use_bf16,
                             const void* ws, hipStream_t stream);
size_t prefill_workspace_bytes(int B, int T_len, int H, int Hk, int K, int n_seqs, bool packed);
hipError_t launch_prefill_prepare(const void* x, int64_t xs, const void* cw, const void* cb,
                                  const void* a, int64_t as, const void* b, int64_t bs,
                                  const float* A_log, const float* dt_bias, const int32_t* cu,
                                  int n_seqs, int B, int T_len, int H, int Hk, int K, float scale,
                                  int l2norm, void* ws, hipStream_t stream);
hipError_t launch_prefill_scan(const void* x, int64_t xs, const void* cw, const void* cb,
                               const float* S0, float* Sf, void* o, const int32_t* cu, int n_seqs,
                               int B, int T_len, int H, int Hk, int K, int V, void* ws,
                               hipStream_t stream);
hipError_t launch_recurrent_decode(const void* x, int64_t xs, const void* ba, int64_t bas,
                                   const float* A_log, const float* dt_bias, float* state,
                                   void* o, int n, int M, int H, int G, int P, int N, float scale,
                                   int l2norm, bool bf16_io, hipStream_t stream);
hipError_t launch_decode_prepare(const void* x, int64_t xs, const void* ba, int64_t bas,
                                 const float* A_log, const float* dt_bias, void* q, void* k,
                                 void* v, float* beta, float* g, int n, int M, int H, int G, int P,
                                 int N, bool bf16_io, hipStream_t stream);
hipError_t launch_conv1d_update(const void* x, int64_t xs, void* state, const int32_t* slot,
                                const void* w, const void* bias, void* y, int64_t ys, int n,
                                int n_slots, int C, int silu, bool bf16_io, hipStream_t stream);
hipError_t launch_gdp_prefill_prepare(const void* x, int64_t xs, const void* ba, int64_t bas,
                                      const float* A_log, const float* dt_bias, const int32_t* cu,
                                      int n_seqs, int32_t* cu_out, void* q, void* k, void* v,
                                      float* g, float* beta, int64_t rows, int M, int H, int G,
                                      int P, int N, bool bf16_io, hipStream_t stream);
}  // namespace gdn

namespace gdn {
int tune_knob[kTuneKnobs] = {0, 0, 0, 0};
}  // namespace gdn

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool valid_dtype(int d) { return d == GDN_FP32 || d == GDN_BF16; }
inline int elem_size(int d) { return d == GDN_BF16 ? 2 : 4; }
inline bool head_dim_ok(int d) { return d == 64 || d == 128; }
// a row stride in elements that keeps every row 16-byte aligned
inline bool stride16(int64_t s, int dtype) { return (s * elem_size(dtype)) % 16 == 0; }

inline int status_from(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ELAUNCH; }

}  // namespace

extern "C" {

const char* gdn_status_string(int status)
{
    switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_EINVAL: return "GDN_EINVAL: invalid argument";
    case GDN_EUNSUPPORTED: return "GDN_EUNSUPPORTED: unsupported size, dtype or alignment";
    case GDN_EWORKSPACE: return "GDN_EWORKSPACE: workspace too small";
    case GDN_ELAUNCH: return "GDN_ELAUNCH: kernel launch failed";
    default: return "GDN_UNKNOWN_STATUS";
    }
}

int gdn_conv1d_causal(const void* x, int64_t x_stride_b, int64_t x_stride_t, const void* w,
                      const void* bias, void* y, int64_t y_stride_b, int64_t y_stride_t,
                      const int32_t* cu_seqlens, int n_seqs, int B, int T, int C, int W, int silu,
                      int dtype, void* stream)
{
    if (B < 1 || T < 0 || C < 1) return GDN_EINVAL;
    if (!w || (T > 0 && (!x || !y))) return GDN_EINVAL;   // no tokens: x, y may be NULL
    if (silu != 0 && silu != 1) return GDN_EINVAL;
    if (T > 0 && x == y) return GDN_EINVAL;
    if (cu_seqlens && (B != 1 || n_seqs < 1)) return GDN_EINVAL;
    if (x_stride_t < C || y_stride_t < C) return GDN_EINVAL;
    if (B > 1 && (x_stride_b < (int64_t)T * x_stride_t || y_stride_b < (int64_t)T * y_stride_t))
        return GDN_EINVAL;
    if (!valid_dtype(dtype) || W != 4) return GDN_EUNSUPPORTED;
    const int vn = 16 / elem_size(dtype);
    if (C % vn != 0) return GDN_EUNSUPPORTED;
    if (!aligned16(x) || !aligned16(y) || !aligned16(w) || (bias && !aligned16(bias)) ||
        !stride16(x_stride_t, dtype) ||
        !stride16(y_stride_t, dtype) || (B > 1 && (!stride16(x_stride_b, dtype) || !stride16(y_stride_b, dtype))))
        return GDN_EUNSUPPORTED;
    if (T == 0) return GDN_OK;
    if ((int64_t)((T + 15) / 16 * B + 7) * ((C / vn + 255) / 256) > INT_MAX) return GDN_EUNSUPPORTED;
    return status_from(gdn::launch_conv1d(x, x_stride_b, x_stride_t, w, bias, y, y_stride_b,
                                          y_stride_t, cu_seqlens, n_seqs, B, T, C, silu,
                                          dtype == GDN_BF16, (hipStream_t)stream));
}

int gdn_gate_prepare(const void* a, int64_t a_stride_row, const void* b, int64_t b_stride_row,
                     const float* A_log, const float* dt_bias, float* g, float* beta, int R, int H,
                     int in_dtype, void* stream)
{
    if (!a || !b || !A_log || !dt_bias || !g || !beta) return GDN_EINVAL;
    if (R < 0 || H < 1) return GDN_EINVAL;
    if (a_stride_row < H || b_stride_row < H) return GDN_EINVAL;
    if ((const void*)g == (const void*)beta) return GDN_EINVAL;
    if (!valid_dtype(in_dtype)) return GDN_EUNSUPPORTED;
    if ((int64_t)R * H > (int64_t)INT_MAX * 256) return GDN_EUNSUPPORTED;
    if (R == 0) return GDN_OK;
    return status_from(gdn::launch_gate_prepare(a, a_stride_row, b, b_stride_row, A_log, dt_bias,
                                                g, beta, R, H, in_dtype == GDN_BF16,
                                                (hipStream_t)stream));
}

int gdn_tune_set(int knob, int value)
{
    switch (knob) {
    case GDN_TUNE_SCAN_TILES:
        if (value != 0 && value != 1 && value != 2 && value != 4) return GDN_EINVAL;
        break;
    case GDN_TUNE_CONV_RUN:
        if (value != 0 && value != 8 && value != 16 && value != 32) return GDN_EINVAL;
        break;
    case GDN_TUNE_CONV_THREADS:
        if (value != 0 && value != 64 && value != 128 && value != 256) return GDN_EINVAL;
        break;
    case GDN_TUNE_SCAN_FORM:
        if (value < 0 || value > 2) return GDN_EINVAL;
        break;
    default:
        return GDN_EINVAL;
    }
    gdn::tune_knob[knob] = value;
    return GDN_OK;
}

int gdn_tune_get(int knob)
{
    if (knob < 0 || knob >= gdn::kTuneKnobs) return -1;
    return gdn::tune_knob[knob];
}

size_t gdn_chunk_fwd_workspace_size(int B, int T, int H, int Hk, int K, int V, int n_seqs, int dtype)
{
    (void)Hk; (void)K; (void)V;
    if (B < 1 || T < 0 || H < 1 || n_seqs < 0) return 0;
    const bool packed = n_seqs > 0;
    return gdn::chunk_workspace_bytes(B, T, H, packed ? n_seqs : 0, packed, dtype == GDN_BF16);
}

// Checks shared by the chunked-forward entry points (prepare, scan and both).
static int check_chunk(const void* q, const void* k, int64_t qk_stride_t, const void* v,
                       int64_t v_stride_t, bool need_v, const float* g, const float* beta,
                       bool need_gates, const float* S0, const float* Sf, const void* o,
                       bool need_o, const int32_t* cu, int n_seqs, int B, int T, int H, int Hk,
                       int K, int V, int qk_l2norm, int dtype, const void* ws, size_t ws_bytes)
{
    if (B < 1 || T < 0 || H < 1 || Hk < 1 || H % Hk != 0) return GDN_EINVAL;
    const bool has_tokens = T > 0;   // with no tokens the token tensors may be NULL
    if (!ws) return GDN_EINVAL;
    if (has_tokens && (!q || !k || (need_v && !v) || (need_gates && (!g || !beta)) || (need_o && !o)))
        return GDN_EINVAL;
    if (qk_l2norm != 0 && qk_l2norm != 1) return GDN_EINVAL;
    if (cu && (B != 1 || n_seqs < 1)) return GDN_EINVAL;
    if ((int64_t)B * T > INT_MAX) return GDN_EINVAL;
    if (!valid_dtype(dtype) || !head_dim_ok(K) || !head_dim_ok(V)) return GDN_EUNSUPPORTED;
    if (qk_stride_t < (int64_t)Hk * K || (need_v && v_stride_t < (int64_t)H * V)) return GDN_EINVAL;
    if (need_o && has_tokens && (o == q || o == k || o == v)) return GDN_EINVAL;
    if (need_o && Sf && (const void*)Sf == o) return GDN_EINVAL;
    const int es = elem_size(dtype);
    if (!aligned16(q) || !aligned16(k) || (need_v && !aligned16(v)) || (need_o && !aligned16(o)) ||
        !stride16(qk_stride_t, dtype) || (need_v && !stride16(v_stride_t, dtype)) ||
        (S0 && !aligned16(S0)) || (Sf && !aligned16(Sf)) ||
        (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return GDN_EUNSUPPORTED;
    // the scan addresses a 64-token chunk with 32-bit byte offsets
    if (64 * qk_stride_t * es > INT_MAX || (need_v && 64 * v_stride_t * es > INT_MAX) ||
        (int64_t)64 * H * V > INT_MAX)
        return GDN_EUNSUPPORTED;
    const size_t need = gdn::chunk_workspace_bytes(B, T, H, cu ? n_seqs : 0, cu != nullptr,
                                                   dtype == GDN_BF16);
    if (ws_bytes < need) return GDN_EWORKSPACE;
    return GDN_OK;
}

int gdn_chunk_prepare(const void* q, const void* k, int64_t qk_stride_t, const float* g,
                      const float* beta, const int32_t* cu_seqlens, int n_seqs, int B, int T, int H,
                      int Hk, int K, float scale, int qk_l2norm, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream)
{
    const int st = check_chunk(q, k, qk_stride_t, nullptr, 0, false, g, beta, true, nullptr, nullptr,
                               nullptr, false, cu_seqlens, n_seqs, B, T, H, Hk, K, 64, qk_l2norm,
                               dtype, workspace, workspace_bytes);
    if (st != GDN_OK) return st;
    return status_from(gdn::launch_chunk_prepare(q, k, qk_stride_t, g, beta, cu_seqlens, n_seqs, B, T,
                                                 H, Hk, K, scale, qk_l2norm, dtype == GDN_BF16,
                                                 workspace, (hipStream_t)stream));
}

int gdn_chunk_scan(const void* q, const void* k, int64_t qk_stride_t, const void* v,
                   int64_t v_stride_t, const float* initial_state, float* final_state, void* o,
                   const int32_t* cu_seqlens, int n_seqs, int B, int T, int H, int Hk, int K, int V,
                   int dtype, const void* workspace, size_t workspace_bytes, void* stream)
{
    const int st = check_chunk(q, k, qk_stride_t, v, v_stride_t, true, nullptr, nullptr, false,
                               initial_state, final_state, o, true, cu_seqlens, n_seqs, B, T, H, Hk,
                               K, V, 0, dtype, workspace, workspace_bytes);
    if (st != GDN_OK) return st;
    return status_from(gdn::launch_chunk_scan(q, k, qk_stride_t, v, v_stride_t, initial_state,
                                              final_state, o, cu_seqlens, n_seqs, B, T, H, Hk, K, V,
                                              dtype == GDN_BF16, workspace, (hipStream_t)stream));
}

// ---------------------------------------------------------------- no-alloc variant
//
// gdn_chunk_fwd_noalloc: gdn_chunk_fwd with the workspace taken from a
// file-scope device array instead of a caller buffer. In host code the
// array's name is only a stand-in for the symbol; its device address, one per
// GPU, comes from hipGetSymbolAddress on the first call made with that device
// current, and only that address is ever handed to a kernel.
}  // extern "C"

namespace {

constexpr size_t kScratchBytes = (size_t)GDN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array (nullptr on failure).
void* device_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        scratch_ptr[dev] = p;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t gdn_chunk_fwd_noalloc_capacity(void) { return kScratchBytes; }

int gdn_chunk_fwd_noalloc(const void* q, const void* k, int64_t qk_stride_t, const void* v,
                          int64_t v_stride_t, const float* g, const float* beta,
                          const float* initial_state, float* final_state, void* o,
                          const int32_t* cu_seqlens, int n_seqs, int B, int T, int H, int Hk,
                          int K, int V, float scale, int qk_l2norm, int dtype, void* stream)
{
    // every check runs before the first HIP call, as for gdn_chunk_fwd; the
    // array's size stands in for the workspace (its address is not needed yet:
    // a placeholder with the array's alignment passes the workspace checks)
    const int st = check_chunk(q, k, qk_stride_t, v, v_stride_t, true, g, beta, true, initial_state,
                               final_state, o, true, cu_seqlens, n_seqs, B, T, H, Hk, K, V,
                               qk_l2norm, dtype, reinterpret_cast<const void*>(uintptr_t(256)),
                               kScratchBytes);
    if (st != GDN_OK) return st;
    void* ws = device_scratch();
    if (!ws) return GDN_ELAUNCH;
    hipError_t e = gdn::launch_chunk_prepare(q, k, qk_stride_t, g, beta, cu_seqlens, n_seqs, B, T, H,
                                             Hk, K, scale, qk_l2norm, dtype == GDN_BF16, ws,
                                             (hipStream_t)stream);
    if (e != hipSuccess) return GDN_ELAUNCH;
    return status_from(gdn::launch_chunk_scan(q, k, qk_stride_t, v, v_stride_t, initial_state,
                                              final_state, o, cu_seqlens, n_seqs, B, T, H, Hk, K, V,
                                              dtype == GDN_BF16, ws, (hipStream_t)stream));
}

int gdn_chunk_fwd(const void* q, const void* k, int64_t qk_stride_t, const void* v,
                  int64_t v_stride_t, const float* g, const float* beta,
                  const float* initial_state, float* final_state, void* o,
                  const int32_t* cu_seqlens, int n_seqs, int B, int T, int H, int Hk, int K, int V,
                  float scale, int qk_l2norm, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream)
{
    const int st = check_chunk(q, k, qk_stride_t, v, v_stride_t, true, g, beta, true, initial_state,
                               final_state, o, true, cu_seqlens, n_seqs, B, T, H, Hk, K, V,
                               qk_l2norm, dtype, workspace, workspace_bytes);
    if (st != GDN_OK) return st;
    hipError_t e = gdn::launch_chunk_prepare(q, k, qk_stride_t, g, beta, cu_seqlens, n_seqs, B, T, H,
                                             Hk, K, scale, qk_l2norm, dtype == GDN_BF16, workspace,
                                             (hipStream_t)stream);
    if (e != hipSuccess) return GDN_ELAUNCH;
    return status_from(gdn::launch_chunk_scan(q, k, qk_stride_t, v, v_stride_t, initial_state,
                                              final_state, o, cu_seqlens, n_seqs, B, T, H, Hk, K, V,
                                              dtype == GDN_BF16, workspace, (hipStream_t)stream));
}

size_t gdn_prefill_workspace_size(int B, int T, int H, int Hk, int K, int V, int n_seqs, int dtype)
{
    (void)V;
    if (B < 1 || T < 0 || H < 1 || Hk < 1 || n_seqs < 0) return 0;
    if (dtype != GDN_BF16 || !head_dim_ok(K)) return 0;
    const bool packed = n_seqs > 0;
    return gdn::prefill_workspace_bytes(B, T, H, Hk, K, packed ? n_seqs : 0, packed);
}

// Checks shared by the whole-prefill entry points (the two phases and both
// of them); need_x: x and conv_w are read, need_gates: a, b and the gate
// parameters, need_out: o and the states.
static int check_prefill(bool need_x, const void* x, int64_t x_stride_t, const void* conv_w,
                         const void* conv_bias, bool need_gates, const void* a,
                         int64_t a_stride_row, const void* b, int64_t b_stride_row,
                         const float* A_log, const float* dt_bias, bool need_out,
                         const float* S0, const float* Sf, const void* o, const int32_t* cu,
                         int n_seqs, int B, int T, int H, int Hk, int K, int V, int qk_l2norm,
                         int dtype, const void* ws, size_t ws_bytes)
{
    if (B < 1 || T < 0 || H < 1 || Hk < 1 || H % Hk != 0) return GDN_EINVAL;
    if (!ws || (need_x && !conv_w)) return GDN_EINVAL;
    if (need_gates && (!A_log || !dt_bias)) return GDN_EINVAL;
    if (T > 0 && ((need_x && !x) || (need_gates && (!a || !b)) || (need_out && !o)))
        return GDN_EINVAL;   // with no tokens the token tensors may be NULL
    if (qk_l2norm != 0 && qk_l2norm != 1) return GDN_EINVAL;
    if (cu && (B != 1 || n_seqs < 1)) return GDN_EINVAL;
    if ((int64_t)B * T > INT_MAX) return GDN_EINVAL;
    if (dtype != GDN_BF16 || !head_dim_ok(K) || !head_dim_ok(V)) return GDN_EUNSUPPORTED;
    const int64_t C = 2 * (int64_t)Hk * K + (int64_t)H * V;
    if (need_x && x_stride_t < C) return GDN_EINVAL;
    if (need_gates && (a_stride_row < H || b_stride_row < H)) return GDN_EINVAL;
    if (need_x && need_out && T > 0 && o == x) return GDN_EINVAL;
    if (need_out && Sf && (const void*)Sf == o) return GDN_EINVAL;
    if ((need_x && (!aligned16(x) || !aligned16(conv_w) || (conv_bias && !aligned16(conv_bias)) ||
                    !stride16(x_stride_t, dtype))) ||
        (need_out && !aligned16(o)) || (S0 && !aligned16(S0)) || (Sf && !aligned16(Sf)) ||
        (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return GDN_EUNSUPPORTED;
    // a 64-token chunk is addressed with 32-bit byte offsets; the q/k
    // convolution's grid is one-dimensional
    if ((need_x && 64 * x_stride_t * 2 > INT_MAX) || (int64_t)64 * H * V > INT_MAX ||
        (int64_t)64 * 2 * Hk * K * 2 > INT_MAX)
        return GDN_EUNSUPPORTED;
    if ((int64_t)((T + 15) / 16 * B + 7) * ((2 * Hk * K / 8 + 255) / 256) > INT_MAX)
        return GDN_EUNSUPPORTED;
    const size_t need = gdn::prefill_workspace_bytes(B, T, H, Hk, K, cu ? n_seqs : 0, cu != nullptr);
    if (ws_bytes < need) return GDN_EWORKSPACE;
    return GDN_OK;
}

int gdn_prefill_prepare(const void* x, int64_t x_stride_t, const void* conv_w,
                        const void* conv_bias, const void* a, int64_t a_stride_row, const void* b,
                        int64_t b_stride_row, const float* A_log, const float* dt_bias,
                        const int32_t* cu_seqlens, int n_seqs, int B, int T, int H, int Hk, int K,
                        int V, float scale, int qk_l2norm, int dtype, void* workspace,
                        size_t workspace_bytes, void* stream)
{
    const int st = check_prefill(true, x, x_stride_t, conv_w, conv_bias, true, a, a_stride_row, b,
                                 b_stride_row, A_log, dt_bias, false, nullptr, nullptr, nullptr,
                                 cu_seqlens, n_seqs, B, T, H, Hk, K, V, qk_l2norm, dtype, workspace,
                                 workspace_bytes);
    if (st != GDN_OK) return st;
    return status_from(gdn::launch_prefill_prepare(x, x_stride_t, conv_w, conv_bias, a, a_stride_row,
                                                   b, b_stride_row, A_log, dt_bias, cu_seqlens,
                                                   n_seqs, B, T, H, Hk, K, scale, qk_l2norm,
                                                   workspace, (hipStream_t)stream));
}

int gdn_prefill_scan(const void* x, int64_t x_stride_t, const void* conv_w, const void* conv_bias,
                     const float* initial_state, float* final_state, void* o,
                     const int32_t* cu_seqlens, int n_seqs, int B, int T, int H, int Hk, int K,
                     int V, int dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    const int st = check_prefill(true, x, x_stride_t, conv_w, conv_bias, false, nullptr, 0, nullptr,
                                 0, nullptr, nullptr, true, initial_state, final_state, o,
                                 cu_seqlens, n_seqs, B, T, H, Hk, K, V, 0, dtype, workspace,
                                 workspace_bytes);
    if (st != GDN_OK) return st;
    return status_from(gdn::launch_prefill_scan(x, x_stride_t, conv_w, conv_bias, initial_state,
                                                final_state, o, cu_seqlens, n_seqs, B, T, H, Hk, K,
                                                V, workspace, (hipStream_t)stream));
}

int gdn_prefill(const void* x, int64_t x_stride_t, const void* conv_w, const void* conv_bias,
                const void* a, int64_t a_stride_row, const void* b, int64_t b_stride_row,
                const float* A_log, const float* dt_bias, const float* initial_state,
                float* final_state, void* o, const int32_t* cu_seqlens, int n_seqs, int B, int T,
                int H, int Hk, int K, int V, float scale, int qk_l2norm, int dtype,
                void* workspace, size_t workspace_bytes, void* stream)
{
    int st = check_prefill(true, x, x_stride_t, conv_w, conv_bias, true, a, a_stride_row, b,
                           b_stride_row, A_log, dt_bias, true, initial_state, final_state, o,
                           cu_seqlens, n_seqs, B, T, H, Hk, K, V, qk_l2norm, dtype, workspace,
                           workspace_bytes);
    if (st != GDN_OK) return st;
    if (T > 0 && (o == a || o == b)) return GDN_EINVAL;
    hipError_t e = gdn::launch_prefill_prepare(x, x_stride_t, conv_w, conv_bias, a, a_stride_row, b,
                                               b_stride_row, A_log, dt_bias, cu_seqlens, n_seqs, B,
                                               T, H, Hk, K, scale, qk_l2norm, workspace,
                                               (hipStream_t)stream);
    if (e != hipSuccess) return GDN_ELAUNCH;
    return status_from(gdn::launch_prefill_scan(x, x_stride_t, conv_w, conv_bias, initial_state,
                                                final_state, o, cu_seqlens, n_seqs, B, T, H, Hk, K,
                                                V, workspace, (hipStream_t)stream));
}

int gdn_recurrent_decode(const void* x, int64_t x_stride_n, const void* ba, int64_t ba_stride_n,
                         const float* A_log, const float* dt_bias, float* state, void* o, int n,
                         int M, int H, int G, int P, int N, float scale, int qk_l2norm, int dtype,
                         void* stream)
{
    if (!x || !ba || !A_log || !dt_bias || !state || !o) return GDN_EINVAL;
    if (n < 0 || M < 1 || H < 1 || G < 1 || H % G != 0) return GDN_EINVAL;
    if (qk_l2norm != 0 && qk_l2norm != 1) return GDN_EINVAL;
    if ((const void*)o == (const void*)state) return GDN_EINVAL;
    if (!valid_dtype(dtype) || !head_dim_ok(P) || !head_dim_ok(N) || M > 4) return GDN_EUNSUPPORTED;
    const int64_t row = (int64_t)M * H * P + (int64_t)M * G * N + (int64_t)G * N;
    if (x_stride_n < row || ba_stride_n < (int64_t)M * H + H) return GDN_EINVAL;
    if (!aligned16(state)) return GDN_EUNSUPPORTED;
    if ((int64_t)n * H > INT_MAX) return GDN_EUNSUPPORTED;
    if (n == 0) return GDN_OK;
    return status_from(gdn::launch_recurrent_decode(x, x_stride_n, ba, ba_stride_n, A_log, dt_bias,
                                                    state, o, n, M, H, G, P, N, scale, qk_l2norm,
                                                    dtype == GDN_BF16, (hipStream_t)stream));
}

int gdn_decode_prepare(const void* x, int64_t x_stride_n, const void* ba, int64_t ba_stride_n,
                       const float* A_log, const float* dt_bias, void* q, void* k, void* v,
                       float* beta, float* g, int n, int M, int H, int G, int P, int N, int dtype,
                       void* stream)
{
    if (!x || !ba || !A_log || !dt_bias || !q || !k || !v || !beta || !g) return GDN_EINVAL;
    if (n < 0 || M < 1 || H < 1 || G < 1 || H % G != 0) return GDN_EINVAL;
    if (q == k || q == v || k == v || (const void*)beta == (const void*)g) return GDN_EINVAL;
    if (!valid_dtype(dtype) || !head_dim_ok(P) || !head_dim_ok(N)) return GDN_EUNSUPPORTED;
    const int64_t row = (int64_t)M * H * P + (int64_t)M * G * N + (int64_t)G * N;
    if (x_stride_n < row || ba_stride_n < (int64_t)M * H + H) return GDN_EINVAL;
    if (!aligned16(x) || !stride16(x_stride_n, dtype) || !aligned16(q) || !aligned16(k) ||
        !aligned16(v))
        return GDN_EUNSUPPORTED;
    // one thread per 16-byte output vector: the grid must fit 32 bits of blocks
    if ((int64_t)n * M * H * (P + 2 * N + 16) / 4 / 256 >= ((int64_t)1 << 31)) return GDN_EUNSUPPORTED;
    if (n == 0) return GDN_OK;
    return status_from(gdn::launch_decode_prepare(x, x_stride_n, ba, ba_stride_n, A_log, dt_bias, q,
                                                  k, v, beta, g, n, M, H, G, P, N,
                                                  dtype == GDN_BF16, (hipStream_t)stream));
}

int gdn_conv1d_update(const void* x, int64_t x_stride_n, void* conv_state, const int32_t* slot,
                      const void* w, const void* bias, void* y, int64_t y_stride_n, int n,
                      int n_slots, int C, int W, int silu, int dtype, void* stream)
{
    if (n < 0 || n_slots < 1 || C < 1) return GDN_EINVAL;
    if (!conv_state || !w || (n > 0 && (!x || !y || !slot))) return GDN_EINVAL;
    if (silu != 0 && silu != 1) return GDN_EINVAL;
    if (n > 0 && (x == y || y == conv_state || x == conv_state)) return GDN_EINVAL;
    if (x_stride_n < C || y_stride_n < C) return GDN_EINVAL;
    if (!valid_dtype(dtype) || W != 4) return GDN_EUNSUPPORTED;
    const int vn = 16 / elem_size(dtype);
    if (C % vn != 0) return GDN_EUNSUPPORTED;
    if (!aligned16(x) || !aligned16(y) || !aligned16(conv_state) || !aligned16(w) ||
        (bias && !aligned16(bias)) || !stride16(x_stride_n, dtype) || !stride16(y_stride_n, dtype))
        return GDN_EUNSUPPORTED;
    if ((C / vn + 255) / 256 > 65535) return GDN_EUNSUPPORTED;
    if (n == 0) return GDN_OK;
    return status_from(gdn::launch_conv1d_update(x, x_stride_n, conv_state, slot, w, bias, y,
                                                 y_stride_n, n, n_slots, C, silu,
                                                 dtype == GDN_BF16, (hipStream_t)stream));
}

int gdn_gdp_prefill_prepare(const void* x, int64_t x_stride_t, const void* ba, int64_t ba_stride_t,
                            const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
                            int n_seqs, int32_t* cu_out, void* q, void* k, void* v, float* g,
                            float* beta, int B, int T, int M, int H, int G, int P, int N,
                            int dtype, void* stream)
{
    if (B < 1 || T < 0 || M < 1 || H < 1 || G < 1 || H % G != 0) return GDN_EINVAL;
    if (!A_log || !dt_bias) return GDN_EINVAL;
    if (T > 0 && (!x || !ba || !q || !k || !v || !g || !beta)) return GDN_EINVAL;
    if (cu_seqlens && (B != 1 || n_seqs < 1)) return GDN_EINVAL;
    if (cu_out && !cu_seqlens) return GDN_EINVAL;
    if (T > 0 && (q == k || q == v || k == v || (const void*)g == (const void*)beta))
        return GDN_EINVAL;
    if (!valid_dtype(dtype) || !head_dim_ok(P) || !head_dim_ok(N)) return GDN_EUNSUPPORTED;
    const int64_t row = (int64_t)M * H * P + (int64_t)M * G * N + (int64_t)G * N;
    if (x_stride_t < row || ba_stride_t < (int64_t)M * H + H) return GDN_EINVAL;
    if (!aligned16(x) || !stride16(x_stride_t, dtype) || !aligned16(q) || !aligned16(k) ||
        !aligned16(v))
        return GDN_EUNSUPPORTED;
    const int64_t rows = (int64_t)B * T;
    if (rows * M > INT_MAX) return GDN_EUNSUPPORTED;
    if (T == 0) return GDN_OK;
    return status_from(gdn::launch_gdp_prefill_prepare(x, x_stride_t, ba, ba_stride_t, A_log,
                                                       dt_bias, cu_seqlens, n_seqs, cu_out, q, k,
                                                       v, g, beta, rows, M, H, G, P, N,
                                                       dtype == GDN_BF16, (hipStream_t)stream));
}

}  // extern "C"
