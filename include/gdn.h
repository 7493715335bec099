/*
 * gdn.h -- C ABI of the gated-delta-rule forward library for MI355X (gfx950).
 *
 * Four operations make the hot path of a Gated DeltaNet / Gated DeltaProduct
 * mixer: the short causal convolution, the gate preparation, the chunked
 * prefill forward and the one-token recurrent decode. Around them: the
 * decode-step short-conv update, the decode preparation exported on its own,
 * and the interleave that runs a Gated DeltaProduct prefill through the
 * chunked forward. Sources (web pages, cited by title and section):
 *   [ZZ]  "ZzCompute", PyTorch Helion Hackathon gallery entry, items 1-4.
 *   [GDP] Megatron-Core API docs, "core.ssm.ops.gdp.decode_prepare".
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers (HIP global memory) unless stated.
 *    `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - Strides are in elements of the tensor's own dtype.
 *  - Ownership: the caller owns every buffer. The library never allocates or
 *    frees memory; intermediates go to the caller's workspace.
 *  - Asynchrony: every call only enqueues kernels on `stream`; it performs no
 *    host synchronisation and no device-to-host read, so it may be captured
 *    in a HIP graph.
 *  - Errors: every call returns a gdn_status. All argument validation happens
 *    before the first HIP call, so a rejected call has no effect. A kernel
 *    launch failure is reported as GDN_ELAUNCH (from hipGetLastError).
 *    NaN/Inf inputs propagate; they are not trapped.
 *  - Determinism: no atomics; every output element has exactly one writer, so
 *    repeated calls on the same inputs give bitwise identical results.
 *  - Alignment: every device base pointer must be 16-byte aligned, and every
 *    row stride a multiple of 16 bytes, else GDN_EUNSUPPORTED.
 *  - bf16 results are rounded to nearest-even from fp32 accumulators.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_EINVAL = 1,        /* null required pointer, bad size, bad stride, aliasing */
    GDN_EUNSUPPORTED = 2,  /* valid but not implemented: head dims, W, alignment, dtype */
    GDN_EWORKSPACE = 3,    /* workspace smaller than the size query returns */
    GDN_ELAUNCH = 4        /* a kernel launch failed (no device, bad stream, ...) */
} gdn_status;

typedef enum gdn_dtype {
    GDN_FP32 = 0,
    GDN_BF16 = 1
} gdn_dtype;

/* Static, NUL-terminated name of a status code ("GDN_OK", ...). Never NULL. */
const char* gdn_status_string(int status);

/* ------------------------------------------------------------------------
 * gdn_tune_set / gdn_tune_get -- launch-configuration knobs, for the offline
 * sweep that stands in for the pages' autotuning ([ZZ] item 1: the conv's
 * block sizes and grouping are autotuned; item 4: one configuration serves
 * every shape). A knob changes only how the work is scheduled, never the
 * arithmetic: every setting gives the same results, bit for bit. 0 =
 * automatic (the default). The knobs are process-wide host state read when
 * an entry point launches; set them between calls, from one thread.
 *   GDN_TUNE_SCAN_TILES    column tiles of 16 value columns per workgroup of
 *                          the state scan (gdn_chunk_fwd, gdn_chunk_scan,
 *                          gdn_prefill, gdn_prefill_scan): 1 or 2 for bf16, 1
 *                          or 4 for fp32; a value that does not fit the
 *                          call's dtype or V means automatic.
 *   GDN_TUNE_CONV_RUN      tokens per thread of gdn_conv1d_causal: 8, 16 or
 *                          32.
 *   GDN_TUNE_CONV_THREADS  threads per workgroup of gdn_conv1d_causal: 64,
 *                          128 or 256.
 *   GDN_TUNE_SCAN_FORM     workgroup form of the bf16 state scan of
 *                          gdn_chunk_fwd, gdn_chunk_scan, gdn_prefill and
 *                          gdn_prefill_scan: 1 = one workgroup per group of
 *                          16 * GDN_TUNE_SCAN_TILES value columns of a
 *                          (sequence, head) unit, waves split by role; 2 = one
 *                          workgroup per unit over all its value columns,
 *                          compute waves each running the whole chunk step for
 *                          16 * GDN_TUNE_SCAN_TILES of them (2: four waves and
 *                          a copy wave, the default; 1: eight waves; the
 *                          whole-prefill scan always has four compute waves
 *                          and four waves that copy and convolve), packed
 *                          sequences longest first. Automatic: 2 from 512
 *                          units on, else 1.
 * gdn_tune_set returns GDN_EINVAL for an unknown knob or value (nothing
 * changes); gdn_tune_get returns the knob's value, or -1 for an unknown knob.
 * ---------------------------------------------------------------------- */
enum {
    GDN_TUNE_SCAN_TILES = 0,
    GDN_TUNE_CONV_RUN = 1,
    GDN_TUNE_CONV_THREADS = 2,
    GDN_TUNE_SCAN_FORM = 3
};
int gdn_tune_set(int knob, int value);
int gdn_tune_get(int knob);

/* ------------------------------------------------------------------------
 * gdn_conv1d_causal -- [ZZ] item 1 "Causal Conv1d".
 * Depthwise causal convolution of width W (only W == 4 is implemented; the
 * width is fixed at compile time so the tap loop unrolls), each channel with
 * its own past, optionally followed by SiLU z/(1+exp(-z)):
 *     y[b,t,c] = act( sum_{j<W} w[c,j] * x[b, t-(W-1)+j, c] (+ bias[c]) )
 * A tap that falls before the start of the token's own sequence reads zero
 * (masked load; nothing is padded on the host), so nothing leaks across a
 * batch row or across a packed-sequence boundary.
 *   x        [B, T, C] in `dtype`, channel dim contiguous; element (b,t,c) at
 *            x + b*x_stride_b + t*x_stride_t + c.
 *   w        [C, W] in `dtype`, contiguous, 16-byte aligned (w[c][W-1] multiplies x_t).
 *   bias     [C] in `dtype`, 16-byte aligned, or NULL for none.
 *   y        [B, T, C] in `dtype`, same addressing with y strides. y must not
 *            overlap x (GDN_EINVAL when the base pointers are equal).
 *   cu_seqlens  int32 [n_seqs + 1] device array of packed-sequence offsets,
 *            or NULL. With it, B must be 1 and T the packed length; it must be
 *            non-decreasing with cu[0] = 0 and cu[n_seqs] = T (not checked:
 *            checking would need a device read).
 *   silu     0 = identity, 1 = SiLU.
 *   dtype    GDN_FP32 or GDN_BF16 (fp32 accumulation either way).
 *   C must be a multiple of 8 (bf16) or 4 (fp32).
 * ---------------------------------------------------------------------- */
int gdn_conv1d_causal(const void* x, int64_t x_stride_b, int64_t x_stride_t,
                      const void* w, const void* bias,
                      void* y, int64_t y_stride_b, int64_t y_stride_t,
                      const int32_t* cu_seqlens, int n_seqs,
                      int B, int T, int C, int W, int silu, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * gdn_gate_prepare -- [GDP] module introduction and "softplus" entry.
 *     beta = sigmoid(b) = 1 / (1 + exp(-b))
 *     g    = -exp(A_log[h]) * softplus(a + dt_bias[h]),
 *     softplus(x) = x if x > 20 else log1p(exp(x))
 * computed in fp32 with IEEE division.
 *   a, b     [R, H] rows in `in_dtype`; row r at a + r*a_stride_row (the last
 *            dim contiguous; rows may be a strided view).
 *   A_log, dt_bias  [H] fp32.
 *   g, beta  [R, H] fp32, contiguous outputs (alpha = exp(g) is the decay).
 * ---------------------------------------------------------------------- */
int gdn_gate_prepare(const void* a, int64_t a_stride_row, const void* b, int64_t b_stride_row,
                     const float* A_log, const float* dt_bias, float* g, float* beta,
                     int R, int H, int in_dtype, void* stream);

/* ------------------------------------------------------------------------
 * gdn_chunk_fwd -- [ZZ] items 2-4: the gated delta rule evaluated in
 * 64-timestep chunks (WY recompute per chunk, sequential inter-chunk K x V
 * state scan, per-chunk output). Per sequence and value head, with state
 * h (K x V, fp32), the result equals the timestep recurrence
 *     h_t = exp(g_t) h_{t-1} + beta_t k_t (v_t - exp(g_t) h_{t-1}^T k_t)^T
 *     o_t = scale * h_t^T q_t
 * (h = S^T for S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T).
 *   q, k     [B*T, Hk, K] token rows in `dtype`: element (token, head, d) at
 *            q + token*qk_stride_t + head*K + d (a batch row b starts at token
 *            b*T, i.e. rows of all batches are evenly strided). Typically
 *            zero-copy views of the conv1d output (token stride = C).
 *   v        [B*T, H, V] token rows in `dtype`, token stride v_stride_t.
 *   g, beta  [B*T, H] fp32 contiguous (the gdn_gate_prepare outputs).
 *   initial_state  [N, H, K, V] fp32 contiguous, or NULL for zero.
 *   final_state    [N, H, K, V] fp32 contiguous output, or NULL to skip.
 *            N = n_seqs with cu_seqlens, else B.
 *   o        [B*T, H, V] in `dtype`, contiguous output.
 *   cu_seqlens  int32 [n_seqs + 1] device offsets of packed sequences or
 *            NULL (same contract as conv1d; B must be 1). The state restarts
 *            at every sequence start; the last chunk of a sequence may be
 *            partial.
 *   H value heads share Hk q/k heads: value head h reads q/k head
 *            h / (H / Hk) (H % Hk == 0).
 *   K, V     head dims; each of 64 or 128.
 *   qk_l2norm  1: q and k are normalised per token and head as
 *            x / sqrt(sum x^2 + 1e-6) before use; 0: used as given.
 *   dtype    GDN_BF16 (bf16 MFMA operands, fp32 accumulation and state) or
 *            GDN_FP32 (fp32 MFMA operands throughout).
 *   workspace  device scratch of at least gdn_chunk_fwd_workspace_size(...)
 *            bytes, 256-byte aligned; contents on entry do not matter.
 *   Token strides times 64 rows must stay below 2^31 bytes (the scan
 *   addresses a chunk with 32-bit offsets), else GDN_EUNSUPPORTED.
 * ---------------------------------------------------------------------- */
size_t gdn_chunk_fwd_workspace_size(int B, int T, int H, int Hk, int K, int V,
                                    int n_seqs, int dtype);

int gdn_chunk_fwd(const void* q, const void* k, int64_t qk_stride_t,
                  const void* v, int64_t v_stride_t,
                  const float* g, const float* beta,
                  const float* initial_state, float* final_state,
                  void* o,
                  const int32_t* cu_seqlens, int n_seqs,
                  int B, int T, int H, int Hk, int K, int V,
                  float scale, int qk_l2norm, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gdn_chunk_fwd_noalloc -- gdn_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that forbid
 * hipMalloc, harnesses without an allocator): the same arguments minus the
 * workspace, the same kernels and results, bit for bit. The workspace is a
 * fixed device array inside the library, GDN_NOALLOC_SCRATCH_BYTES bytes
 * (64 MiB) on every GPU the library runs on, held until the process ends.
 *   - A call whose workspace (gdn_chunk_fwd_workspace_size) exceeds that
 *     size returns GDN_EWORKSPACE before any HIP call; the prefill workload
 *     (B=4, T=4096, H=16) fits, with room to spare.
 *   - The call itself allocates nothing: no hipMalloc, no hipFree, no
 *     allocating library routine. The first call on a device looks up the
 *     array's address there (hipGetSymbolAddress) and keeps it.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero: each call writes
 *     everything it reads). Calls that overlap on one GPU -- on different
 *     streams, or from several host threads without ordering -- race on it;
 *     the caller must order them (one stream, or events).
 * gdn_chunk_fwd_noalloc_capacity returns the array's size in bytes.
 * ---------------------------------------------------------------------- */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)

size_t gdn_chunk_fwd_noalloc_capacity(void);

int gdn_chunk_fwd_noalloc(const void* q, const void* k, int64_t qk_stride_t,
                          const void* v, int64_t v_stride_t,
                          const float* g, const float* beta,
                          const float* initial_state, float* final_state,
                          void* o,
                          const int32_t* cu_seqlens, int n_seqs,
                          int B, int T, int H, int Hk, int K, int V,
                          float scale, int qk_l2norm, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * gdn_chunk_prepare / gdn_chunk_scan -- the two phases of gdn_chunk_fwd,
 * exposed separately (same arguments, same workspace) so that each can be
 * launched and timed on its own; gdn_chunk_fwd(...) is exactly
 * gdn_chunk_prepare(...) followed by gdn_chunk_scan(...) on one stream.
 *   gdn_chunk_prepare  [ZZ] item 4 (WY recompute): for every 64-token chunk
 *            and value head, in parallel, the cumulative log-decay, the
 *            inverse (I + A)^-1 diag(beta) of the chunk's unit-lower-triangular
 *            system, the gated intra-chunk attention (q k^T o decay) and the
 *            per-row scale factors, written to `workspace`.
 *   gdn_chunk_scan     [ZZ] items 2-3: the sequential inter-chunk state scan
 *            and the per-chunk outputs, reading the records gdn_chunk_prepare
 *            left in `workspace` (which must be the result of a prepare call
 *            with the same q, k, g, beta, cu_seqlens, sizes, scale, qk_l2norm
 *            and dtype; the workspace is otherwise unchecked).
 * Error codes as for gdn_chunk_fwd (the prepare call checks V as if 64).
 * ---------------------------------------------------------------------- */
int gdn_chunk_prepare(const void* q, const void* k, int64_t qk_stride_t,
                      const float* g, const float* beta,
                      const int32_t* cu_seqlens, int n_seqs,
                      int B, int T, int H, int Hk, int K,
                      float scale, int qk_l2norm, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

int gdn_chunk_scan(const void* q, const void* k, int64_t qk_stride_t,
                   const void* v, int64_t v_stride_t,
                   const float* initial_state, float* final_state, void* o,
                   const int32_t* cu_seqlens, int n_seqs,
                   int B, int T, int H, int Hk, int K, int V, int dtype,
                   const void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gdn_prefill -- the whole prefill of a gated delta rule layer from the
 * projections: [ZZ] item 1 (causal conv1d, W = 4, + SiLU over the q | k | v
 * channels), the gates of [GDP] (module introduction and "softplus" entry)
 * and [ZZ] items 2-4 (the chunked forward). The result is exactly that of
 *     gdn_conv1d_causal(x, conv_w, conv_bias, silu = 1) -> y = q | k | v,
 *     gdn_gate_prepare(a, b, A_log, dt_bias)           -> g, beta,
 *     gdn_chunk_fwd(q, k, v, g, beta, ...)              -> o, final_state
 * on the same bf16 inputs, bit for bit (the same formulas, rounding points
 * and accumulation order), in two kernel launches instead of four: the
 * per-chunk solve convolving the q and k rows and forming the gates itself,
 * and the scan convolving the value rows as it reads them. y, g and beta are
 * never written (the convolved q and k rows live in the workspace).
 *   x        [B*T, C] bf16 token rows before the convolution, C = 2*Hk*K +
 *            H*V channels laid out q [Hk][K] | k [Hk][K] | v [H][V]; row t at
 *            x + t*x_stride_t (batch row b starts at token b*T).
 *   conv_w   [C, 4] bf16 contiguous taps (conv_w[c][3] multiplies x_t);
 *   conv_bias  [C] bf16 or NULL.
 *   a, b     [B*T, H] bf16 gate inputs; row t at a + t*a_stride_row.
 *   A_log, dt_bias  [H] fp32.
 *   initial_state, final_state, o, cu_seqlens, n_seqs, B, T, H, Hk, K, V,
 *   scale, qk_l2norm: as for gdn_chunk_fwd (final_state may be NULL; it may
 *            equal initial_state for an in-place update).
 *   dtype    GDN_BF16 only (GDN_EUNSUPPORTED otherwise).
 *   workspace  device scratch of at least gdn_prefill_workspace_size(...)
 *            bytes, 256-byte aligned; contents on entry do not matter.
 * x, conv_w, conv_bias and o must be 16-byte aligned and x_stride_t*2 a
 * multiple of 16 (else GDN_EUNSUPPORTED); o must not be x, a or b
 * (GDN_EINVAL). gdn_prefill_workspace_size returns 0 for a dtype other than
 * GDN_BF16, a head dim other than 64 or 128, or invalid sizes.
 *
 * gdn_prefill_prepare / gdn_prefill_scan -- the two phases of gdn_prefill
 * (the same arguments where they take them, the same workspace), exposed so
 * that each kernel can be launched and timed on its own; gdn_prefill(...) is
 * exactly the two in this order on one stream:
 *   prepare  the q and k channels of x convolved (+ SiLU) into `workspace`,
 *            the gates formed from a, b, A_log, dt_bias, and the per-chunk
 *            solve of gdn_chunk_prepare on those rows, into `workspace`;
 *   scan     the state scan and outputs of gdn_chunk_scan, the value rows of x
 *            convolved as they are read.
 * The scan reads what the prepare call left in `workspace`, which must come
 * from a call with the same x, conv_w, conv_bias, a, b, gate parameters,
 * cu_seqlens, sizes, scale and qk_l2norm (the workspace is otherwise
 * unchecked).
 * ---------------------------------------------------------------------- */
size_t gdn_prefill_workspace_size(int B, int T, int H, int Hk, int K, int V, int n_seqs,
                                  int dtype);

int gdn_prefill(const void* x, int64_t x_stride_t, const void* conv_w, const void* conv_bias,
                const void* a, int64_t a_stride_row, const void* b, int64_t b_stride_row,
                const float* A_log, const float* dt_bias,
                const float* initial_state, float* final_state, void* o,
                const int32_t* cu_seqlens, int n_seqs,
                int B, int T, int H, int Hk, int K, int V,
                float scale, int qk_l2norm, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

int gdn_prefill_prepare(const void* x, int64_t x_stride_t, const void* conv_w,
                        const void* conv_bias, const void* a, int64_t a_stride_row,
                        const void* b, int64_t b_stride_row,
                        const float* A_log, const float* dt_bias,
                        const int32_t* cu_seqlens, int n_seqs,
                        int B, int T, int H, int Hk, int K, int V,
                        float scale, int qk_l2norm, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

int gdn_prefill_scan(const void* x, int64_t x_stride_t, const void* conv_w, const void* conv_bias,
                     const float* initial_state, float* final_state, void* o,
                     const int32_t* cu_seqlens, int n_seqs,
                     int B, int T, int H, int Hk, int K, int V, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gdn_recurrent_decode -- [GDP] "gdp_decode_prepare" fused with the
 * recurrent update it feeds: one decode token for n requests of a Gated
 * DeltaProduct layer with M Householder copies.
 *   x        [n, M*H*P + M*G*N + G*N] in `dtype`: the post-conv row, value |
 *            key | query, laid out v [M][H][P], k [M][G][N], q [G][N]; row r
 *            at x + r*x_stride_n.
 *   ba       [n, M*H + H] in `dtype`: b [M][H] then a [H]; row r at
 *            ba + r*ba_stride_n (may be a strided view).
 *   A_log, dt_bias  [H] fp32.
 *   state    [n, H, N, P] fp32 (K x V orientation: N = key dim rows, P =
 *            value dim columns), read and updated IN PLACE.
 *   o        [n, H, P] in `dtype`, contiguous output.
 * Per request and value head h (q/k group h / (H/G), H % G == 0), the M
 * copies run as an M-step sequence: copy 0 carries the decay
 * exp(-exp(A_log)*softplus(a+dt_bias)), later copies none; every copy m
 * writes with beta_m = sigmoid(b_m) and key k_m; only the last copy carries
 * the query, and o is that copy's output scale * h^T q.
 *   P, N     64 or 128.  M in 1..4.
 *   qk_l2norm  as for gdn_chunk_fwd.
 * ---------------------------------------------------------------------- */
int gdn_recurrent_decode(const void* x, int64_t x_stride_n,
                         const void* ba, int64_t ba_stride_n,
                         const float* A_log, const float* dt_bias,
                         float* state, void* o,
                         int n, int M, int H, int G, int P, int N,
                         float scale, int qk_l2norm, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * gdn_decode_prepare -- [GDP] "gdp_decode_prepare": the five tensors one
 * decode step's recurrent update consumes, from the post-conv row and the
 * ba slice (the preparation gdn_recurrent_decode performs internally,
 * exported on its own).
 *   x, ba, A_log, dt_bias   as for gdn_recurrent_decode.
 *   q, k     [n, M, H, N] in `dtype`, contiguous: q is the query of group
 *            h / (H/G) on copy M-1 and zero on earlier copies; k is copy m's
 *            key of group h / (H/G). Plain copies: bit-identical to x.
 *   v        [n, M, H, P] in `dtype`, contiguous: copy m's value of head h.
 *   beta, g  [n, M, H] fp32, contiguous: beta = sigmoid(b[m][h]); g =
 *            -exp(A_log[h]) * softplus(a[h] + dt_bias[h]) on copy 0 and 0 on
 *            later copies (softplus the identity above 20). The same fp32
 *            formulas as gdn_gate_prepare and gdn_recurrent_decode.
 *   P, N     64 or 128. H % G == 0.
 * Errors: NULL pointer, n < 0, M < 1, H % G != 0, short strides, outputs
 * sharing memory -> GDN_EINVAL; P, N, dtype, alignment (x, its row stride,
 * q, k, v) -> GDN_EUNSUPPORTED.
 * ---------------------------------------------------------------------- */
int gdn_decode_prepare(const void* x, int64_t x_stride_n,
                       const void* ba, int64_t ba_stride_n,
                       const float* A_log, const float* dt_bias,
                       void* q, void* k, void* v, float* beta, float* g,
                       int n, int M, int H, int G, int P, int N, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * gdn_conv1d_update -- the short-conv update of one decode token per
 * request, the step [GDP] places before the decode preparation, with its
 * padding rule (a -1 slot zeroes the request's output).
 *   x          [n, C] in `dtype`: this token's pre-conv row of each request
 *              (row r at x + r*x_stride_n).
 *   conv_state [n_slots, W-1, C] in `dtype`, contiguous, updated IN PLACE:
 *              row j of a slot holds the input W-1-j tokens back (row W-2 is
 *              the latest), zero for a fresh sequence.
 *   slot       [n] int32 (device): the conv_state slot of each request; a
 *              value outside [0, n_slots) (-1 marks padding) zeroes that
 *              request's output row and leaves every slot untouched. Two
 *              requests naming the same slot race (unchecked: device data).
 *   w, bias    [C, W] and [C] (bias may be NULL), as for gdn_conv1d_causal.
 *   y          [n, C] in `dtype` (row r at y + r*y_stride_n):
 *              act(sum_{j<W-1} w[c][j] state[j][c] + w[c][W-1] x[c] + bias[c]),
 *              act = SiLU if silu else identity; then the slot's rows move one
 *              token on and take x as the latest. The arithmetic is that of
 *              gdn_conv1d_causal, so a sequence fed one token at a time from a
 *              zero state gives bit-identical outputs.
 *   W        4.
 * Errors: n < 0, n_slots < 1, C < 1, NULL pointer, silu not 0/1, short
 * strides, x / y / conv_state the same buffer -> GDN_EINVAL; W, dtype, C not
 * a multiple of 16 bytes, alignment -> GDN_EUNSUPPORTED.
 * ---------------------------------------------------------------------- */
int gdn_conv1d_update(const void* x, int64_t x_stride_n, void* conv_state,
                      const int32_t* slot, const void* w, const void* bias,
                      void* y, int64_t y_stride_n,
                      int n, int n_slots, int C, int W, int silu, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * gdn_gdp_prefill_prepare -- a Gated DeltaProduct prefill as a gated delta
 * rule over M*T positions: [GDP]'s interleave of the Householder copies
 * (query on the last copy, the decay on the first) applied to every token of
 * a prefill, so that gdn_chunk_fwd runs the layer unchanged.
 *   x        [B*T, M*H*P + M*G*N + G*N] in `dtype`: post-conv rows, value |
 *            key | query as for gdn_recurrent_decode; token t of batch b at
 *            x + (b*T + t)*x_stride_t (packed: B = 1, sequences by cu_seqlens).
 *   ba       [B*T, M*H + H]: b [M][H] then a [H], row stride ba_stride_t.
 *   A_log, dt_bias  [H] fp32.
 *   q, k     [B, M*T, G, N] in `dtype`, contiguous; v [B, M*T, H, P]; g, beta
 *            [B, M*T, H] fp32. Row t*M + m (within its batch) is copy m of
 *            token t: k, v, beta of copy m; q of token t on m = M-1, else
 *            zero; g of token t on m = 0, else zero.
 *   cu_seqlens, n_seqs  packed sequences of x (B == 1) or NULL; cu_out
 *            (optional, n_seqs + 1 int32, device) receives M * cu_seqlens,
 *            the offsets of the interleaved sequence.
 * Then gdn_chunk_fwd(q, k, G*N, v, H*P, g, beta, ..., T' = M*T, H, Hk = G,
 * K = N, V = P, cu_seqlens = cu_out) gives the layer: token t's output is
 * row t*M + M-1 of o, and the final state is the layer's.
 * Errors: bad sizes, H % G != 0, NULL pointers with T > 0, cu_seqlens with
 * B != 1, cu_out without cu_seqlens, outputs sharing memory, short strides
 * -> GDN_EINVAL; P, N, dtype, alignment -> GDN_EUNSUPPORTED.
 * ---------------------------------------------------------------------- */
int gdn_gdp_prefill_prepare(const void* x, int64_t x_stride_t,
                            const void* ba, int64_t ba_stride_t,
                            const float* A_log, const float* dt_bias,
                            const int32_t* cu_seqlens, int n_seqs, int32_t* cu_out,
                            void* q, void* k, void* v, float* g, float* beta,
                            int B, int T, int M, int H, int G, int P, int N,
                            int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
