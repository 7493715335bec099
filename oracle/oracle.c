/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the gated-delta-rule forward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path loads this file or
 * the library built from it: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg do. It shares no code, header, table or helper
 * with the HIP library; the two meet only in the seeded input generators.
 *
 * Every function is the plain definition of what the method computes, written
 * out one timestep / one output element at a time, in double precision, with
 * no blocking, fusion or reordering beyond what the definition states.
 * Parallelism is an OpenMP loop over independent units only (batch x time x
 * channel for the conv; sequence x head for the recurrence; request x head for
 * the decode), so every unit's arithmetic is the sequential definition.
 *
 * Sources (web pages; cited by title and section):
 *  [ZZ]  "ZzCompute", PyTorch Helion Hackathon gallery entry:
 *        item 1 "Causal Conv1d", item 2 "Gated DeltaNet Chunk Forward H",
 *        item 3 "Gated DeltaNet Chunk Forward O", item 4 "Recompute W/U".
 *  [GDP] Megatron-Core API docs, "core.ssm.ops.gdp.decode_prepare":
 *        the module introduction, the "softplus" entry, the
 *        "gdp_decode_prepare_kernel" entry and the "gdp_decode_prepare"
 *        Parameters / Returns lists.
 *
 * The per-timestep recurrence (the gated delta rule that the chunk kernels of
 * [ZZ] items 2-4 evaluate in chunked form) is, with state S of shape V x K:
 *     S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = scale * S_t q_t,            alpha_t = exp(g_t).
 * At the boundary the state is stored transposed, as the K x V state that
 * [ZZ] item 2 names: state[k][v] = S[v][k].
 *
 * Readings of points the pages leave open (each also listed in the design
 * notes of the repository):
 *  - L2 normalisation of q and k: x / sqrt(sum x^2 + 1e-6), per token and head.
 *  - Conv tap order: w[c][W-1] multiplies x_t, w[c][W-1-j] multiplies x_{t-j}.
 *  - Conv input is zero before the start of each token's own sequence.
 *  - softplus(x) = x when x > 20 (strictly), else log1p(exp(x)).
 *  - Decode row order v | k | q with v [M][H][P], k [M][G][N], q [G][N];
 *    ba row = b [M][H] then a [H]; value head h reads q/k group h / (H/G).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_L2_EPS 1e-6

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- conv1d */

/* [ZZ] item 1: depthwise causal convolution, each channel convolved with its
 * own past only; out-of-range taps read zero (masked loads, no host padding).
 * x, y: [B, T, C] contiguous. w: [C, W]. bias: [C] or NULL.
 * cu_seqlens (int32 [n_seqs + 1], B == 1) marks packed sequences; a tap before
 * the start of the token's own sequence reads zero, so nothing leaks across a
 * sequence boundary. silu != 0 applies z / (1 + exp(-z)). */
void oracle_conv1d_causal(const double* x, const double* w, const double* bias,
                          double* y, const int32_t* cu_seqlens, int n_seqs,
                          int B, int T, int C, int W, int silu)
{
    long BT = (long)B * T;
#pragma omp parallel for schedule(static)
    for (long bt = 0; bt < BT; ++bt) {
        long t = bt % T;
        long start = 0; /* first token of this token's sequence (local t) */
        if (cu_seqlens) {
            for (int i = 0; i < n_seqs; ++i)
                if (cu_seqlens[i] <= t && t < cu_seqlens[i + 1]) start = cu_seqlens[i];
        }
        for (int c = 0; c < C; ++c) {
            double acc = bias ? bias[c] : 0.0;
            for (int j = 0; j < W; ++j) {
                long tau = t - (W - 1) + j;
                if (tau < start) continue;
                acc += w[(long)c * W + j] * x[(bt - t + tau) * C + c];
            }
            y[bt * C + c] = silu ? acc / (1.0 + exp(-acc)) : acc;
        }
    }
}

/* ----------------------------------------------------------------- gates */

/* [GDP] "softplus": log1p(exp(x)), the identity once x exceeds 20 (torch's
 * threshold rule at beta = 1). */
static double oracle_softplus(double x)
{
    return x > 20.0 ? x : log1p(exp(x));
}

/* [GDP] module introduction: beta = sigmoid(b),
 * g = -exp(A_log) * softplus(a + dt_bias), per row and head.
 * a, b, g, beta: [R, H] contiguous. A_log, dt_bias: [H]. */
void oracle_gate_prepare(const double* a, const double* b, const double* A_log,
                         const double* dt_bias, double* g, double* beta, int R, int H)
{
    long n = (long)R * H;
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; ++i) {
        int h = (int)(i % H);
        beta[i] = 1.0 / (1.0 + exp(-b[i]));
        g[i] = -exp(A_log[h]) * oracle_softplus(a[i] + dt_bias[h]);
    }
}

/* ------------------------------------------------------------ recurrence */

static void l2_normalise(const double* src, double* dst, int n)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += src[i] * src[i];
    double inv = 1.0 / sqrt(ss + ORACLE_L2_EPS);
    for (int i = 0; i < n; ++i) dst[i] = src[i] * inv;
}

/* One timestep of the gated delta rule on S (V x K, row-major):
 * S <- alpha * S (I - beta k k^T) + beta v k^T.  sk is scratch of length V. */
static void gdr_step(double* S, int K, int V, const double* k, const double* v,
                     double alpha, double beta, double* sk)
{
    for (int i = 0; i < V; ++i) {
        double acc = 0.0;
        for (int j = 0; j < K; ++j) acc += S[(long)i * K + j] * k[j];
        sk[i] = acc; /* S k */
    }
    for (int i = 0; i < V; ++i)
        for (int j = 0; j < K; ++j) {
            double s = S[(long)i * K + j];
            S[(long)i * K + j] = alpha * (s - beta * sk[i] * k[j]) + beta * v[i] * k[j];
        }
}

/* o = scale * S q */
static void gdr_readout(const double* S, int K, int V, const double* q, double scale, double* o)
{
    for (int i = 0; i < V; ++i) {
        double acc = 0.0;
        for (int j = 0; j < K; ++j) acc += S[(long)i * K + j] * q[j];
        o[i] = scale * acc;
    }
}

/* The gated delta rule over whole sequences, one timestep at a time
 * ([ZZ] items 2-4 compute the same result in 64-step chunks).
 *   q, k : [B*T, Hk, K]   (token rows)
 *   v    : [B*T, H, V]
 *   g, beta : [B*T, H]    (log-decay and write strength per token and head)
 *   S0   : [N, H, K, V] or NULL (zero), N = n_seqs if cu_seqlens else B
 *   o    : [B*T, H, V]
 *   S_final : [N, H, K, V] or NULL
 * Value head h reads q/k head h / (H / Hk). With cu_seqlens (B == 1) the
 * state restarts at every sequence start. */
void oracle_gated_delta_rule(const double* q, const double* k, const double* v,
                             const double* g, const double* beta, const double* S0,
                             double* o, double* S_final, const int32_t* cu_seqlens,
                             int n_seqs, int B, int T, int H, int Hk, int K, int V,
                             double scale, int l2norm)
{
    int N = cu_seqlens ? n_seqs : B;
    int group = H / Hk;
    long units = (long)N * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u) {
        int n = (int)(u / H), h = (int)(u % H), hk = h / group;
        long t0 = cu_seqlens ? cu_seqlens[n] : (long)n * T;
        long t1 = cu_seqlens ? cu_seqlens[n + 1] : (long)(n + 1) * T;
        double* S = (double*)calloc((size_t)V * K, sizeof(double));
        double* sk = (double*)malloc(sizeof(double) * (size_t)V);
        double* kt = (double*)malloc(sizeof(double) * (size_t)K);
        double* qt = (double*)malloc(sizeof(double) * (size_t)K);
        if (S0) {
            const double* s0 = S0 + ((long)n * H + h) * K * V;
            for (int j = 0; j < K; ++j)
                for (int i = 0; i < V; ++i) S[(long)i * K + j] = s0[(long)j * V + i];
        }
        for (long t = t0; t < t1; ++t) {
            const double* kr = k + (t * Hk + hk) * K;
            const double* qr = q + (t * Hk + hk) * K;
            if (l2norm) {
                l2_normalise(kr, kt, K);
                l2_normalise(qr, qt, K);
            } else {
                memcpy(kt, kr, sizeof(double) * K);
                memcpy(qt, qr, sizeof(double) * K);
            }
            double alpha = exp(g[t * H + h]);
            gdr_step(S, K, V, kt, v + (t * H + h) * V, alpha, beta[t * H + h], sk);
            gdr_readout(S, K, V, qt, scale, o + (t * H + h) * V);
        }
        if (S_final) {
            double* sf = S_final + ((long)n * H + h) * K * V;
            for (int j = 0; j < K; ++j)
                for (int i = 0; i < V; ++i) sf[(long)j * V + i] = S[(long)i * K + j];
        }
        free(S); free(sk); free(kt); free(qt);
    }
}

/* --------------------------------------------------------------- decode */

/* [GDP] "gdp_decode_prepare": split one decode step's post-conv row into
 * value, key and query, expand q/k groups to heads, interleave the M
 * Householder copies (query only on the last copy, the decay only on the
 * first) and gate the ba row.
 *   x  : [n, M*H*P + M*G*N + G*N]   value | key | query
 *   ba : [n, M*H + H]               b (one per copy and head) | a (per head)
 * Outputs (the layouts [GDP] lists under Returns):
 *   qo, ko : [n, M, H, N];  vo : [n, M, H, P];  beta, g : [n, M, H]. */
void oracle_gdp_decode_prepare(const double* x, const double* ba, const double* A_log,
                               const double* dt_bias, double* qo, double* ko, double* vo,
                               double* beta, double* g, int n, int M, int H, int G,
                               int P, int N)
{
    long row = (long)M * H * P + (long)M * G * N + (long)G * N;
    long barow = (long)M * H + H;
    int per_group = H / G;
    long k_base = (long)M * H * P, q_base = k_base + (long)M * G * N;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < n; ++r) {
        const double* xr = x + r * row;
        const double* br = ba + r * barow;
        for (int m = 0; m < M; ++m)
            for (int h = 0; h < H; ++h) {
                int grp = h / per_group;
                long o = ((r * M + m) * H + h);
                for (int p = 0; p < P; ++p) vo[o * P + p] = xr[((long)m * H + h) * P + p];
                for (int i = 0; i < N; ++i) {
                    ko[o * N + i] = xr[k_base + ((long)m * G + grp) * N + i];
                    qo[o * N + i] = (m == M - 1) ? xr[q_base + (long)grp * N + i] : 0.0;
                }
                beta[o] = 1.0 / (1.0 + exp(-br[(long)m * H + h]));
                g[o] = (m == 0)
                    ? -exp(A_log[h]) * oracle_softplus(br[(long)M * H + h] + dt_bias[h])
                    : 0.0;
            }
    }
}

/* One decode token of the Gated DeltaProduct: prepare ([GDP]) and then the
 * gated delta rule over the M-length sequence of each request, the order
 * [GDP] Returns names for the recurrent kernel.
 *   state : [n, H, N, P] (K x V orientation, N = key dim, P = value dim),
 *           updated in place.
 *   o     : [n, H, P], the output of the last copy (earlier copies carry a
 *           zero query, so their outputs are exactly zero). */
void oracle_gdp_decode(const double* x, const double* ba, const double* A_log,
                       const double* dt_bias, double* state, double* o, int n, int M,
                       int H, int G, int P, int N, double scale, int l2norm)
{
    size_t nm = (size_t)n * M * H;
    double* qo = (double*)malloc(sizeof(double) * nm * N);
    double* ko = (double*)malloc(sizeof(double) * nm * N);
    double* vo = (double*)malloc(sizeof(double) * nm * P);
    double* bo = (double*)malloc(sizeof(double) * nm);
    double* go = (double*)malloc(sizeof(double) * nm);
    oracle_gdp_decode_prepare(x, ba, A_log, dt_bias, qo, ko, vo, bo, go, n, M, H, G, P, N);
    long units = (long)n * H;
#pragma omp parallel for schedule(dynamic, 4)
    for (long u = 0; u < units; ++u) {
        long r = u / H;
        int h = (int)(u % H);
        double* S = (double*)malloc(sizeof(double) * (size_t)P * N);
        double* sk = (double*)malloc(sizeof(double) * (size_t)P);
        double* kt = (double*)malloc(sizeof(double) * (size_t)N);
        double* qt = (double*)malloc(sizeof(double) * (size_t)N);
        double* st = state + u * (long)N * P;
        for (int j = 0; j < N; ++j)
            for (int i = 0; i < P; ++i) S[(long)i * N + j] = st[(long)j * P + i];
        for (int m = 0; m < M; ++m) {
            long idx = (r * M + m) * H + h;
            if (l2norm) {
                l2_normalise(ko + idx * N, kt, N);
                if (m == M - 1) l2_normalise(qo + idx * N, qt, N);
                else memset(qt, 0, sizeof(double) * N);
            } else {
                memcpy(kt, ko + idx * N, sizeof(double) * N);
                memcpy(qt, qo + idx * N, sizeof(double) * N);
            }
            gdr_step(S, N, P, kt, vo + idx * P, exp(go[idx]), bo[idx], sk);
            if (m == M - 1) gdr_readout(S, N, P, qt, scale, o + u * P);
        }
        for (int j = 0; j < N; ++j)
            for (int i = 0; i < P; ++i) st[(long)j * P + i] = S[(long)i * N + j];
        free(S); free(sk); free(kt); free(qt);
    }
    free(qo); free(ko); free(vo); free(bo); free(go);
}

/* ------------------------------------------------------- decode short conv */

/* The short-conv update of one decode token per request, the step [GDP]'s
 * module introduction places before the decode preparation, with its padding
 * rule (a -1 slot zeroes the request's output). The convolution is [ZZ] item
 * 1's, evaluated at the newest token of a window held per slot:
 *   state [n_slots][W-1][C]: row j is the input W-1-j tokens back;
 *   y[r][c] = act(bias[c] + sum_{j<W-1} w[c][j] state[s][j][c] + w[c][W-1] x[r][c]);
 *   then the slot's rows shift one token and x[r] becomes the newest row.
 * A slot outside [0, n_slots) (-1 marks padding) gives a zero row and no
 * update. Requests are independent (distinct slots). */
void oracle_conv1d_update(const double* x, double* state, const int32_t* slot,
                          const double* w, const double* bias, double* y,
                          int n, int n_slots, int C, int W, int silu)
{
    for (long r = 0; r < n; ++r) {
        int s = slot[r];
        if (s < 0 || s >= n_slots) {
            for (int c = 0; c < C; ++c) y[r * C + c] = 0.0;
            continue;
        }
        double* st = state + (long)s * (W - 1) * C;
        for (int c = 0; c < C; ++c) {
            double acc = bias ? bias[c] : 0.0;
            for (int j = 0; j < W - 1; ++j) acc += w[(long)c * W + j] * st[(long)j * C + c];
            acc += w[(long)c * W + W - 1] * x[r * C + c];
            y[r * C + c] = silu ? acc / (1.0 + exp(-acc)) : acc;
        }
        for (int j = 0; j + 1 < W - 1; ++j)
            for (int c = 0; c < C; ++c) st[(long)j * C + c] = st[(long)(j + 1) * C + c];
        for (int c = 0; c < C; ++c) st[(long)(W - 2) * C + c] = x[r * C + c];
    }
}

/* ------------------------------------------------- Gated DeltaProduct prefill */

/* A Gated DeltaProduct layer over a whole prefill, by its definition: every
 * token of a sequence is one decode step of oracle_gdp_decode (the M
 * Householder copies as an M-step sequence, [GDP] module introduction and
 * "gdp_decode_prepare"), with the state carried from token to token.
 *   x [rows][M*H*P + M*G*N + G*N], ba [rows][M*H + H]: token t of batch b is
 *   row b*T + t (packed: B == 1, sequences by cu_seqlens);
 *   state [n_seq][H][N][P]: the initial state on entry, the final on return;
 *   o [rows][H][P]. */
void oracle_gdp_prefill(const double* x, const double* ba, const double* A_log,
                        const double* dt_bias, double* state, double* o,
                        const int32_t* cu_seqlens, int n_seqs, int B, int T, int M, int H,
                        int G, int P, int N, double scale, int l2norm)
{
    long row = (long)M * H * P + (long)M * G * N + (long)G * N;
    long barow = (long)M * H + H;
    int nseq = cu_seqlens ? n_seqs : B;
    for (int s = 0; s < nseq; ++s) {
        long t0 = cu_seqlens ? cu_seqlens[s] : (long)s * T;
        long t1 = cu_seqlens ? cu_seqlens[s + 1] : (long)(s + 1) * T;
        double* st = state + (long)s * H * N * P;
        for (long t = t0; t < t1; ++t)
            oracle_gdp_decode(x + t * row, ba + t * barow, A_log, dt_bias, st, o + t * H * P,
                              1, M, H, G, P, N, scale, l2norm);
    }
}
