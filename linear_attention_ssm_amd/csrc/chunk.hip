// chunk.hip -- the gated delta rule in 64-timestep chunks (prefill forward).
//
// "ZzCompute" (PyTorch Helion Hackathon gallery) splits the chunked forward
// into a WY recompute of keys/values per chunk (item 4, fully parallel), a
// sequential inter-chunk K x V state scan parallel over batch x head (item 2,
// "the sequential bottleneck") and a per-chunk output mixing the inter-chunk
// state query with intra-chunk causal attention (item 3). The equations it
// cites by number are not printed; the ones used here follow from the
// timestep recurrence (per chunk r = 1..L, entering state h, G_r = inclusive
// cumsum of g inside the chunk, gamma_r = exp(G_r), Gamma_rs = exp(G_r - G_s)
// for s <= r else 0):
//     A  = strict_lower(diag(beta) (K K^T o Gamma)),  T = (I + A)^-1 diag(beta)
//     U  = T (V - diag(gamma) K h)
//     O  = scale * (diag(gamma) Q h + (Q K^T o Gamma) U)
//     h' = gamma_L h + (diag(gamma_L / gamma) K)^T U
//
// Split for CDNA4 (two kernels on one stream):
//   chunk_prep  one workgroup per (chunk, q/k head), all chunks in parallel:
//               L2-normalise K, K K^T on MFMA, per value head of the group the
//               cumsum G, A, and the 64 x 64 unit-lower-triangular inverse
//               (16 x 16 diagonal blocks by forward substitution, off-diagonal
//               blocks by block substitution on fp32 MFMA), then T = N diag(beta)
//               and G go to the workspace.
//   chunk_scan  one workgroup per (sequence, value head, 16*NW value columns),
//               sequential over the sequence's chunks. Each wave owns 16 value
//               columns of the fp32 state, kept in MFMA accumulators for the
//               whole sequence; accumulator tiles feed the next product
//               directly as B operands (see gdn_common.hpp), so the chain
//               h -> K h -> U = T(V - gamma K h) -> h' never leaves registers.
//               Q K^T o Gamma (the intra-chunk attention) is formed per chunk
//               on MFMA and shared through LDS.
// The state is never written per chunk: only the final state (if asked for).
#include "gdn_common.hpp"

namespace gdn {

constexpr int kPrepThreads = 256;
constexpr int kLowerTiles = 10;     // 16 x 16 tiles on or below the diagonal of a 64 x 64 matrix

// Lower tile t (0..9) in row order: (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
__device__ __forceinline__ int tri_row(int t) { return t >= 6 ? 3 : (t >= 3 ? 2 : (t >= 1 ? 1 : 0)); }
__device__ __forceinline__ int tri_col(int t) { const int r = tri_row(t); return t - r * (r + 1) / 2; }

// LDS row padding (elements) of the staged tiles.
template <typename T> struct Pad { static constexpr int row = 8; };
template <> struct Pad<float> { static constexpr int row = 4; };

// ------------------------------------------------------------ chunk plan

// offsets[i] = sum_{j < i} ceil(len_j / 64) for packed sequences (one block).
__global__ __launch_bounds__(256) void chunk_plan_kernel(const int32_t* __restrict__ cu, int n,
                                                         int32_t* __restrict__ offsets)
{
    __shared__ int32_t buf[256];
    __shared__ int32_t carry_s;
    if (threadIdx.x == 0) { carry_s = 0; offsets[0] = 0; }
    __syncthreads();
    for (int base = 0; base < n; base += 256) {
        int i = base + threadIdx.x;
        int c = 0;
        if (i < n) c = (cu[i + 1] - cu[i] + kChunk - 1) / kChunk;
        buf[threadIdx.x] = c;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            int add = threadIdx.x >= d ? buf[threadIdx.x - d] : 0;
            __syncthreads();
            buf[threadIdx.x] += add;
            __syncthreads();
        }
        int carry = carry_s;
        if (i < n) offsets[i + 1] = carry + buf[threadIdx.x];
        __syncthreads();
        if (threadIdx.x == 255) carry_s = carry + buf[255];
        __syncthreads();
    }
}

struct ChunkLoc {
    int tok0;   // first token row of the chunk
    int L;      // valid rows (1..64)
    int seq;    // sequence index
};

// tile -> (sequence, chunk). Dense: tile = seq * nck + c. Packed: offsets
// from chunk_plan_kernel, the largest seq with offsets[seq] <= tile.
__device__ __forceinline__ bool locate_tile(int tile, const int32_t* __restrict__ cu,
                                            const int32_t* __restrict__ offsets, int n_seqs,
                                            int T_len, ChunkLoc& loc)
{
    if (!cu) {
        const int nck = (T_len + kChunk - 1) / kChunk;
        const int seq = tile / nck, c = tile - seq * nck;
        loc.seq = seq;
        loc.tok0 = seq * T_len + c * kChunk;
        loc.L = min(kChunk, T_len - c * kChunk);
        return true;
    }
    if (tile >= offsets[n_seqs]) return false;
    int lo = 0, hi = n_seqs;   // offsets[lo] <= tile < offsets[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (offsets[mid] <= tile) lo = mid; else hi = mid;
    }
    const int c = tile - offsets[lo];
    loc.seq = lo;
    loc.tok0 = cu[lo] + c * kChunk;
    loc.L = min(kChunk, cu[lo + 1] - loc.tok0);
    return true;
}

// Stage a 64 x KD tile of token rows (rows >= L zero) into a row-major LDS
// tile with row stride `ld`, L2-normalising each row when asked. Optionally
// also writes the transpose (KD x 64, row stride ldt).
template <typename T, int KD, int NT>
__device__ __forceinline__ void stage_rows(const T* __restrict__ src, int64_t stride, int L,
                                           int l2norm, T* dst, int ld, T* dstT, int ldt)
{
    typedef V16<T> V;
    constexpr int VN = V::n;
    constexpr int SEGS = KD / VN;          // 16-byte segments per row
    constexpr int RPP = NT / SEGS;         // rows per pass
    static_assert(SEGS <= kWave && NT % SEGS == 0 && kChunk % RPP == 0, "staging shape");
    const int tid = threadIdx.x;
    const int seg = tid % SEGS;
#pragma unroll
    for (int p = 0; p < kChunk / RPP; ++p) {
        const int row = p * RPP + tid / SEGS;
        typename V::type raw{};
        if (row < L) raw = *reinterpret_cast<const typename V::type*>(src + row * stride + seg * VN);
        typename V::ftype f = V::to_float(raw);
        if (l2norm) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < VN; ++e) ss += f[e] * f[e];
            ss = group_sum<SEGS>(ss);
            const float inv = 1.f / sqrtf(ss + 1e-6f);
#pragma unroll
            for (int e = 0; e < VN; ++e) f[e] *= inv;
        }
        typename V::type out = V::from_float(f);
        *reinterpret_cast<typename V::type*>(dst + row * ld + seg * VN) = out;
        if (dstT) {
#pragma unroll
            for (int e = 0; e < VN; ++e) dstT[(seg * VN + e) * ldt + row] = out[e];
        }
    }
}

// ------------------------------------------------------------ chunk_prep

template <typename T, int KD>
struct PrepSmem {
    static constexpr int ldk = KD + Pad<T>::row;
    static constexpr int lda = kChunk + 4;
    T k[kChunk * ldk];
    float a[kChunk * lda];     // A, strictly lower
    float n[kChunk * lda];     // N = (I + A)^-1, lower
    float G[kChunk];
    float beta[kChunk];
};

template <typename T, int KD>
__global__ __launch_bounds__(kPrepThreads) void chunk_prep_kernel(
    const T* __restrict__ kp, int64_t qk_stride, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ offsets, int n_seqs, int T_len, int H, int Hk, int l2norm,
    float* __restrict__ ws_G, T* __restrict__ ws_T)
{
    typedef Mma<T> MT;
    typedef PrepSmem<T, KD> SM;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    const int tile = blockIdx.x;
    const int hk = blockIdx.y;
    ChunkLoc loc;
    if (!locate_tile(tile, cu, offsets, n_seqs, T_len, loc)) return;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int grp = lane >> 4;
    const int col = lane & 15;

    stage_rows<T, KD, kPrepThreads>(kp + (int64_t)loc.tok0 * qk_stride + hk * KD, qk_stride,
                                    loc.L, l2norm, sm.k, SM::ldk, (T*)nullptr, 0);
    __syncthreads();

    // K K^T: the 10 lower 16 x 16 tiles, dealt round-robin to the 4 waves.
    f32x4 S[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        S[j] = zero4();
        const int t = wave + 4 * j;
        if (t < kLowerTiles) {
#pragma unroll
            for (int kb = 0; kb < KD / 32; ++kb) {
                auto a = MT::lds_frag(sm.k, SM::ldk, 16 * tri_row(t) + col, 32 * kb, grp);
                auto b = MT::lds_frag(sm.k, SM::ldk, 16 * tri_col(t) + col, 32 * kb, grp);
                S[j] = MT::mma(a, b, S[j]);
            }
        }
    }

    const int per = H / Hk;
    for (int hv = 0; hv < per; ++hv) {
        const int h = hk * per + hv;
        const int64_t wsidx = (int64_t)tile * H + h;
        if (wave == 0) {
            // G = inclusive cumsum of g over the chunk (rows >= L carry g = 0)
            float gv = 0.f, bv = 0.f;
            if (lane < loc.L) {
                gv = g[(int64_t)(loc.tok0 + lane) * H + h];
                bv = beta[(int64_t)(loc.tok0 + lane) * H + h];
            }
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                float up = __shfl_up(gv, d, kWave);
                if (lane >= d) gv += up;
            }
            sm.G[lane] = gv;
            sm.beta[lane] = bv;
            ws_G[wsidx * kChunk + lane] = gv;
        }
        __syncthreads();

        // A[r][s] = beta_r exp(G_r - G_s) (k_r . k_s) for s < r
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int t = wave + 4 * j;
            if (t < kLowerTiles) {
                const int s = 16 * tri_col(t) + col;
                const float Gs = sm.G[s];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * tri_row(t) + 4 * grp + e;
                    float a = 0.f;
                    if (s < r) a = sm.beta[r] * __expf(sm.G[r] - Gs) * S[j][e];
                    sm.a[r * SM::lda + s] = a;
                }
            }
        }
        __syncthreads();

        // diagonal blocks: wave w inverts I + A_ww by forward substitution,
        // lane j < 16 solving for column j.
        if (lane < 16) {
            const int b0 = 16 * wave;
            float xcol[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == lane) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc -= sm.a[(b0 + r) * SM::lda + b0 + s] * xcol[s];
                xcol[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.n[(b0 + r) * SM::lda + b0 + lane] = xcol[r];
        }
        __syncthreads();

        // off-diagonal blocks by block rows: N_iw = -N_ii sum_{k=w}^{i-1} A_ik N_kw
        for (int i = 1; i < 4; ++i) {
            if (wave < i) {
                const int w = wave;
                f32x4 X = zero4();
                for (int kk = w; kk < i; ++kk) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const float av = sm.a[(16 * i + col) * SM::lda + 16 * kk + 4 * grp + s];
                        const float bv = sm.n[(16 * kk + 4 * grp + s) * SM::lda + 16 * w + col];
                        X = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, X, 0, 0, 0);
                    }
                }
                f32x4 Y = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float av = sm.n[(16 * i + col) * SM::lda + 16 * i + 4 * grp + s];
                    Y = __builtin_amdgcn_mfma_f32_16x16x4f32(av, X[s], Y, 0, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.n[(16 * i + 4 * grp + e) * SM::lda + 16 * w + col] = -Y[e];
            }
            __syncthreads();
        }

        // T = N diag(beta), zero above the diagonal; 64 x 64 row-major.
        {
            const int r = tid >> 2;
            const int s0 = (tid & 3) * 16;
            T* dst = ws_T + wsidx * (kChunk * kChunk) + r * kChunk + s0;
            typedef V16<T> V;
#pragma unroll
            for (int v = 0; v < 16 / V::n; ++v) {
                typename V::ftype f;
#pragma unroll
                for (int e = 0; e < V::n; ++e) {
                    const int s = s0 + v * V::n + e;
                    f[e] = (s <= r) ? sm.n[r * SM::lda + s] * sm.beta[s] : 0.f;
                }
                *reinterpret_cast<typename V::type*>(dst + v * V::n) = V::from_float(f);
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ chunk_scan

template <typename T, int KD>
struct ScanSmem {
    static constexpr int ldk = KD + Pad<T>::row;       // K, Q tiles [64][ldk]
    static constexpr int ldt = kChunk + Pad<T>::row;   // K^T [KD][ldt]; T, P [64][ldt]
    T k[kChunk * ldk];
    T q[kChunk * ldk];
    T kt[KD * ldt];
    T tm[kChunk * ldt];
    T p[kChunk * ldt];
    float G[kChunk];
};

template <typename T, int KD, int NW>
__global__ __launch_bounds__(NW * kWave) void chunk_scan_kernel(
    const T* __restrict__ qp, const T* __restrict__ kp, int64_t qk_stride,
    const T* __restrict__ vp, int64_t v_stride,
    const float* __restrict__ S0, float* __restrict__ Sfin, T* __restrict__ o,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ offsets,
    const float* __restrict__ ws_G, const T* __restrict__ ws_T,
    int n_seqs, int T_len, int H, int Hk, int V, int units, int groups, float scale, int l2norm)
{
    typedef Mma<T> MT;
    typedef ScanSmem<T, KD> SM;
    constexpr int NT = NW * kWave;
    constexpr int RT = KD / 16;      // 16-row tiles of the state
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    // XCD-aware block order: all column groups of one (seq, head) unit get the
    // same blockIdx % 8, i.e. run on the same XCD and share its L2 for K, Q, T.
    const int bid = blockIdx.x;
    const int rest = bid >> 3;
    const int cgrp = rest % groups;
    const int u = (rest / groups) * 8 + (bid & 7);
    if (u >= units) return;
    const int seq = u / H;
    const int h = u - seq * H;
    const int hk = h / (H / Hk);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int grp = lane >> 4;
    const int col = lane & 15;
    const int c0 = (cgrp * NW + wave) * 16;     // this wave's value columns c0..c0+15
    const int vc = c0 + col;

    int tok_begin, tok_end, tile0;
    if (cu) {
        tok_begin = cu[seq];
        tok_end = cu[seq + 1];
        tile0 = offsets[seq];
    } else {
        tok_begin = seq * T_len;
        tok_end = tok_begin + T_len;
        tile0 = seq * ((T_len + kChunk - 1) / kChunk);
    }

    // state tile rt holds h[16 rt + 4 grp + e][vc]
    f32x4 hs[RT];
    const int64_t sbase = ((int64_t)seq * H + h) * KD * V;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            hs[rt][e] = S0 ? S0[sbase + (int64_t)(16 * rt + 4 * grp + e) * V + vc] : 0.f;

    // P's tiles above the diagonal are read by P U as zeros and never written
    for (int i = tid; i < kChunk * SM::ldt; i += NT) sm.p[i] = from_f32<T>(0.f);
    __syncthreads();

    const int nchunks = (tok_end - tok_begin + kChunk - 1) / kChunk;
    for (int c = 0; c < nchunks; ++c) {
        const int tok0 = tok_begin + c * kChunk;
        const int L = min(kChunk, tok_end - tok0);
        const int64_t wsidx = (int64_t)(tile0 + c) * H + h;

        // ---- stage K (row-major and transposed), Q, T, G
        stage_rows<T, KD, NT>(kp + (int64_t)tok0 * qk_stride + hk * KD, qk_stride, L, l2norm,
                              sm.k, SM::ldk, sm.kt, SM::ldt);
        stage_rows<T, KD, NT>(qp + (int64_t)tok0 * qk_stride + hk * KD, qk_stride, L, l2norm,
                              sm.q, SM::ldk, (T*)nullptr, 0);
        {
            typedef V16<T> VV;
            constexpr int SEGS = kChunk / VV::n;
            const T* src = ws_T + wsidx * (kChunk * kChunk);
            for (int i = tid; i < kChunk * SEGS; i += NT) {
                const int r = i / SEGS, sg = i - r * SEGS;
                *reinterpret_cast<typename VV::type*>(sm.tm + r * SM::ldt + sg * VV::n) =
                    *reinterpret_cast<const typename VV::type*>(src + r * kChunk + sg * VV::n);
            }
            for (int i = tid; i < kChunk; i += NT) sm.G[i] = ws_G[wsidx * kChunk + i];
        }
        // values of this wave's columns, in accumulator layout (rows >= L zero)
        float vreg[4][4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * grp + e;
                vreg[rt][e] = (r < L) ? to_f32(vp[(int64_t)(tok0 + r) * v_stride + h * V + vc]) : 0.f;
            }
        __syncthreads();

        // ---- h as B operand (contraction over the key dim)
        typename MT::Frag hf[KD / 32];
#pragma unroll
        for (int kb = 0; kb < KD / 32; ++kb) hf[kb] = MT::acc_frag(hs[2 * kb], hs[2 * kb + 1]);

        // ---- X = K h, Y = Q h
        f32x4 X[4], Y[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            X[rt] = zero4();
            Y[rt] = zero4();
#pragma unroll
            for (int kb = 0; kb < KD / 32; ++kb) {
                X[rt] = MT::mma(MT::lds_frag(sm.k, SM::ldk, 16 * rt + col, 32 * kb, grp), hf[kb], X[rt]);
                Y[rt] = MT::mma(MT::lds_frag(sm.q, SM::ldk, 16 * rt + col, 32 * kb, grp), hf[kb], Y[rt]);
            }
        }

        // ---- P = (Q K^T) o Gamma (lower incl. diagonal), tiles dealt to waves
        // (the tiles above the diagonal stay zero from the fill before the loop)
        for (int t = wave; t < kLowerTiles; t += NW) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < KD / 32; ++kb)
                acc = MT::mma(MT::lds_frag(sm.q, SM::ldk, 16 * tri_row(t) + col, 32 * kb, grp),
                              MT::lds_frag(sm.k, SM::ldk, 16 * tri_col(t) + col, 32 * kb, grp), acc);
            const int s = 16 * tri_col(t) + col;
            const float Gs = sm.G[s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tri_row(t) + 4 * grp + e;
                const float pv = (s <= r) ? acc[e] * __expf(sm.G[r] - Gs) : 0.f;
                sm.p[r * SM::ldt + s] = from_f32<T>(pv);
            }
        }

        // ---- V' = V - gamma o X
        float gam[4][4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gam[rt][e] = __expf(sm.G[16 * rt + 4 * grp + e]);
                X[rt][e] = vreg[rt][e] - gam[rt][e] * X[rt][e];
            }

        // ---- U = T V'  (T lower triangular: row tile rt needs kb <= rt/2)
        f32x4 U[4];
        {
            typename MT::Frag vf0 = MT::acc_frag(X[0], X[1]);
            typename MT::Frag vf1 = MT::acc_frag(X[2], X[3]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                U[rt] = MT::mma(MT::lds_frag(sm.tm, SM::ldt, 16 * rt + col, 0, grp), vf0, zero4());
                if (rt >= 2) U[rt] = MT::mma(MT::lds_frag(sm.tm, SM::ldt, 16 * rt + col, 32, grp), vf1, U[rt]);
            }
        }
        __syncthreads();   // P complete

        // ---- O = scale (gamma o Y + P U)
        {
            typename MT::Frag uf0 = MT::acc_frag(U[0], U[1]);
            typename MT::Frag uf1 = MT::acc_frag(U[2], U[3]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 acc = MT::mma(MT::lds_frag(sm.p, SM::ldt, 16 * rt + col, 0, grp), uf0, zero4());
                if (rt >= 2) acc = MT::mma(MT::lds_frag(sm.p, SM::ldt, 16 * rt + col, 32, grp), uf1, acc);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rt + 4 * grp + e;
                    if (r < L)
                        o[((int64_t)(tok0 + r) * H + h) * V + vc] =
                            from_f32<T>(scale * (gam[rt][e] * Y[rt][e] + acc[e]));
                }
            }
        }

        // ---- h' = gamma_L h + K^T (diag(gamma_L / gamma) U)
        {
            const float GL = sm.G[kChunk - 1];
            const float gL = __expf(GL);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) U[rt][e] *= __expf(GL - sm.G[16 * rt + 4 * grp + e]);
            typename MT::Frag df0 = MT::acc_frag(U[0], U[1]);
            typename MT::Frag df1 = MT::acc_frag(U[2], U[3]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f32x4 acc = hs[rt] * gL;
                acc = MT::mma(MT::lds_frag(sm.kt, SM::ldt, 16 * rt + col, 0, grp), df0, acc);
                acc = MT::mma(MT::lds_frag(sm.kt, SM::ldt, 16 * rt + col, 32, grp), df1, acc);
                hs[rt] = acc;
            }
        }
        __syncthreads();   // LDS free for the next chunk
    }

    if (Sfin) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Sfin[sbase + (int64_t)(16 * rt + 4 * grp + e) * V + vc] = hs[rt][e];
    }
}

// ------------------------------------------------------------ launchers

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static inline int64_t tiles_upper_bound(int B, int T_len, int n_seqs, bool packed) {
    if (!packed) return (int64_t)B * ((T_len + kChunk - 1) / kChunk);
    return ((int64_t)T_len + (int64_t)(kChunk - 1) * n_seqs) / kChunk;
}

size_t chunk_workspace_bytes(int B, int T_len, int H, int n_seqs, bool packed, bool use_bf16) {
    const int64_t tiles = tiles_upper_bound(B, T_len, n_seqs, packed);
    const size_t esz = use_bf16 ? 2 : 4;
    size_t off = align256(sizeof(int32_t) * (size_t)(n_seqs + 1));
    off += align256(sizeof(float) * (size_t)tiles * H * kChunk);
    off += align256(esz * (size_t)tiles * H * kChunk * kChunk);
    return off;
}

template <typename K>
static hipError_t set_smem(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, int KD, int NW>
static hipError_t launch_scan(const void* q, const void* k, int64_t qks, const void* v, int64_t vs,
                              const float* S0, float* Sf, void* o, const int32_t* cu,
                              const int32_t* offsets, const float* wsG, const void* wsT,
                              int n_seqs, int T_len, int H, int Hk, int V, int N, float scale,
                              int l2norm, hipStream_t stream)
{
    const int units = N * H;
    const int groups = V / (16 * NW);
    const int upad = (units + 7) / 8 * 8;
    const size_t smem = sizeof(ScanSmem<T, KD>);
    auto kern = chunk_scan_kernel<T, KD, NW>;
    hipError_t err = set_smem(kern, smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3((unsigned)(upad * groups)), dim3(NW * kWave), smem, stream,
                       (const T*)q, (const T*)k, qks, (const T*)v, vs, S0, Sf, (T*)o, cu, offsets,
                       wsG, (const T*)wsT, n_seqs, T_len, H, Hk, V, units, groups, scale, l2norm);
    return hipGetLastError();
}

template <typename T, int KD>
static hipError_t launch_chunk_t(const void* q, const void* k, int64_t qks, const void* v,
                                 int64_t vs, const float* g, const float* beta, const float* S0,
                                 float* Sf, void* o, const int32_t* cu, int n_seqs, int B,
                                 int T_len, int H, int Hk, int V, float scale, int l2norm,
                                 void* ws, hipStream_t stream)
{
    const bool packed = cu != nullptr;
    const int N = packed ? n_seqs : B;
    const int64_t tiles = tiles_upper_bound(B, T_len, n_seqs, packed);
    char* base = (char*)ws;
    int32_t* offsets = (int32_t*)base;
    size_t off = align256(sizeof(int32_t) * (size_t)(n_seqs + 1));
    float* wsG = (float*)(base + off);
    off += align256(sizeof(float) * (size_t)tiles * H * kChunk);
    T* wsT = (T*)(base + off);

    if (packed) {
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(256), 0, stream, cu, n_seqs, offsets);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (tiles > 0) {
        const size_t smem = sizeof(PrepSmem<T, KD>);
        auto kern = chunk_prep_kernel<T, KD>;
        hipError_t e = set_smem(kern, smem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)tiles, Hk), dim3(kPrepThreads), smem, stream,
                           (const T*)k, qks, g, beta, cu, offsets, n_seqs, T_len, H, Hk, l2norm,
                           wsG, wsT);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // columns per workgroup: enough workgroups to cover the 256 CUs, more
    // waves per workgroup (shared K/Q/T staging) when there is parallelism to spare
    const int units = N * H;
    const int slabs = V / 16;
    int nw = 1;
    if (units * (slabs / 4) >= 512 && slabs % 4 == 0) nw = 4;
    else if (units * (slabs / 2) >= 256 && slabs % 2 == 0) nw = 2;
    switch (nw) {
    case 4: return launch_scan<T, KD, 4>(q, k, qks, v, vs, S0, Sf, o, cu, offsets, wsG, wsT, n_seqs, T_len, H, Hk, V, N, scale, l2norm, stream);
    case 2: return launch_scan<T, KD, 2>(q, k, qks, v, vs, S0, Sf, o, cu, offsets, wsG, wsT, n_seqs, T_len, H, Hk, V, N, scale, l2norm, stream);
    default: return launch_scan<T, KD, 1>(q, k, qks, v, vs, S0, Sf, o, cu, offsets, wsG, wsT, n_seqs, T_len, H, Hk, V, N, scale, l2norm, stream);
    }
}

hipError_t launch_chunk_fwd(const void* q, const void* k, int64_t qks, const void* v, int64_t vs,
                            const float* g, const float* beta, const float* S0, float* Sf,
                            void* o, const int32_t* cu, int n_seqs, int B, int T_len, int H,
                            int Hk, int K, int V, float scale, int l2norm, bool use_bf16, void* ws,
                            hipStream_t stream)
{
    if (use_bf16) {
        if (K == 128)
            return launch_chunk_t<bf16, 128>(q, k, qks, v, vs, g, beta, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, scale, l2norm, ws, stream);
        return launch_chunk_t<bf16, 64>(q, k, qks, v, vs, g, beta, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, scale, l2norm, ws, stream);
    }
    if (K == 128)
        return launch_chunk_t<float, 128>(q, k, qks, v, vs, g, beta, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, scale, l2norm, ws, stream);
    return launch_chunk_t<float, 64>(q, k, qks, v, vs, g, beta, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, scale, l2norm, ws, stream);
}

}  // namespace gdn
