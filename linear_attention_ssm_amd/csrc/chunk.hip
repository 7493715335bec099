// chunk.hip -- the gated delta rule in 64-timestep chunks (prefill forward).
//
// "ZzCompute" (PyTorch Helion Hackathon gallery) splits the chunked forward
// into a WY recompute of keys/values per chunk (item 4, fully parallel), a
// sequential inter-chunk K x V state scan parallel over batch x head (item 2,
// "the sequential bottleneck") and a per-chunk output mixing the inter-chunk
// state query with intra-chunk causal attention (item 3). The equations it
// cites by number are not printed; the ones used here follow from the
// timestep recurrence. Per chunk (rows r = 1..L, entering state h (K x V),
// G_r = inclusive cumsum of g inside the chunk, gamma_r = exp(G_r),
// Gamma_rs = exp(G_r - G_s) for s <= r else 0, k^ / q^ = L2-normalised rows):
//     A  = strict_lower(diag(beta) (K^ K^T o Gamma)),  T = (I + A)^-1 diag(beta)
//     U  = T (V - diag(gamma) K^ h)
//     O  = scale (diag(gamma) Q^ h + (Q^ K^T o Gamma) U)
//     h' = gamma_L h + (diag(gamma_L / gamma) K^)^T U
// With the row norms n_r of k and m_r of q kept as per-row factors, the MFMA
// operands of the state products are the RAW q/k rows:
//     U  = T (V - a o (K h)),   a_r = gamma_r / n_r
//     O  = b o (Q h) + P U,     b_r = scale gamma_r / m_r,
//                               P = scale (Q K^T o Gamma) / (m_r n_s)
//     h' = gamma_L h + K^T (c o U),  c_r = gamma_L / (gamma_r n_r)
//
// Split for CDNA4 (two kernels on one stream):
//   chunk_prep  one workgroup per (chunk, q/k head), every chunk in parallel:
//               row norms, K K^T and Q K^T on MFMA (shared by the value heads
//               of a GQA group), then per value head the cumsum, A, the
//               64 x 64 unit-lower-triangular inverse (16 x 16 diagonal blocks
//               by forward substitution, off-diagonal blocks by block
//               substitution on fp32 MFMA), T, P and the factors a, b, c,
//               gamma_L. T and P are written as ready MFMA A-operand
//               fragments (only the 6 non-zero 16 x 32 blocks of each).
//   chunk_scan  one workgroup per (sequence, value head, 16*NW value columns),
//               sequential over the sequence's chunks. Each wave owns 16 value
//               columns of the fp32 state, held in MFMA accumulators for the
//               whole sequence; accumulator tiles feed the next product
//               directly as B operands (see gdn_common.hpp), so the chain
//               h -> K h -> U -> h' never leaves registers. The raw K and Q
//               tiles and the chunk's record are copied global -> LDS with
//               direct-to-LDS loads one chunk ahead (double buffer), K^T
//               operands are read from the row-major K tile with the gfx950
//               transposing LDS read, and nothing but the outputs and the
//               final state is written.
#include "gdn_common.hpp"

namespace gdn {

constexpr int kPrepThreads = 256;
constexpr int kPrepWavesPerEU = 2;
constexpr int kPrepHeads = 4;      // value heads per key head whose gates the prep requests up front
constexpr int kLowerTiles = 10;     // 16 x 16 tiles on or below the diagonal of a 64 x 64 matrix
constexpr int kTriFrags = 6;        // non-zero 16 x 32 A-operand blocks of a lower-triangular 64 x 64

// Lower tile t (0..9) in row order: (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
__device__ __forceinline__ int tri_row(int t) { return t >= 6 ? 3 : (t >= 3 ? 2 : (t >= 1 ? 1 : 0)); }
__device__ __forceinline__ int tri_col(int t) { const int r = tri_row(t); return t - r * (r + 1) / 2; }
// A-operand block (row tile rt, 32-wide contraction block kb) of a lower-triangular matrix:
// (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
__device__ __forceinline__ int tri_frag(int rt, int kb) { return rt < 2 ? rt : 2 + 2 * (rt - 2) + kb; }
__device__ __forceinline__ int tri_frag_rt(int f) { return f < 2 ? f : 2 + (f - 2) / 2; }
__device__ __forceinline__ int tri_frag_kb(int f) { return f < 2 ? 0 : (f - 2) % 2; }

// Contraction index of operand slot j of lane group grp (see gdn_common.hpp).
__device__ __forceinline__ int slot_k(int grp, int j) { return j < 4 ? 4 * grp + j : 12 + 4 * grp + j; }

// LDS row padding (elements) of the prep kernel's staged tiles.
template <typename T> struct Pad { static constexpr int row = 8; };
template <> struct Pad<float> { static constexpr int row = 4; };

// Per (chunk, value head) record written by chunk_prep and read by chunk_scan:
//   T fragments [6][64 lanes], P fragments [6][64 lanes], factors float [4][64]
//   (a, b, c per row; row 3 holds gamma_L).
template <typename T> struct Rec {
    typedef typename Mma<T>::Frag Frag;
    static constexpr int frag_bytes = (int)sizeof(Frag);                  // 16 (bf16) / 32 (fp32)
    static constexpr int tfrag = 0;
    static constexpr int pfrag = kTriFrags * kWave * frag_bytes;
    static constexpr int fac = 2 * kTriFrags * kWave * frag_bytes;
    static constexpr int bytes = fac + 4 * kChunk * 4;
    static_assert(bytes % 1024 == 0, "records are copied in 1 KiB pieces");
};

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
    loc.tok0 = cu[lo] + (tile - offsets[lo]) * kChunk;
    loc.L = min(kChunk, cu[lo + 1] - loc.tok0);
    return true;
}

// ------------------------------------------------------------ chunk_prep

template <typename T, int KD>
struct PrepSmem {
    static constexpr int ldk = KD + Pad<T>::row;
    static constexpr int lda = kChunk + 4;
    static constexpr int ldp = kChunk + Pad<T>::row;
    // the raw rows are only read by the products that open an item; A and N
    // take their place for the rest of it
    union {
        struct {
            T k[kChunk * ldk];     // raw k rows (rows >= L zero)
            T q[kChunk * ldk];     // raw q rows
        };
        struct {
            float a[kChunk * lda]; // A, strictly lower
            float n[kChunk * lda]; // N = (I + A)^-1, lower
        };
    };
    T p[kChunk * ldp];         // P
    float G[kChunk];
    float beta[kChunk];
    float rk[kChunk];          // 1 / |k_r| (1 without normalisation)
    float rq[kChunk];
};

// A 64 x KD tile of token rows, loaded by NT threads in 16-byte segments (thread
// tid owns segment tid % SEGS of rows tid / SEGS + p * RPP). All loads are
// issued before any is used; rows >= L read row L-1 and are zeroed on store.
template <typename T, int KD, int NT>
struct RowTile {
    typedef V16<T> V;
    static constexpr int VN = V::n;
    static constexpr int SEGS = KD / VN;
    static constexpr int RPP = NT / SEGS;
    static constexpr int NP = kChunk / RPP;
    static_assert(SEGS <= kWave && NT % SEGS == 0 && kChunk % RPP == 0, "staging shape");
    typename V::type raw[NP];

    __device__ __forceinline__ void load(const T* __restrict__ src, int64_t stride, int L) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = p * RPP + tid / SEGS;
            raw[p] = *reinterpret_cast<const typename V::type*>(src + min(row, L - 1) * stride +
                                                                (tid % SEGS) * VN);
        }
    }
    // Store into a padded row-major LDS tile and record each row's inverse L2 norm.
    __device__ __forceinline__ void store(int L, int l2norm, T* dst, int ld, float* rnorm) const {
        const int tid = threadIdx.x;
        const int seg = tid % SEGS;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = p * RPP + tid / SEGS;
            typename V::type r = raw[p];
            if (row >= L) r = typename V::type{};
            typename V::ftype f = V::to_float(r);
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < VN; ++e) ss += f[e] * f[e];
            ss = group_sum<SEGS>(ss);
            const float rn = l2norm ? __builtin_amdgcn_rsqf(ss + 1e-6f) : 1.f;   // (v_rsq_f32, ~1 ulp)
            if (seg == 0) rnorm[row] = rn;
            *reinterpret_cast<typename V::type*>(dst + row * ld + seg * VN) = r;
        }
    }
};

// Two workgroups per CU (registers sized for it): the item's steps
// are short dependent chains, hidden by the other workgroups.
template <typename T, int KD>
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(kPrepWavesPerEU)))
void chunk_prep_kernel(
    const T* __restrict__ qp, const T* __restrict__ kp, int64_t qk_stride,
    const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ offsets, int n_seqs, int T_len,
    int H, int Hk, float scale, int l2norm, unsigned char* __restrict__ ws_rec, int n_items)
{
    typedef Mma<T> MT;
    typedef PrepSmem<T, KD> SM;
    typedef Rec<T> RC;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int grp = lane >> 4;
    const int col = lane & 15;
    const int per = H / Hk;

    // Persistent workgroups: item it = (tile, key head) = (it / Hk, it % Hk). The
    // next item's K and Q rows are loaded into registers while this one is
    // computed, so their HBM latency is hidden behind the arithmetic.
    // T = N diag(beta) and P as A-operand fragments: 12 fragments, 3 per wave.
    // Operand slots j < 4 and j >= 4 are 4 consecutive columns each.
    auto write_frags = [&](unsigned char* rec) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int f = wave + 4 * j;
            const bool isT = f < kTriFrags;
            const int ff = isT ? f : f - kTriFrags;
            const int r = 16 * tri_frag_rt(ff) + col;
            const int kb = tri_frag_kb(ff);
            f32x8 v;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int c0 = 32 * kb + 16 * hh + 4 * grp;     // slots 4 hh .. 4 hh + 3
                f32x4 x;
                if (isT) {
                    x = *reinterpret_cast<const f32x4*>(&sm.n[r * SM::lda + c0]) *
                        *reinterpret_cast<const f32x4*>(&sm.beta[c0]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = to_f32(sm.p[r * SM::ldp + c0 + e]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * hh + e] = (c0 + e <= r) ? x[e] : 0.f;
            }
            typename MT::Frag fr;
            if constexpr (sizeof(typename MT::Frag) == 16) fr = __builtin_convertvector(v, bf16x8);
            else fr = v;
            *reinterpret_cast<typename MT::Frag*>(rec + (isT ? RC::tfrag : RC::pfrag) +
                                                  (ff * kWave + lane) * RC::frag_bytes) = fr;
        }
    };

    // gate values (g, beta) of the first kPrepHeads value heads of an item,
    // lane = row (rows past the end repeat the last one; they are masked later)
    float gn[kPrepHeads], bn[kPrepHeads];
    auto load_gates = [&](int hk_, const ChunkLoc& l) {
        const int lr = min(lane, l.L - 1);
#pragma unroll
        for (int i = 0; i < kPrepHeads; ++i) {
            const int hh = hk_ * per + min(i, per - 1);
            gn[i] = g[(int64_t)(l.tok0 + lr) * H + hh];
            bn[i] = beta[(int64_t)(l.tok0 + lr) * H + hh];
        }
    };
    RowTile<T, KD, kPrepThreads> kt, qt;
    int it = blockIdx.x;
    ChunkLoc loc;
    bool have = it < n_items && locate_tile(it / Hk, cu, offsets, n_seqs, T_len, loc);
    if (have) {
        load_gates(it % Hk, loc);
        const int64_t rowoff = (int64_t)loc.tok0 * qk_stride + (it % Hk) * KD;
        kt.load(kp + rowoff, qk_stride, loc.L);
        qt.load(qp + rowoff, qk_stride, loc.L);
    }
    while (it < n_items) {
        const int tile = it / Hk;
        const int hk = it - tile * Hk;
        const ChunkLoc cur = loc;
        const bool cur_ok = have;
        const int L = cur.L;
        // Order of the vector-memory operations at the top of an item (their
        // counter retires in issue order): the wait for this item's rows and
        // gate values (both requested one item earlier), then the next item's
        // gate values and rows. Every wave issues the same operations, so the
        // counts do not depend on the wave.
        if (cur_ok) {
            kt.store(L, l2norm, sm.k, SM::ldk, sm.rk);
            qt.store(L, l2norm, sm.q, SM::ldk, sm.rq);
        }
        float gv[kPrepHeads], bv[kPrepHeads];
#pragma unroll
        for (int i = 0; i < kPrepHeads; ++i) { gv[i] = gn[i]; bv[i] = bn[i]; }
        const int nit = it + gridDim.x;
        have = nit < n_items && locate_tile(nit / Hk, cu, offsets, n_seqs, T_len, loc);
        if (have) {
            load_gates(nit % Hk, loc);
            const int64_t rowoff = (int64_t)loc.tok0 * qk_stride + (nit % Hk) * KD;
            kt.load(kp + rowoff, qk_stride, loc.L);
            qt.load(qp + rowoff, qk_stride, loc.L);
        }
        if (!cur_ok) { it = nit; continue; }   // (uniform: a packed item past the last chunk)
        __syncthreads();

        // raw K K^T (tiles 0..9) and Q K^T (tiles 10..19), lower 16 x 16 tiles, 5 per wave
        f32x4 S[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int t = wave + 4 * j;
            const int tt = t < kLowerTiles ? t : t - kLowerTiles;
            const T* am = t < kLowerTiles ? sm.k : sm.q;
            S[j] = zero4();
#pragma unroll
            for (int kb = 0; kb < KD / 32; ++kb)
                S[j] = MT::mma(MT::lds_frag(am, SM::ldk, 16 * tri_row(tt) + col, 32 * kb, grp),
                               MT::lds_frag(sm.k, SM::ldk, 16 * tri_col(tt) + col, 32 * kb, grp), S[j]);
        }

        for (int hv = 0; hv < per; ++hv) {
            const int h = hk * per + hv;
            unsigned char* rec = ws_rec + ((int64_t)tile * H + h) * RC::bytes;
            if (wave == 0) {
                // G = inclusive cumsum of g over the chunk (rows >= L carry g = 0)
                float gh = 0.f, bh = 0.f;
#pragma unroll
                for (int i = 0; i < kPrepHeads; ++i)
                    if (i == hv) { gh = gv[i]; bh = bv[i]; }
                if (hv >= kPrepHeads) {   // (more value heads per key head than held above)
                    const int lr = min(lane, L - 1);
                    gh = g[(int64_t)(cur.tok0 + lr) * H + h];
                    bh = beta[(int64_t)(cur.tok0 + lr) * H + h];
                }
                float gc = lane < L ? gh : 0.f;
                const float bc = lane < L ? bh : 0.f;
                gc = wave_inclusive_scan(gc);
                sm.G[lane] = gc;
                sm.beta[lane] = bc;
                const float GL = lane_value(gc, kWave - 1);
                const bool live = lane < L;
                const float gam = __expf(gc);
                float* fac = reinterpret_cast<float*>(rec + RC::fac);
                fac[0 * kChunk + lane] = live ? gam * sm.rk[lane] : 0.f;
                fac[1 * kChunk + lane] = live ? scale * gam * sm.rq[lane] : 0.f;
                fac[2 * kChunk + lane] = live ? __expf(GL - gc) * sm.rk[lane] : 0.f;
                fac[3 * kChunk + lane] = __expf(GL);
            }
            __syncthreads();

            // A (normalised keys, strictly lower) and P (scaled, lower incl. diagonal)
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                const int t = wave + 4 * j;
                const bool isA = t < kLowerTiles;
                const int tt = isA ? t : t - kLowerTiles;
                const int s = 16 * tri_col(tt) + col;
                const int r0 = 16 * tri_row(tt) + 4 * grp;
                const float Gs = sm.G[s];
                const float rks = sm.rk[s];
                const f32x4 Gr = *reinterpret_cast<const f32x4*>(&sm.G[r0]);
                const f32x4 br = *reinterpret_cast<const f32x4*>(&sm.beta[r0]);
                const f32x4 rr = *reinterpret_cast<const f32x4*>(isA ? &sm.rk[r0] : &sm.rq[r0]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = r0 + e;
                    const float decay = __expf(fminf(Gr[e] - Gs, 0.f));
                    if (isA) {
                        sm.a[r * SM::lda + s] = (s < r) ? br[e] * decay * rr[e] * rks * S[j][e] : 0.f;
                    } else {
                        sm.p[r * SM::ldp + s] =
                            from_f32<T>((s <= r) ? scale * decay * rr[e] * rks * S[j][e] : 0.f);
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
                            const float bvv = sm.n[(16 * kk + 4 * grp + s) * SM::lda + 16 * w + col];
                            X = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bvv, X, 0, 0, 0);
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

            // T = N diag(beta) and P as A-operand fragments
            write_frags(rec);
            __syncthreads();
        }
        it = nit;
    }
}

// ------------------------------------------------------------ chunk_scan
//
// State layout in registers. A wave owns 16 value columns of h (K x V); state
// tile rt, lane group grp, accumulator element e holds key row
//     d = 32 (rt / 2) + 8 grp + 4 ((grp / 2 + rt) % 2) + e.
// Tiles 2 kb and 2 kb + 1 together cover key rows 32 kb + 8 grp .. + 7 of each
// lane group, so the B operand built from them (halves swapped in groups 2, 3)
// holds key row 32 kb + 8 grp + j in slot j, and the matching A operand of K
// (or Q) is 8 consecutive elements of one row: a single 16-byte LDS read (two
// for fp32). The K^T products that update h produce rows in the same order;
// the half each tile takes in a group is chosen so that the transposing reads
// of K^T spread over all LDS banks.
//
// Chunk inputs reach LDS through buffer loads with per-chunk resources whose
// size covers only the chunk's valid rows: rows past the end of a sequence
// fall outside the resource and are never fetched, so a partial chunk needs no
// separate path and no clamping. The chunk's outputs leave the same way.

__device__ __forceinline__ int state_half(int rt, int grp) { return ((grp >> 1) + rt) & 1; }
__device__ __forceinline__ int state_row(int rt, int grp, int e) {
    return 32 * (rt >> 1) + 8 * grp + 4 * state_half(rt, grp) + e;
}
// B operand of the state for contraction block kb: slot j holds key row
// 32 kb + 8 grp + j (tile 2 kb supplies the low half in groups 0, 1 and the
// high half in groups 2, 3).
template <typename T>
__device__ __forceinline__ typename Mma<T>::Frag state_frag(const f32x4& t0, const f32x4& t1, int grp) {
    const bool sw = grp >= 2;
    f32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = sw ? t1[e] : t0[e];
        hi[e] = sw ? t0[e] : t1[e];
    }
    return Mma<T>::acc_frag(lo, hi);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Raw buffer resource over [base, base + bytes) (gfx9 descriptor word 3). The
// arguments are wave-uniform; reading them from the first lane keeps the
// resource in scalar registers.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    void* p = (void*)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                             0x00020000);
}
typedef __attribute__((address_space(3))) void* lds_ptr_t;
// 64 lanes x 16 bytes from rsrc + voffset (+ soffset) to LDS dst + 16 lane
__device__ __forceinline__ void dma16(rsrc_t r, unsigned char* dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, voff, soff, 0, 0);
}

// LDS staging of one chunk for the scan: raw K and Q tiles, the chunk's record
// and each wave's 64 x 16 slab of values, all written by direct-to-LDS loads
// in 1 KiB pieces (64 lanes x 16 bytes; each lane picks its source). A wave's
// value slab also carries its outputs of the chunk back out.
template <typename T, int KD, int NW>
struct ScanBuf {
    static constexpr int ES = (int)sizeof(T);
    static constexpr int VN = 16 / ES;                 // elements per 16-byte segment
    static constexpr int RB = KD * ES;                 // bytes per K/Q row
    static constexpr int SPR = RB / 16;                // segments per row
    static constexpr int FSEG = ES / 2;                // segments per operand fragment
    static constexpr int RPI = 1024 / RB;              // rows per 1 KiB piece
    static constexpr int tile_pieces = kChunk * RB / 1024;
    static constexpr int rec_pieces = Rec<T>::bytes / 1024;
    static constexpr int VRB = 16 * ES;                // bytes per row of a wave's value slab
    static constexpr int LPR = VRB / 16;               // lanes per value row
    static constexpr int v_pieces = kChunk * VRB / 1024;
    static constexpr int RPV = kChunk / v_pieces;      // value rows per piece
    // pieces a wave copies per chunk: an equal share of each tile, a share of
    // the record (rpw each; a wave past the last piece repeats it) and its values
    static constexpr int tpw = tile_pieces / NW;
    static constexpr int rpw = (rec_pieces + NW - 1) / NW;
    static constexpr int loads = 2 * tpw + rpw + v_pieces;
    static_assert(tile_pieces % NW == 0, "K/Q pieces are dealt evenly over the waves");
    static_assert(Rec<T>::bytes % 1024 == 0, "the record is whole pieces");
    unsigned char k[kChunk * RB];
    unsigned char q[kChunk * RB];
    unsigned char rec[Rec<T>::bytes];
    unsigned char v[NW][kChunk * VRB];
};

// Physical 16-byte segment of logical segment s of row r in a staged K/Q tile:
// segments are XOR-ed with a row-dependent mask that moves whole fragments
// (FSEG segments). Over 8 consecutive rows the mask takes 8 distinct values
// (row reads of 16 rows hit distinct banks), and over the 4 x 4 rows and
// segments of a transposing read it pairs rows so that, with the half each
// state tile takes, every 8-byte read of a 16-lane group has its own banks.
template <typename T, int KD, int NW>
__device__ __forceinline__ int tile_mask(int r) {
    typedef ScanBuf<T, KD, NW> SB;
    const int m = 2 * (r & 3) + ((r >> 2) & 1) + 8 * ((r >> 3) & 1);
    return SB::FSEG * (m % (SB::SPR / SB::FSEG));
}
template <typename T, int KD, int NW>
__device__ __forceinline__ int tile_off(int r, int e) {
    typedef ScanBuf<T, KD, NW> SB;
    return r * SB::RB + ((e / SB::VN) ^ tile_mask<T, KD, NW>(r)) * 16 + (e % SB::VN) * SB::ES;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// gfx950 transposing LDS read (ds_read_b64_tr_b16): in each 16-lane group,
// result slot e of lane m is element m % 4 of the 8 bytes addressed by lane
// 4 e + m / 4 of the group.
__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

template <typename V>
__device__ __forceinline__ V ld(const unsigned char* p) { return *reinterpret_cast<const V*>(p); }

// Per-lane constants of the scan, computed once per workgroup.
template <typename T, int KD, int NW>
struct ScanLane {
    typedef ScanBuf<T, KD, NW> SB;
    static constexpr int KB = KD / 32;
    uint32_t tsrc[SB::tpw];       // K/Q source offset (bytes from the chunk's key block) per piece
    uint32_t vsrc[SB::v_pieces];  // value source offset per piece
    uint32_t rf[KB];              // K / Q fragment offset (row tile 0) per contraction block
    uint32_t tf[2][KB];           // K^T fragment offset (bf16) per tile parity and pair of state tiles
    uint32_t vtr;                 // value slab read in accumulator layout
    uint32_t oacc;                // output write into the value slab (accumulator layout)
};

template <typename T, int KD, int NW>
struct ScanArgs {
    const T* qp;
    const T* kp;
    int64_t qk_stride;
    const T* vp;
    int64_t v_stride;
    T* op;
    const unsigned char* ws_rec;
    int tok_begin, tok_end, nchunks, tile0, H, V, h, hk, c0, wave, lane;
    // chunk 0 of this unit: byte addresses of its K and Q key blocks, its value
    // columns (from the head's first column) and its record; bytes per row
    uint64_t k0, q0, v0, r0;
    uint32_t qk_row, v_row;
};

// Prefetch of later chunks into L2: the waves of a unit (nwu of them) split the
// 64-byte sectors of the unit's K, Q, value and record data, one dword per
// sector, loaded into a per-wave LDS scratch word that nothing reads. By the
// time a chunk is staged into LDS its data is on chip, which keeps far more of
// the sequence's HBM traffic in flight than the LDS ring can hold.
constexpr int kPrefetchSlots = 4;      // prefetch loads per wave per chunk
constexpr int kPrefetchAhead = 2;      // chunks beyond the furthest staged one

// Per-wave prefetch plan, fixed for the kernel: slot s reads sector lane of
// block `sub` of tensor sel (0 K, 1 Q, 2 values, 3 record, 4 none).
template <typename T, int KD, int NW>
struct PrefetchPlan {
    uint64_t base[kPrefetchSlots];     // chunk-0 address of the slot's tensor block
    uint64_t step[kPrefetchSlots];     // bytes from one chunk to the next
    uint32_t row[kPrefetchSlots];      // bytes per row (0: the record; ~0u: unused slot)
    uint32_t off[kPrefetchSlots];      // this lane's byte offset in the chunk's block
    __device__ __forceinline__ void init(const ScanArgs<T, KD, NW>& a, int wu, int nwu) {
        constexpr int ES = (int)sizeof(T);
        constexpr int kq_sh = __builtin_ctz(KD * ES / 64);     // log2 sectors per K/Q row
        constexpr int kq_spr = 1 << kq_sh;
        constexpr int rec_slots = (Rec<T>::bytes / 64 + kWave - 1) / kWave;
        // value rows: the unit's V * ES bytes, whole power-of-two sectors only
        const int v_spr0 = a.V * ES / 64;
        const int v_sh = v_spr0 > 0 ? 31 - __builtin_clz(v_spr0) : 0;
        const int v_spr = v_spr0 > 0 ? 1 << v_sh : 0;
#pragma unroll
        for (int i = 0; i < kPrefetchSlots; ++i) {
            const int j = wu + i * nwu;                        // slot (wave-uniform)
            const int t = j < kq_spr ? 0 : j < 2 * kq_spr ? 1 : j < 2 * kq_spr + v_spr ? 2
                        : j < 2 * kq_spr + v_spr + rec_slots ? 3 : 4;
            const int sub = j - (t == 0 ? 0 : t == 1 ? kq_spr : t == 2 ? 2 * kq_spr : 2 * kq_spr + v_spr);
            base[i] = t == 0 ? a.k0 : t == 1 ? a.q0 : t == 2 ? a.v0 : a.r0;
            step[i] = t <= 1 ? (uint64_t)kChunk * a.qk_row : t == 2 ? (uint64_t)kChunk * a.v_row
                                                                   : (uint64_t)a.H * Rec<T>::bytes;
            row[i] = t <= 1 ? a.qk_row : t == 2 ? a.v_row : t == 3 ? 0u : ~0u;
            const int sct = sub * kWave + a.lane;
            const int sh = t == 2 ? v_sh : kq_sh;
            off[i] = t >= 3 ? (uint32_t)sct * 64
                            : (uint32_t)(sct >> sh) * row[i] + (uint32_t)(sct & ((1 << sh) - 1)) * 64;
        }
    }
};

// Byte ranges of one chunk's K, Q, values and record; a chunk index past the
// sequence gets empty ranges, whose loads fetch nothing.
struct ChunkSpan {
    uint64_t k, q, v, r;
    uint32_t kq_bytes, v_bytes, r_bytes;
};

template <typename T, int KD, int NW>
__device__ __forceinline__ ChunkSpan chunk_span(int c, const ScanArgs<T, KD, NW>& a, int vcol) {
    constexpr int ES = (int)sizeof(T);
    const bool valid = c < a.nchunks;
    const int cc = valid ? c : 0;
    const int L = valid ? min(kChunk, a.tok_end - (a.tok_begin + c * kChunk)) : 0;
    ChunkSpan r;
    r.k = a.k0 + (uint64_t)cc * (kChunk * a.qk_row);
    r.q = a.q0 + (uint64_t)cc * (kChunk * a.qk_row);
    r.v = a.v0 + (uint64_t)cc * (kChunk * a.v_row) + vcol * ES;
    r.r = a.r0 + (uint64_t)cc * (uint32_t)(a.H * Rec<T>::bytes);
    r.kq_bytes = (uint32_t)L * a.qk_row;
    r.v_bytes = (uint32_t)L * a.v_row;
    r.r_bytes = valid ? (uint32_t)Rec<T>::bytes : 0u;
    return r;
}

struct ChunkRsrc {
    rsrc_t k, q, v, r;
};

// This wave's loads for one step of the pipeline: the direct-to-LDS copies of
// the chunk being staged into `nxt`, then its prefetch slots for a later
// chunk. issue<I>() issues load I; the chunk step calls them spread between
// its matrix ops, so the memory pipeline works while the wave computes.
template <typename T, int KD, int NW>
struct Stager {
    typedef ScanBuf<T, KD, NW> SB;
    static constexpr int count = SB::loads + kPrefetchSlots;
    ChunkRsrc st;                      // chunk being staged
    rsrc_t pf[kPrefetchSlots];         // prefetch resources
    const uint32_t* tsrc;
    const uint32_t* vsrc;
    const uint32_t* pfoff;
    int w, lane;

    __device__ __forceinline__ void init(int c_stage, int c_pref, const ScanLane<T, KD, NW>& ln,
                                         const PrefetchPlan<T, KD, NW>& plan,
                                         const ScanArgs<T, KD, NW>& a) {
        // (opaque copy of the wave index: keeps the per-piece LDS destinations
        // from being hoisted out of the chunk loop into spilled registers)
        w = a.wave;
        asm volatile("" : "+s"(w));
        lane = a.lane;
        tsrc = ln.tsrc;
        vsrc = ln.vsrc;
        pfoff = plan.off;
        const ChunkSpan sp = chunk_span<T, KD, NW>(c_stage, a, a.c0);
        st.k = make_rsrc((const void*)sp.k, sp.kq_bytes);
        st.q = make_rsrc((const void*)sp.q, sp.kq_bytes);
        st.v = make_rsrc((const void*)sp.v, sp.v_bytes);
        st.r = make_rsrc((const void*)sp.r, sp.r_bytes);
        const bool pvalid = c_pref < a.nchunks;
        const int pc = pvalid ? c_pref : 0;
        const uint32_t pL = pvalid ? (uint32_t)min(kChunk, a.tok_end - (a.tok_begin + c_pref * kChunk)) : 0u;
#pragma unroll
        for (int i = 0; i < kPrefetchSlots; ++i) {
            const uint32_t rb = plan.row[i];
            const uint32_t bytes = !pvalid || rb == ~0u ? 0u : rb == 0u ? (uint32_t)Rec<T>::bytes : pL * rb;
            pf[i] = make_rsrc((const void*)(plan.base[i] + (uint64_t)pc * plan.step[i]), bytes);
        }
    }
    // (the destination buffer and scratch word are arguments, so that the
    // caller's restrict-qualified pointers tell the compiler these copies
    // never touch the buffer being read)
    template <int I>
    __device__ __forceinline__ void issue(ScanBuf<T, KD, NW>* __restrict__ nxt,
                                          unsigned char* __restrict__ scratch) const {
        if constexpr (I < 2 * SB::tpw) {
            constexpr int j = I / 2;
            const int dst = (w + j * NW) * 1024;
            if constexpr (I % 2 == 0) dma16(st.k, nxt->k + dst, tsrc[j], 0);
            else dma16(st.q, nxt->q + dst, tsrc[j], 0);
        } else if constexpr (I < 2 * SB::tpw + SB::rpw) {
            constexpr int j = I - 2 * SB::tpw;
            const int pc = min(w + j * NW, SB::rec_pieces - 1);
            dma16(st.r, nxt->rec + pc * 1024, lane * 16, pc * 1024);
        } else if constexpr (I < SB::loads) {
            constexpr int p = I - 2 * SB::tpw - SB::rpw;
            dma16(st.v, nxt->v[w] + p * 1024, vsrc[p], 0);
        } else if constexpr (I < count) {
            constexpr int sl = I - SB::loads;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(pf[sl], (lds_ptr_t)scratch, 4, pfoff[sl], 0, 0, 0);
        }
    }
    // loads [B, E)
    template <int B, int E>
    __device__ __forceinline__ void issue_range(ScanBuf<T, KD, NW>* __restrict__ nxt,
                                                unsigned char* __restrict__ scratch) const {
        if constexpr (B < E && B < count) {
            issue<B>(nxt, scratch);
            issue_range<B + 1, E>(nxt, scratch);
        }
    }
    // share p of n of the loads
    template <int P, int N>
    __device__ __forceinline__ void issue_share(ScanBuf<T, KD, NW>* __restrict__ nxt,
                                                unsigned char* __restrict__ scratch) const {
        issue_range<P * count / N, (P + 1) * count / N>(nxt, scratch);
    }
};

// One chunk of the scan from the staged buffer `cur`: updates the state tiles
// hs and writes the chunk's outputs into this wave's value slab (row-major).
template <typename T, int KD, int NW>
__device__ __forceinline__ void scan_compute(ScanBuf<T, KD, NW>* __restrict__ cur,
                                             ScanBuf<T, KD, NW>* __restrict__ nxt,
                                             unsigned char* __restrict__ scratch,
                                             const Stager<T, KD, NW>& st, int nload,
                                             const ScanLane<T, KD, NW>& ln, int wave, int grp,
                                             int col, f32x4 (&hs)[KD / 16])
{
    // this step's loads (nload of them: the copies only, or copies and prefetches)
    if (nload == Stager<T, KD, NW>::count) st.template issue_range<0, Stager<T, KD, NW>::count>(nxt, scratch);
    else if (nload > 0) st.template issue_range<0, ScanBuf<T, KD, NW>::loads>(nxt, scratch);
    typedef Mma<T> MT;
    typedef typename MT::Frag Frag;
    typedef ScanBuf<T, KD, NW> SB;
    typedef Rec<T> RC;
    typedef ScanLane<T, KD, NW> LN;
    constexpr int ES = SB::ES;
    constexpr int KB = LN::KB;
    constexpr int RT = KD / 16;
    const int lane = 16 * grp + col;
    const unsigned char* kt = cur->k;
    const unsigned char* qt = cur->q;
    const unsigned char* rec = cur->rec;
    unsigned char* vs = cur->v[wave];

    // h as B operand (contraction over the key dim)
    Frag hf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) hf[kb] = state_frag<T>(hs[2 * kb], hs[2 * kb + 1], grp);

    // A fragment of a K/Q tile: rows 16 rt + col, key elements 32 kb + 8 grp .. + 7
    auto row_frag = [&](const unsigned char* tile, int rt, int kb) -> Frag {
        return ld<Frag>(tile + ln.rf[kb] + 16 * rt * SB::RB);
    };
    auto fac4 = [&](int which, int rt) -> f32x4 {
        return ld<f32x4>(rec + RC::fac + (which * kChunk + 16 * rt + 4 * grp) * 4);
    };
    auto rec_frag = [&](int region, int f) -> Frag {
        return ld<Frag>(rec + region + (f * kWave + lane) * RC::frag_bytes);
    };

    // values in accumulator layout
    f32x4 vv[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        if constexpr (ES == 2) {
            const s16x4 raw = lds_read_tr16(vs + ln.vtr + rt * 16 * SB::VRB);
            vv[rt] = __builtin_convertvector(__builtin_bit_cast(bf16x4, raw), f32x4);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) vv[rt][e] = ld<float>(vs + (16 * rt + 4 * grp + e) * SB::VRB + col * 4);
        }
    }

    // X = K h;  V' = V - a o X
    f32x4 X[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        X[rt] = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) X[rt] = MT::mma(row_frag(kt, rt, kb), hf[kb], X[rt]);
        X[rt] = vv[rt] - fac4(0, rt) * X[rt];
    }
    // U = T V'
    f32x4 U[4];
    {
        const Frag vf0 = MT::acc_frag(X[0], X[1]);
        const Frag vf1 = MT::acc_frag(X[2], X[3]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            U[rt] = MT::mma(rec_frag(RC::tfrag, tri_frag(rt, 0)), vf0, zero4());
            if (rt >= 2) U[rt] = MT::mma(rec_frag(RC::tfrag, tri_frag(rt, 1)), vf1, U[rt]);
        }
    }
    // O = b o (Q h) + P U, written row-major into the value slab (whose values
    // were read above)
    {
        const Frag uf0 = MT::acc_frag(U[0], U[1]);
        const Frag uf1 = MT::acc_frag(U[2], U[3]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 Y = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) Y = MT::mma(row_frag(qt, rt, kb), hf[kb], Y);
            f32x4 acc = MT::mma(rec_frag(RC::pfrag, tri_frag(rt, 0)), uf0, zero4());
            if (rt >= 2) acc = MT::mma(rec_frag(RC::pfrag, tri_frag(rt, 1)), uf1, acc);
            const f32x4 ov = acc + fac4(1, rt) * Y;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                *reinterpret_cast<T*>(vs + ln.oacc + (16 * rt + e) * SB::VRB) = from_f32<T>(ov[e]);
        }
    }
    // h' = gamma_L h + K^T (c o U)
    {
        const float gL = ld<float>(rec + RC::fac + 3 * kChunk * 4);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) U[rt] *= fac4(2, rt);
        const Frag df0 = MT::acc_frag(U[0], U[1]);
        const Frag df1 = MT::acc_frag(U[2], U[3]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            Frag k0, k1;
            if constexpr (ES == 2) {
                // A rows: key elements of state tile rt; contraction over the chunk rows
                const unsigned char* p = kt + ln.tf[rt & 1][rt >> 1];
                const s16x4 a = lds_read_tr16(p);
                const s16x4 b = lds_read_tr16(p + 16 * SB::RB);
                const s16x4 cc = lds_read_tr16(p + 32 * SB::RB);
                const s16x4 d = lds_read_tr16(p + 48 * SB::RB);
                k0 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
                k1 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(cc, d, 0, 1, 2, 3, 4, 5, 6, 7));
            } else {
                const int dd = state_row(rt, col >> 2, col & 3);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = slot_k(grp, j);
                    k0[j] = ld<float>(kt + tile_off<T, KD, NW>(t, dd));
                    k1[j] = ld<float>(kt + tile_off<T, KD, NW>(t + 32, dd));
                }
            }
            f32x4 acc = hs[rt] * gL;
            acc = MT::mma(k0, df0, acc);
            acc = MT::mma(k1, df1, acc);
            hs[rt] = acc;
        }
    }
}

// Compiler scheduling fence: nothing is moved across it, so the operand reads
// issued before a group of matrix ops stay ahead of it and their LDS latency
// is covered by the work in between.
#define SCAN_FENCE() __builtin_amdgcn_sched_barrier(0)

// bf16 chunk step with an explicit issue order: the LDS operands of each
// group of matrix ops are requested one or two groups ahead.
template <int KD, int NW>
__device__ __forceinline__ void scan_compute_bf16(ScanBuf<bf16, KD, NW>* __restrict__ cur,
                                                  ScanBuf<bf16, KD, NW>* __restrict__ nxt,
                                                  unsigned char* __restrict__ scratch,
                                                  const Stager<bf16, KD, NW>& st,
                                                  const ScanLane<bf16, KD, NW>& ln, int wave,
                                                  int grp, int col, f32x4 (&hs)[KD / 16])
{
    // The step's loads (copies of a later chunk into nxt, prefetches) are
    // issued in NP shares, one per group of matrix ops below.
    constexpr int NP = 11 + KD / 32;
    typedef Mma<bf16> MT;
    typedef bf16x8 Frag;
    typedef ScanBuf<bf16, KD, NW> SB;
    typedef Rec<bf16> RC;
    constexpr int KB = KD / 32;
    constexpr int RT = KD / 16;
    const int lane = 16 * grp + col;
    const unsigned char* kt = cur->k;
    const unsigned char* qt = cur->q;
    const unsigned char* rec = cur->rec;
    unsigned char* vs = cur->v[wave];

    // A operand of a K/Q tile: rows 16 rt + col, key elements 32 kb + 8 grp .. + 7
    auto row_frag = [&](const unsigned char* tile, int rt, int kb) -> Frag {
        return ld<Frag>(tile + ln.rf[kb] + 16 * rt * SB::RB);
    };
    auto fac4 = [&](int which, int rt) -> f32x4 {
        return ld<f32x4>(rec + RC::fac + (which * kChunk + 16 * rt + 4 * grp) * 4);
    };
    auto rec_frag = [&](int region, int f) -> Frag {
        return ld<Frag>(rec + region + (f * kWave + lane) * RC::frag_bytes);
    };
    // A operand of K^T: key rows of state tile rt, chunk rows 32 half .. + 31
    auto kt_frag = [&](int rt, int half) -> Frag {
        const unsigned char* p = kt + ln.tf[rt & 1][rt >> 1] + 32 * half * SB::RB;
        const s16x4 lo = lds_read_tr16(p);
        const s16x4 hi = lds_read_tr16(p + 16 * SB::RB);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // h as B operand (contraction over the key dim)
    Frag hf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) hf[kb] = state_frag<bf16>(hs[2 * kb], hs[2 * kb + 1], grp);

    // ---- X = K h and Y = Q h, one row tile at a time
    const float gL = ld<float>(rec + RC::fac + 3 * kChunk * 4);
    Frag kf[4][KB], qf[4][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kf[0][kb] = row_frag(kt, 0, kb);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qf[0][kb] = row_frag(qt, 0, kb);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kf[1][kb] = row_frag(kt, 1, kb);
    st.template issue_share<0, NP>(nxt, scratch);
    SCAN_FENCE();
    f32x4 X[4], Y[4], vv[4], f0[4];
    Frag tfr[kTriFrags], pfr[kTriFrags];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        X[rt] = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) X[rt] = MT::mma(kf[rt][kb], hf[kb], X[rt]);
        if (rt < 3) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) qf[rt + 1][kb] = row_frag(qt, rt + 1, kb);
        } else {
#pragma unroll
            for (int f = 0; f < kTriFrags; ++f) tfr[f] = rec_frag(RC::tfrag, f);
        }
        // decayed state, the accumulator of the update (tiles in step with rt)
#pragma unroll
        for (int i = 0; i < RT / 4; ++i) hs[(RT / 4) * rt + i] *= gL;
        if (rt == 0) st.template issue_share<1, NP>(nxt, scratch);
        if (rt == 1) st.template issue_share<3, NP>(nxt, scratch);
        if (rt == 2) st.template issue_share<5, NP>(nxt, scratch);
        if (rt == 3) st.template issue_share<7, NP>(nxt, scratch);
        SCAN_FENCE();
        Y[rt] = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) Y[rt] = MT::mma(qf[rt][kb], hf[kb], Y[rt]);
        if (rt < 2) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) kf[rt + 2][kb] = row_frag(kt, rt + 2, kb);
        } else if (rt == 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const s16x4 raw = lds_read_tr16(vs + ln.vtr + i * 16 * SB::VRB);
                vv[i] = __builtin_convertvector(__builtin_bit_cast(bf16x4, raw), f32x4);
                f0[i] = fac4(0, i);
            }
        } else {
#pragma unroll
            for (int f = 0; f < kTriFrags; ++f) pfr[f] = rec_frag(RC::pfrag, f);
        }
        if (rt == 0) st.template issue_share<2, NP>(nxt, scratch);
        if (rt == 1) st.template issue_share<4, NP>(nxt, scratch);
        if (rt == 2) st.template issue_share<6, NP>(nxt, scratch);
        if (rt == 3) st.template issue_share<8, NP>(nxt, scratch);
        SCAN_FENCE();
    }

    // ---- U = T (V - a o X)
    f32x4 f1[4], f2[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) f1[rt] = fac4(1, rt);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) X[rt] = vv[rt] - f0[rt] * X[rt];
    f32x4 U[4];
    {
        const Frag vf0 = MT::acc_frag(X[0], X[1]);
        const Frag vf1 = MT::acc_frag(X[2], X[3]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            U[rt] = MT::mma(tfr[tri_frag(rt, 0)], vf0, zero4());
            if (rt >= 2) U[rt] = MT::mma(tfr[tri_frag(rt, 1)], vf1, U[rt]);
        }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) f2[rt] = fac4(2, rt);
    Frag ktf[RT][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        ktf[rt][0] = kt_frag(rt, 0);
        ktf[rt][1] = kt_frag(rt, 1);
    }
    st.template issue_share<9, NP>(nxt, scratch);
    SCAN_FENCE();

    // ---- O = b o Y + P U (into the value slab, row-major) and h' = gamma_L h + K^T (c o U)
    f32x4 O[4];
    {
        const Frag uf0 = MT::acc_frag(U[0], U[1]);
        const Frag uf1 = MT::acc_frag(U[2], U[3]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            O[rt] = MT::mma(pfr[tri_frag(rt, 0)], uf0, zero4());
            if (rt >= 2) O[rt] = MT::mma(pfr[tri_frag(rt, 1)], uf1, O[rt]);
        }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) U[rt] *= f2[rt];
    const Frag df0 = MT::acc_frag(U[0], U[1]);
    const Frag df1 = MT::acc_frag(U[2], U[3]);
#pragma unroll
    for (int rt = 2; rt < (RT < 4 ? RT : 4); ++rt) {
        ktf[rt][0] = kt_frag(rt, 0);
        ktf[rt][1] = kt_frag(rt, 1);
    }
    st.template issue_share<10, NP>(nxt, scratch);
    SCAN_FENCE();
#pragma unroll
    for (int rt = 0; rt < RT; rt += 2) {
        // update two state tiles, then request the K^T operands two tiles ahead
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            hs[rt + i] = MT::mma(ktf[rt + i][0], df0, hs[rt + i]);
            hs[rt + i] = MT::mma(ktf[rt + i][1], df1, hs[rt + i]);
        }
        if (rt + 4 < RT) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                ktf[rt + 4 + i][0] = kt_frag(rt + 4 + i, 0);
                ktf[rt + 4 + i][1] = kt_frag(rt + 4 + i, 1);
            }
        }
        if (rt / 2 < 4) {
            // one output row tile per step, between the matrix ops
            const int ot = rt / 2;
            const f32x4 ov = O[ot] + f1[ot] * Y[ot];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                *reinterpret_cast<bf16*>(vs + ln.oacc + (16 * ot + e) * SB::VRB) = from_f32<bf16>(ov[e]);
        }
        if (rt == 0) st.template issue_share<11, NP>(nxt, scratch);
        if (rt == 2) st.template issue_share<12, NP>(nxt, scratch);
        if (rt == 4) st.template issue_share<13, NP>(nxt, scratch);
        if (rt == 6) st.template issue_share<14, NP>(nxt, scratch);
        SCAN_FENCE();
    }
    if constexpr (RT < 8) {
        // fewer state tiles than output tiles: write the remaining outputs
#pragma unroll
        for (int ot = RT / 2; ot < 4; ++ot) {
            const f32x4 ov = O[ot] + f1[ot] * Y[ot];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                *reinterpret_cast<bf16*>(vs + ln.oacc + (16 * ot + e) * SB::VRB) = from_f32<bf16>(ov[e]);
        }
    }
}

// Store chunk c's outputs, left row-major in this wave's slab of `buf`: lane r
// writes row r (rows past the end of the sequence fall outside the resource).
template <typename T, int KD, int NW>
__device__ __forceinline__ void scan_store(const ScanBuf<T, KD, NW>* __restrict__ buf, int c,
                                           const ScanArgs<T, KD, NW>& a)
{
    typedef ScanBuf<T, KD, NW> SB;
    constexpr int ES = SB::ES;
    const int tok0 = a.tok_begin + c * kChunk;
    const int L = min(kChunk, a.tok_end - tok0);
    const int64_t HV = (int64_t)a.H * a.V;
    const uint32_t o_row = (uint32_t)(HV * ES);
    const rsrc_t ro = make_rsrc(a.op + (int64_t)tok0 * HV + a.h * a.V + a.c0, (uint32_t)L * o_row);
    const unsigned char* src = buf->v[a.wave] + a.lane * SB::VRB;
#pragma unroll
    for (int s = 0; s < SB::VRB / 16; ++s) {
        const f32x4 d = ld<f32x4>(src + 16 * s);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, d), ro,
                                                   (uint32_t)a.lane * o_row + 16 * s, 0, 0);
    }
}

// s_waitcnt with only the vector-memory count bounded (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt and lgkmcnt at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS hand-off only. __syncthreads() also fences global
// memory, which costs a wait for every outstanding vector-memory operation,
// including the copies of chunks still meant to be in flight. Here the caller
// waits for exactly what it needs (wait_vmcnt), this wave's LDS accesses are
// drained, and the signal fences keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One workgroup per CU (its LDS buffers take most of the 160 KiB), one wave
// per SIMD: the compiler may spend registers on latency hiding.
template <typename T, int KD, int NW, int NBUF>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(1, 1))) void chunk_scan_kernel(
    const T* __restrict__ qp, const T* __restrict__ kp, int64_t qk_stride,
    const T* __restrict__ vp, int64_t v_stride,
    const float* __restrict__ S0, float* __restrict__ Sfin, T* __restrict__ o,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ offsets,
    const unsigned char* __restrict__ ws_rec,
    int T_len, int H, int Hk, int V, int units, int groups)
{
    typedef ScanBuf<T, KD, NW> SB;
    typedef ScanLane<T, KD, NW> LN;
    constexpr int ES = SB::ES;
    constexpr int RT = KD / 16;
    extern __shared__ __align__(1024) unsigned char smem_raw[];
    SB* bufs = reinterpret_cast<SB*>(smem_raw);

    // XCD-aware block order: all column groups of one (seq, head) unit get the
    // same blockIdx % 8, i.e. run on the same XCD and share its L2.
    const int bid = blockIdx.x;
    const int rest = bid >> 3;
    const int cgrp = rest % groups;
    const int u = (rest / groups) * 8 + (bid & 7);
    if (u >= units) return;
    const int seq = u / H;
    const int h = u - seq * H;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int grp = lane >> 4;
    const int col = lane & 15;

    ScanArgs<T, KD, NW> a;
    a.qp = qp; a.kp = kp; a.qk_stride = qk_stride; a.vp = vp; a.v_stride = v_stride; a.op = o;
    a.ws_rec = ws_rec; a.H = H; a.V = V; a.h = h; a.hk = h / (H / Hk); a.wave = wave; a.lane = lane;
    a.c0 = (cgrp * NW + wave) * 16;              // this wave's first value column
    if (cu) {
        a.tok_begin = cu[seq];
        a.tok_end = cu[seq + 1];
        a.tile0 = offsets[seq];
    } else {
        a.tok_begin = seq * T_len;
        a.tok_end = a.tok_begin + T_len;
        a.tile0 = seq * ((T_len + kChunk - 1) / kChunk);
    }
    const int nchunks = (a.tok_end - a.tok_begin + kChunk - 1) / kChunk;
    a.nchunks = nchunks;
    const int vc = a.c0 + col;                   // this lane's value column
    a.qk_row = (uint32_t)(qk_stride * ES);
    a.v_row = (uint32_t)(v_stride * ES);
    a.k0 = (uint64_t)(kp + (int64_t)a.tok_begin * qk_stride + a.hk * KD);
    a.q0 = (uint64_t)(qp + (int64_t)a.tok_begin * qk_stride + a.hk * KD);
    a.v0 = (uint64_t)(vp + (int64_t)a.tok_begin * v_stride + h * V);
    a.r0 = (uint64_t)(ws_rec + ((int64_t)a.tile0 * H + h) * Rec<T>::bytes);

    // ---- per-lane constants ----
    LN ln;
    const int64_t qk_row = qk_stride * ES;
#pragma unroll
    for (int j = 0; j < SB::tpw; ++j) {
        const int row = (wave + j * NW) * SB::RPI + lane / SB::SPR;   // row in the chunk
        const int s = (lane % SB::SPR) ^ tile_mask<T, KD, NW>(row);  // logical segment
        ln.tsrc[j] = (uint32_t)(row * qk_row + s * 16);
    }
#pragma unroll
    for (int p = 0; p < SB::v_pieces; ++p)
        ln.vsrc[p] = (uint32_t)((p * SB::RPV + lane / SB::LPR) * v_stride * ES + (lane % SB::LPR) * 16);
#pragma unroll
    for (int kb = 0; kb < LN::KB; ++kb) {
        ln.rf[kb] = (uint32_t)tile_off<T, KD, NW>(col, 32 * kb + 8 * grp);
        // transposing read: lane col of a group addresses chunk row 4 grp + col / 4
        // and the 4 key elements of A-operand rows 4 (col % 4) .. + 3
#pragma unroll
        for (int par = 0; par < 2; ++par)
            ln.tf[par][kb] = (uint32_t)tile_off<T, KD, NW>(4 * grp + (col >> 2), state_row(2 * kb + par, col & 3, 0));
    }
    ln.vtr = (uint32_t)((4 * grp + (col >> 2)) * SB::VRB + (col & 3) * 8);
    ln.oacc = (uint32_t)((4 * grp) * SB::VRB + col * ES);

    // ---- state ----
    f32x4 hs[RT];
    const int64_t sbase = ((int64_t)seq * H + h) * KD * V;
    if (S0) {   // (one branch around all loads, so they are issued together)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) hs[rt][e] = S0[sbase + (int64_t)state_row(rt, grp, e) * V + vc];
    } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) hs[rt] = zero4();
    }

    // A partial last chunk leaves the rows past the sequence unfetched: start
    // them at zero so they hold finite values (their factors are zero).
    if ((a.tok_end - a.tok_begin) % kChunk != 0) {
        const f32x4 z = zero4();
        for (int i = threadIdx.x * 16; i < NBUF * (int)sizeof(SB); i += NW * kWave * 16)
            *reinterpret_cast<f32x4*>(smem_raw + i) = z;
        lds_barrier();
    }

    typedef Stager<T, KD, NW> ST;
    if constexpr (NBUF >= 2) {
        // NBUF - 1 chunks are in flight into LDS while a chunk is computed, and
        // the kPrefetchAhead chunks after those are on their way into L2
        unsigned char* scratch = smem_raw + NBUF * sizeof(SB) + wave * 256;
        PrefetchPlan<T, KD, NW> plan;
        plan.init(a, cgrp * NW + wave, groups * NW);
        ST st;
#pragma unroll
        for (int i = 0; i < NBUF - 1; ++i) {
            st.init(i, 0, ln, plan, a);
            st.template issue_range<0, SB::loads>(&bufs[i], scratch);
        }
#pragma unroll
        for (int i = 0; i < kPrefetchAhead; ++i) {
            st.init(0, NBUF - 1 + i, ln, plan, a);
            st.template issue_range<SB::loads, ST::count>(&bufs[0], scratch);
        }
        // loads younger than chunk 0's copies: chunks 1 .. NBUF - 2, the prefetches
        wait_vmcnt<(NBUF - 2) * SB::loads + kPrefetchAhead * kPrefetchSlots>();
        lds_barrier();
        int b = 0;
        for (int c = 0; c < nchunks; ++c) {
            const int bp = b == 0 ? NBUF - 1 : b - 1;     // buffer of chunk c - 1 and c + NBUF - 1
            st.init(c + NBUF - 1, c + NBUF - 1 + kPrefetchAhead, ln, plan, a);
            if constexpr (ES == 2)
                scan_compute_bf16<KD, NW>(&bufs[b], &bufs[bp], scratch, st, ln, wave, grp, col, hs);
            else
                scan_compute<T, KD, NW>(&bufs[b], &bufs[bp], scratch, st, ST::count, ln, wave, grp, col, hs);
            // chunk c + 1 has landed. Loads issued after its copies: the
            // copies of chunks c + 2 .. c + NBUF - 1 and NBUF - 1 prefetches
            // (stores are not counted: they are never needed to complete here)
            wait_vmcnt<(NBUF - 2) * SB::loads + (NBUF - 1) * kPrefetchSlots>();
            scan_store<T, KD, NW>(&bufs[b], c, a);
            lds_barrier();
            b = b == NBUF - 1 ? 0 : b + 1;
        }
    } else {
        // one buffer: stage, wait, compute, in turn
        unsigned char* scratch = smem_raw + sizeof(SB) + wave * 256;
        PrefetchPlan<T, KD, NW> plan;
        plan.init(a, cgrp * NW + wave, groups * NW);
        ST st;
        st.init(0, 0, ln, plan, a);
        st.template issue_range<0, SB::loads>(&bufs[0], scratch);
        wait_vmcnt<0>();
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            scan_compute<T, KD, NW>(&bufs[0], &bufs[0] + 1, scratch, st, 0, ln, wave, grp, col, hs);
            scan_store<T, KD, NW>(&bufs[0], c, a);
            lds_barrier();   // every wave is done with the single buffer
            st.init(c + 1, 0, ln, plan, a);
            st.template issue_range<0, SB::loads>(&bufs[0], scratch);
            wait_vmcnt<0>();
            lds_barrier();
        }
    }
    wait_vmcnt<0>();   // no copy into LDS may outlive the workgroup

    if (Sfin) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Sfin[sbase + (int64_t)state_row(rt, grp, e) * V + vc] = hs[rt][e];
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
    const size_t rec = use_bf16 ? Rec<bf16>::bytes : Rec<float>::bytes;
    return align256(sizeof(int32_t) * (size_t)(n_seqs + 1)) + rec * (size_t)tiles * H;
}

template <typename K>
static hipError_t set_smem(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, int KD, int NW>
static hipError_t launch_scan(const void* q, const void* k, int64_t qks, const void* v, int64_t vs,
                              const float* S0, float* Sf, void* o, const int32_t* cu,
                              const int32_t* offsets, const unsigned char* wsrec, int T_len,
                              int H, int Hk, int V, int N, hipStream_t stream)
{
    const int units = N * H;
    const int groups = V / (16 * NW);
    const int upad = (units + 7) / 8 * 8;
    typedef ScanBuf<T, KD, NW> SB;
    // three buffers (two chunks in flight) where they fit in LDS and one
    // chunk's copies fit the 6-bit vector-memory counter
    constexpr int NBUF = 3 * sizeof(SB) + NW * 256 <= 160 * 1024 && SB::loads + 2 * kPrefetchSlots < 64 ? 3
                         : 2 * sizeof(SB) + NW * 256 <= 160 * 1024                                       ? 2
                                                                                                       : 1;
    const size_t smem = NBUF * sizeof(SB) + NW * 256;   // + the prefetch scratch words
    auto kern = chunk_scan_kernel<T, KD, NW, NBUF>;
    hipError_t err = set_smem(kern, smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3((unsigned)(upad * groups)), dim3(NW * kWave), smem, stream,
                       (const T*)q, (const T*)k, qks, (const T*)v, vs, S0, Sf, (T*)o, cu, offsets,
                       wsrec, T_len, H, Hk, V, units, groups);
    return hipGetLastError();
}

struct ChunkWs {
    int32_t* offsets;
    unsigned char* rec;
};

static inline ChunkWs carve(void* ws, int n_seqs) {
    ChunkWs w;
    w.offsets = (int32_t*)ws;
    w.rec = (unsigned char*)ws + align256(sizeof(int32_t) * (size_t)(n_seqs + 1));
    return w;
}

template <typename T, int KD>
static hipError_t launch_prepare_t(const void* q, const void* k, int64_t qks, const float* g,
                                   const float* beta, const int32_t* cu, int n_seqs, int B,
                                   int T_len, int H, int Hk, float scale, int l2norm, void* ws,
                                   hipStream_t stream)
{
    const bool packed = cu != nullptr;
    const int64_t tiles = tiles_upper_bound(B, T_len, n_seqs, packed);
    const ChunkWs w = carve(ws, n_seqs);
    if (packed) {
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(256), 0, stream, cu, n_seqs, w.offsets);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (tiles > 0) {
        const size_t smem = sizeof(PrepSmem<T, KD>);
        auto kern = chunk_prep_kernel<T, KD>;
        hipError_t e = set_smem(kern, smem);
        if (e != hipSuccess) return e;
        // persistent workgroups (as many as are resident at once), each walking
        // the (tile, key head) items
        const int64_t items = tiles * Hk;
        const int per_cu = kPrepWavesPerEU * 4 / (kPrepThreads / kWave);
        const int fit = (int)((160 * 1024) / smem);
        const int64_t cap = 256 * (int64_t)(fit < per_cu ? (fit > 0 ? fit : 1) : per_cu);
        const int grid = (int)(items < cap ? items : cap);
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kPrepThreads), smem, stream,
                           (const T*)q, (const T*)k, qks, g, beta, cu, w.offsets, n_seqs, T_len, H,
                           Hk, scale, l2norm, w.rec, (int)items);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T, int KD>
static hipError_t launch_scan_t(const void* q, const void* k, int64_t qks, const void* v,
                                int64_t vs, const float* S0, float* Sf, void* o, const int32_t* cu,
                                int n_seqs, int B, int T_len, int H, int Hk, int V, const void* ws,
                                hipStream_t stream)
{
    const int N = cu ? n_seqs : B;
    const ChunkWs w = carve(const_cast<void*>(ws), n_seqs);
    // columns per workgroup: enough workgroups to cover the 256 CUs, more waves
    // per workgroup (shared staging) when there is parallelism to spare
    const int units = N * H;
    const int slabs = V / 16;
    int nw = 1;
    if (units * (slabs / 4) >= 512 && slabs % 4 == 0) nw = 4;
    else if (units * (slabs / 2) >= 256 && slabs % 2 == 0) nw = 2;
    if (nw == 4)
        return launch_scan<T, KD, 4>(q, k, qks, v, vs, S0, Sf, o, cu, w.offsets, w.rec, T_len, H, Hk, V, N, stream);
    // the fp32 operand path (small parity workloads) runs with 1 or 4 waves per
    // workgroup only: its 2-wave instance does not get through the gfx950 backend
    if constexpr (sizeof(T) == 2) {
        if (nw == 2)
            return launch_scan<T, KD, 2>(q, k, qks, v, vs, S0, Sf, o, cu, w.offsets, w.rec, T_len, H, Hk, V, N, stream);
    }
    return launch_scan<T, KD, 1>(q, k, qks, v, vs, S0, Sf, o, cu, w.offsets, w.rec, T_len, H, Hk, V, N, stream);
}

hipError_t launch_chunk_prepare(const void* q, const void* k, int64_t qks, const float* g,
                                const float* beta, const int32_t* cu, int n_seqs, int B, int T_len,
                                int H, int Hk, int K, float scale, int l2norm, bool use_bf16,
                                void* ws, hipStream_t stream)
{
    if (use_bf16)
        return K == 128 ? launch_prepare_t<bf16, 128>(q, k, qks, g, beta, cu, n_seqs, B, T_len, H, Hk, scale, l2norm, ws, stream)
                        : launch_prepare_t<bf16, 64>(q, k, qks, g, beta, cu, n_seqs, B, T_len, H, Hk, scale, l2norm, ws, stream);
    return K == 128 ? launch_prepare_t<float, 128>(q, k, qks, g, beta, cu, n_seqs, B, T_len, H, Hk, scale, l2norm, ws, stream)
                    : launch_prepare_t<float, 64>(q, k, qks, g, beta, cu, n_seqs, B, T_len, H, Hk, scale, l2norm, ws, stream);
}

hipError_t launch_chunk_scan(const void* q, const void* k, int64_t qks, const void* v, int64_t vs,
                             const float* S0, float* Sf, void* o, const int32_t* cu, int n_seqs,
                             int B, int T_len, int H, int Hk, int K, int V, bool use_bf16,
                             const void* ws, hipStream_t stream)
{
    if (use_bf16)
        return K == 128 ? launch_scan_t<bf16, 128>(q, k, qks, v, vs, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, ws, stream)
                        : launch_scan_t<bf16, 64>(q, k, qks, v, vs, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, ws, stream);
    return K == 128 ? launch_scan_t<float, 128>(q, k, qks, v, vs, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, ws, stream)
                    : launch_scan_t<float, 64>(q, k, qks, v, vs, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, ws, stream);
}

}  // namespace gdn
