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
    T k[kChunk * ldk];         // raw k rows (rows >= L zero)
    T q[kChunk * ldk];         // raw q rows
    float a[kChunk * lda];     // A, strictly lower
    float n[kChunk * lda];     // N = (I + A)^-1, lower
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
            if (seg == 0) rnorm[row] = l2norm ? 1.f / sqrtf(ss + 1e-6f) : 1.f;
            *reinterpret_cast<typename V::type*>(dst + row * ld + seg * VN) = r;
        }
    }
};

template <typename T, int KD>
__global__ __launch_bounds__(kPrepThreads) void chunk_prep_kernel(
    const T* __restrict__ qp, const T* __restrict__ kp, int64_t qk_stride,
    const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ offsets, int n_seqs, int T_len,
    int H, int Hk, float scale, int l2norm, unsigned char* __restrict__ ws_rec)
{
    typedef Mma<T> MT;
    typedef PrepSmem<T, KD> SM;
    typedef Rec<T> RC;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    const int tile = blockIdx.x;
    const int hk = blockIdx.y;
    ChunkLoc loc;
    if (!locate_tile(tile, cu, offsets, n_seqs, T_len, loc)) return;
    const int L = loc.L;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int grp = lane >> 4;
    const int col = lane & 15;

    const int64_t rowoff = (int64_t)loc.tok0 * qk_stride + hk * KD;
    {
        RowTile<T, KD, kPrepThreads> kt, qt;
        kt.load(kp + rowoff, qk_stride, L);
        qt.load(qp + rowoff, qk_stride, L);
        kt.store(L, l2norm, sm.k, SM::ldk, sm.rk);
        qt.store(L, l2norm, sm.q, SM::ldk, sm.rq);
    }
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

    const int per = H / Hk;
    for (int hv = 0; hv < per; ++hv) {
        const int h = hk * per + hv;
        unsigned char* rec = ws_rec + ((int64_t)tile * H + h) * RC::bytes;
        if (wave == 0) {
            // G = inclusive cumsum of g over the chunk (rows >= L carry g = 0)
            const int lr = min(lane, L - 1);
            float gv = g[(int64_t)(loc.tok0 + lr) * H + h];
            float bv = beta[(int64_t)(loc.tok0 + lr) * H + h];
            if (lane >= L) { gv = 0.f; bv = 0.f; }
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                float up = __shfl_up(gv, d, kWave);
                if (lane >= d) gv += up;
            }
            sm.G[lane] = gv;
            sm.beta[lane] = bv;
            const float GL = __shfl(gv, kWave - 1, kWave);
            const bool live = lane < L;
            const float gam = __expf(gv);
            float* fac = reinterpret_cast<float*>(rec + RC::fac);
            fac[0 * kChunk + lane] = live ? gam * sm.rk[lane] : 0.f;
            fac[1 * kChunk + lane] = live ? scale * gam * sm.rq[lane] : 0.f;
            fac[2 * kChunk + lane] = live ? __expf(GL - gv) * sm.rk[lane] : 0.f;
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
            const float Gs = sm.G[s];
            const float rks = sm.rk[s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tri_row(tt) + 4 * grp + e;
                const float decay = __expf(fminf(sm.G[r] - Gs, 0.f));
                if (isA) {
                    sm.a[r * SM::lda + s] = (s < r) ? sm.beta[r] * decay * sm.rk[r] * rks * S[j][e] : 0.f;
                } else {
                    sm.p[r * SM::ldp + s] =
                        from_f32<T>((s <= r) ? scale * decay * sm.rq[r] * rks * S[j][e] : 0.f);
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

        // T = N diag(beta) and P as A-operand fragments: 12 fragments, 3 per wave
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int f = wave + 4 * j;
            const bool isT = f < kTriFrags;
            const int ff = isT ? f : f - kTriFrags;
            const int r = 16 * tri_frag_rt(ff) + col;
            const int kb = tri_frag_kb(ff);
            f32x8 v;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int c = 32 * kb + slot_k(grp, jj);
                float x = 0.f;
                if (c <= r) x = isT ? sm.n[r * SM::lda + c] * sm.beta[c] : to_f32(sm.p[r * SM::ldp + c]);
                v[jj] = x;
            }
            typename MT::Frag fr;
            if constexpr (sizeof(typename MT::Frag) == 16) fr = __builtin_convertvector(v, bf16x8);
            else fr = v;
            *reinterpret_cast<typename MT::Frag*>(rec + (isT ? RC::tfrag : RC::pfrag) +
                                                  (ff * kWave + lane) * RC::frag_bytes) = fr;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ chunk_scan

// LDS staging of one chunk for the scan: raw K and Q tiles (row-major, 16-byte
// segments XOR-swizzled by row so that fragment reads spread over the banks),
// the chunk's record, and each wave's 64 x 16 slab of values, all written by
// direct-to-LDS loads in 1 KiB pieces.
template <typename T, int KD, int NW>
struct ScanBuf {
    static constexpr int ES = (int)sizeof(T);
    static constexpr int VN = 16 / ES;                 // elements per 16-byte segment
    static constexpr int RB = KD * ES;                 // bytes per K/Q row
    static constexpr int SPR = RB / 16;                // segments per row
    static constexpr int RPI = 1024 / RB;              // rows per 1 KiB piece
    static constexpr int tile_pieces = kChunk * RB / 1024;
    static constexpr int rec_pieces = Rec<T>::bytes / 1024;
    static constexpr int shared_pieces = 2 * tile_pieces + rec_pieces;   // dealt over the waves
    static constexpr int VRB = 16 * ES;                // bytes per row of a wave's value slab
    static constexpr int LPR = VRB / 16;               // lanes per value row
    static constexpr int v_pieces = kChunk * VRB / 1024;
    static constexpr int RPV = kChunk / v_pieces;      // value rows per piece
    unsigned char k[kChunk * RB];
    unsigned char q[kChunk * RB];
    unsigned char rec[Rec<T>::bytes];
    unsigned char v[NW][kChunk * VRB];
};

template <typename T, int KD, int NW>
__device__ __forceinline__ int swz(int row, int seg) {
    typedef ScanBuf<T, KD, NW> SB;
    return row * SB::RB + ((seg ^ (row % SB::SPR)) << 4);
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
    static constexpr int RT = KD / 16;
    static constexpr int PPW = (SB::shared_pieces + NW - 1) / NW;
    static constexpr int RTP = SB::SPR > 16 ? 2 : 1;   // (16 rt + col) % SPR depends on rt only for SPR = 32
    uint32_t soff[PPW];           // staging source offsets (bytes) of this wave's shared pieces
    uint32_t voff[SB::v_pieces];  // staging source offsets of this wave's value pieces
    uint32_t rf[RTP][KB][2];      // K / Q fragment reads (row tile 0 / 1), per block and half
    uint32_t tf[RT];              // transposed K fragment reads (bf16), per state row tile
    uint32_t vtr;                 // value slab read in accumulator layout
    int vrow0;
};

template <typename T, int KD, int NW>
struct ScanArgs {
    const T* qp;
    const T* kp;
    int64_t qk_stride;
    const T* vp;
    int64_t v_stride;
    const unsigned char* ws_rec;
    int tok_begin, tok_end, tile0, H, h, wave, lane;
};

// Issue this wave's direct-to-LDS copies of chunk c into `nxt`. Rows past the
// end of a partial chunk re-read row L-1 (their factors are zero).
template <typename T, int KD, int NW>
__device__ __forceinline__ void scan_stage(ScanBuf<T, KD, NW>* __restrict__ nxt, int c,
                                           const ScanLane<T, KD, NW>& ln,
                                           const ScanArgs<T, KD, NW>& a)
{
    typedef ScanBuf<T, KD, NW> SB;
    typedef __attribute__((address_space(1))) const void* gptr;
    typedef __attribute__((address_space(3))) void* lptr;
    constexpr int ES = SB::ES;
    const int tok0 = a.tok_begin + c * kChunk;
    const int L = min(kChunk, a.tok_end - tok0);
    const int lastrow = L - 1;
    const unsigned char* kb8 = reinterpret_cast<const unsigned char*>(a.kp + (int64_t)tok0 * a.qk_stride);
    const unsigned char* qb8 = reinterpret_cast<const unsigned char*>(a.qp + (int64_t)tok0 * a.qk_stride);
    const unsigned char* rb8 = a.ws_rec + ((int64_t)(a.tile0 + c) * a.H + a.h) * Rec<T>::bytes;
    const unsigned char* vb8 = reinterpret_cast<const unsigned char*>(a.vp + (int64_t)tok0 * a.v_stride);
#pragma unroll
    for (int j = 0; j < ScanLane<T, KD, NW>::PPW; ++j) {
        const int piece = a.wave + j * NW;
        if (piece >= SB::shared_pieces) break;
        uint32_t off = ln.soff[j];
        const unsigned char* base;
        unsigned char* dst;
        if (piece < 2 * SB::tile_pieces) {
            const bool isq = piece >= SB::tile_pieces;
            const int pc = isq ? piece - SB::tile_pieces : piece;
            if (L < kChunk) {
                const int row = pc * SB::RPI + a.lane / SB::SPR;
                off -= (uint32_t)(max(row - lastrow, 0) * a.qk_stride * ES);
            }
            base = isq ? qb8 : kb8;
            dst = (isq ? nxt->q : nxt->k) + pc * 1024;
        } else {
            base = rb8;
            dst = nxt->rec + (piece - 2 * SB::tile_pieces) * 1024;
        }
        __builtin_amdgcn_global_load_lds((gptr)(base + off), (lptr)dst, 16, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < SB::v_pieces; ++p) {
        uint32_t off = ln.voff[p];
        if (L < kChunk) off -= (uint32_t)(max(p * SB::RPV + ln.vrow0 - lastrow, 0) * a.v_stride * ES);
        __builtin_amdgcn_global_load_lds((gptr)(vb8 + off), (lptr)(nxt->v[a.wave] + p * 1024), 16, 0, 0);
    }
}

// One chunk of the scan from the staged buffer `cur`: updates the state tiles
// hs and leaves the chunk's outputs (accumulator layout) in ov.
template <typename T, int KD, int NW>
__device__ __forceinline__ void scan_compute(const ScanBuf<T, KD, NW>* __restrict__ cur,
                                             const ScanLane<T, KD, NW>& ln, int wave, int grp,
                                             int col, f32x4 (&hs)[KD / 16], f32x4 (&ov)[4])
{
    typedef Mma<T> MT;
    typedef typename MT::Frag Frag;
    typedef ScanBuf<T, KD, NW> SB;
    typedef Rec<T> RC;
    typedef ScanLane<T, KD, NW> LN;
    constexpr int ES = SB::ES;
    constexpr int VN = SB::VN;
    constexpr int KB = LN::KB;
    constexpr int RT = LN::RT;
    constexpr int RTP = LN::RTP;
    const int lane = 16 * grp + col;
    const unsigned char* kt = cur->k;
    const unsigned char* qt = cur->q;
    const unsigned char* rec = cur->rec;
    const unsigned char* vs = cur->v[wave];

    // h as B operand (contraction over the key dim)
    Frag hf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) hf[kb] = MT::acc_frag(hs[2 * kb], hs[2 * kb + 1]);

    auto row_frag = [&](const unsigned char* tile, int rt, int kb) -> Frag {
        const int rtoff = (16 * rt - 16 * (rt % RTP)) * SB::RB;
        const unsigned char* p0 = tile + ln.rf[rt % RTP][kb][0] + rtoff;
        const unsigned char* p1 = tile + ln.rf[rt % RTP][kb][1] + rtoff;
        if constexpr (ES == 2) {
            const bf16x4 lo = ld<bf16x4>(p0), hi = ld<bf16x4>(p1);
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            const f32x4 lo = ld<f32x4>(p0), hi = ld<f32x4>(p1);
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
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
    // O = b o (Q h) + P U
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
            ov[rt] = acc + fac4(1, rt) * Y;
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
                const unsigned char* p = kt + ln.tf[rt];
                const s16x4 a = lds_read_tr16(p);
                const s16x4 b = lds_read_tr16(p + 16 * SB::RB);
                const s16x4 cc = lds_read_tr16(p + 32 * SB::RB);
                const s16x4 d = lds_read_tr16(p + 48 * SB::RB);
                k0 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
                k1 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(cc, d, 0, 1, 2, 3, 4, 5, 6, 7));
            } else {
                const int dd = 16 * rt + col;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = slot_k(grp, j);
                    k0[j] = ld<float>(kt + swz<T, KD, NW>(t, dd / VN) + (dd % VN) * 4);
                    k1[j] = ld<float>(kt + swz<T, KD, NW>(t + 32, dd / VN) + (dd % VN) * 4);
                }
            }
            f32x4 acc = hs[rt] * gL;
            acc = MT::mma(k0, df0, acc);
            acc = MT::mma(k1, df1, acc);
            hs[rt] = acc;
        }
    }
}

// Double-buffered step: the copies of chunk c + 1 into `nxt` are in flight
// while chunk c is computed from `cur` (the two never alias).
template <typename T, int KD, int NW>
__device__ __forceinline__ void scan_step(const ScanBuf<T, KD, NW>* __restrict__ cur,
                                          ScanBuf<T, KD, NW>* __restrict__ nxt, int c, bool more,
                                          const ScanLane<T, KD, NW>& ln,
                                          const ScanArgs<T, KD, NW>& a, int grp, int col,
                                          f32x4 (&hs)[KD / 16], f32x4 (&ov)[4])
{
    if (more) scan_stage<T, KD, NW>(nxt, c + 1, ln, a);
    scan_compute<T, KD, NW>(cur, ln, a.wave, grp, col, hs, ov);
}

template <typename T, int KD, int NW, int NBUF>
__global__ __launch_bounds__(NW * kWave) void chunk_scan_kernel(
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
    constexpr int VN = SB::VN;
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
    const int hk = h / (H / Hk);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int grp = lane >> 4;
    const int col = lane & 15;
    const int c0 = (cgrp * NW + wave) * 16;     // this wave's first value column
    const int vc = c0 + col;                    // this lane's value column

    ScanArgs<T, KD, NW> a;
    a.qp = qp; a.kp = kp; a.qk_stride = qk_stride; a.vp = vp; a.v_stride = v_stride;
    a.ws_rec = ws_rec; a.H = H; a.h = h; a.wave = wave; a.lane = lane;
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

    // ---- per-lane constants ----
    LN ln;
#pragma unroll
    for (int j = 0; j < LN::PPW; ++j) {
        const int piece = wave + j * NW;
        if (piece < 2 * SB::tile_pieces) {
            const int pc = piece % SB::tile_pieces;
            const int row = pc * SB::RPI + lane / SB::SPR;
            const int seg = (lane % SB::SPR) ^ (row % SB::SPR);
            ln.soff[j] = (uint32_t)(((int64_t)row * qk_stride + hk * KD + seg * VN) * ES);
        } else {
            ln.soff[j] = (uint32_t)((piece - 2 * SB::tile_pieces) * 1024 + lane * 16);
        }
    }
    ln.vrow0 = lane / SB::LPR;
#pragma unroll
    for (int p = 0; p < SB::v_pieces; ++p)
        ln.voff[p] = (uint32_t)(((int64_t)(p * SB::RPV + ln.vrow0) * v_stride + h * V + c0 +
                                 (lane % SB::LPR) * VN) * ES);
#pragma unroll
    for (int r = 0; r < LN::RTP; ++r)
#pragma unroll
        for (int kb = 0; kb < LN::KB; ++kb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int e0 = 32 * kb + 16 * hf + 4 * grp;
                ln.rf[r][kb][hf] = (uint32_t)(swz<T, KD, NW>(16 * r + col, e0 / VN) + (e0 % VN) * ES);
            }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int t0 = 4 * grp + (col >> 2);
        const int d0 = 16 * rt + 4 * (col & 3);
        ln.tf[rt] = (uint32_t)(swz<T, KD, NW>(t0, d0 / VN) + (d0 % VN) * 2);
    }
    ln.vtr = (uint32_t)((4 * grp + (col >> 2)) * SB::VRB + (col & 3) * 8);

    const uint32_t ooff = (uint32_t)((4 * grp) * H * V + h * V + vc);   // output lane offset
    const int64_t HV = (int64_t)H * V;
    auto store_o = [&](int c, const f32x4 (&ov)[4]) {
        const int tok0 = a.tok_begin + c * kChunk;
        const int L = min(kChunk, a.tok_end - tok0);
        T* ochunk = o + (int64_t)tok0 * HV;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                T* orow = ochunk + (16 * rt + e) * HV;     // uniform row base
                if (L == kChunk || 16 * rt + 4 * grp + e < L) orow[ooff] = from_f32<T>(ov[rt][e]);
            }
    };

    // ---- state: tile rt holds h[16 rt + 4 grp + e][vc] ----
    f32x4 hs[RT];
    const int64_t sbase = ((int64_t)seq * H + h) * KD * V;
    if (S0) {   // (one branch around all loads, so they are issued together)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) hs[rt][e] = S0[sbase + (int64_t)(16 * rt + 4 * grp + e) * V + vc];
    } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) hs[rt] = zero4();
    }

    if (nchunks > 0) scan_stage<T, KD, NW>(&bufs[0], 0, ln, a);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x4 ov[4];
    for (int c = 0; c < nchunks; ++c) {
        // the previous chunk's outputs go out first: their stores then have the
        // whole chunk to complete before the wait below
        if (c > 0) store_o(c - 1, ov);
        if constexpr (NBUF == 2) {
            scan_step<T, KD, NW>(&bufs[c & 1], &bufs[(c & 1) ^ 1], c, c + 1 < nchunks, ln, a, grp,
                                 col, hs, ov);
        } else {
            scan_compute<T, KD, NW>(&bufs[0], ln, wave, grp, col, hs, ov);
            if (c + 1 < nchunks) {
                __syncthreads();   // every wave is done with the single buffer
                scan_stage<T, KD, NW>(&bufs[0], c + 1, ln, a);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of the next chunk have landed
        __syncthreads();
    }
    if (nchunks > 0) store_o(nchunks - 1, ov);

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
    constexpr int NBUF = 2 * sizeof(ScanBuf<T, KD, NW>) <= 160 * 1024 ? 2 : 1;
    const size_t smem = NBUF * sizeof(ScanBuf<T, KD, NW>);
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
        hipLaunchKernelGGL(kern, dim3((unsigned)tiles, Hk), dim3(kPrepThreads), smem, stream,
                           (const T*)q, (const T*)k, qks, g, beta, cu, w.offsets, n_seqs, T_len, H,
                           Hk, scale, l2norm, w.rec);
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
