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
//   chunk_prep  one wave per (chunk, q/k head), every chunk in parallel:
//               K K^T and Q K^T on MFMA straight from the rows in registers
//               (shared by the value heads of a GQA group; the row norms are
//               their diagonals), then per value head the cumsum, A, the
//               64 x 64 unit-lower-triangular inverse (16 x 16 diagonal blocks
//               by forward substitution, off-diagonal blocks by block
//               substitution on fp32 MFMA), T, P and the factors a, b, c,
//               gamma_L. T and P are written as ready MFMA A-operand
//               fragments (only the 6 non-zero 16 x 32 blocks of each).
//   chunk_scan  one workgroup per (sequence, value head, group of value
//               columns), sequential over the sequence's chunks. The fp32
//               state of each 16-column tile stays in MFMA accumulators for the
//               whole sequence; accumulator tiles feed the next product
//               directly as B operands (see gdn_common.hpp), so the chain
//               h -> K h -> U -> h' never leaves registers. The raw K and Q
//               tiles, the values and the chunk's record are copied global ->
//               LDS with direct-to-LDS loads two chunks ahead (three buffers),
//               K^T operands are read from the row-major K tile with the gfx950
//               transposing LDS read, and nothing but the outputs and the
//               final state is written. bf16 operands with up to two column
//               tiles per workgroup take the role-split form below (chain,
//               output and copy waves on separate SIMDs); the fp32 operand
//               path and wide workgroups share one wave per column tile.
#include <utility>

#include "gdn_common.hpp"

namespace gdn {

constexpr int kLowerTiles = 10;     // 16 x 16 tiles on or below the diagonal of a 64 x 64 matrix
constexpr int kTriFrags = 6;        // non-zero 16 x 32 A-operand blocks of a lower-triangular 64 x 64

// A-operand block (row tile rt, 32-wide contraction block kb) of a lower-triangular matrix:
// (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
__device__ __forceinline__ int tri_frag(int rt, int kb) { return rt < 2 ? rt : 2 + 2 * (rt - 2) + kb; }

// Contraction index of operand slot j of lane group grp (see gdn_common.hpp).
__device__ __forceinline__ int slot_k(int grp, int j) { return j < 4 ? 4 * grp + j : 12 + 4 * grp + j; }

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

// offsets[i] = sum_{j < i} ceil(len_j / 64) for packed sequences (one block),
// and order[r] = the sequence of rank r by length, longest first (ties by
// index), so the whole-unit scan can start the longest sequences first;
// beyond kPlanSortMax sequences the order is the identity.
constexpr int kPlanSortMax = 1024;
__global__ __launch_bounds__(256) void chunk_plan_kernel(const int32_t* __restrict__ cu, int n,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ order)
{
    __shared__ int32_t buf[256];
    __shared__ int32_t carry_s;
    __shared__ int32_t len_s[kPlanSortMax];
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
    if (n > kPlanSortMax) {
        for (int i = threadIdx.x; i < n; i += 256) order[i] = i;
        return;
    }
    for (int i = threadIdx.x; i < n; i += 256) len_s[i] = cu[i + 1] - cu[i];
    __syncthreads();
    // rank of sequence i: the sequences longer than it, or as long with a smaller index
    for (int i = threadIdx.x; i < n; i += 256) {
        const int li = len_s[i];
        int r = 0;
        for (int j = 0; j < n; ++j) {
            const int lj = len_s[j];
            r += (lj > li) | ((lj == li) & (j < i));
        }
        order[r] = i;
    }
}

struct ChunkLoc {
    int tok0;     // first token row of the chunk
    int L;        // valid rows (1..64)
    bool first;   // the chunk starts its sequence
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
        loc.first = c == 0;
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
    loc.first = tile == offsets[lo];
    return true;
}

// ------------------------------------------------------------ chunk_prep
//
// One wave per (chunk, key head) item and nothing shared between waves, so
// no workgroup barriers: eight items are in flight per CU and each hides the
// others' memory latency. The raw K and Q rows go straight from global memory
// into MFMA operand registers; every later step works on 16 x 16 fp32 tiles
// held as MFMA accumulators. For such a tile M (lane l, c = l & 15,
// g = l >> 4, element e = 0..3) two layouts are used:
//     column layout C(M): lane holds M[4 g + e][c]   (what an MFMA yields)
//     row layout    R(M): lane holds M[c][4 g + e]   (= C(M^T))
// A 16 x 16 x 16 product D = X Y as four v_mfma_f32_16x16x4f32 steps, step s
// taking contraction index 4 g + s in every lane, reads X in R and Y in C and
// yields C(D). The record's A-operand fragments of T and P are R tiles in
// pairs, so the tiles are built in R: S = K K^T and Q K^T come out of the
// products already in R by feeding the K rows as the first operand.

// Per-wave LDS: the row vectors of the item and a scratch area for 16 x 16
// blocks (first the four diagonal blocks of -A and of N, then the six
// off-diagonal blocks of N on their way from C to R).
constexpr int kBlk = 272;     // diagonal block stride (floats): 256 + 16 keeps the 4 blocks on distinct banks
constexpr int kTrRow = 20;    // transpose staging: row stride and block stride (floats)
constexpr int kTrBlk = 320;
struct PrepLds {
    float G2[kChunk];          // log2(e) x inclusive cumsum of g (rows >= L: g taken as 0)
    float beta[kChunk];        // beta (rows >= L: 0)
    float rk[kChunk];          // 1 / |k_r| (1 without normalisation)
    float rq[kChunk];          // 1 / |q_r|
    float blk[8 * kBlk];
};
static_assert(6 * kTrBlk <= 8 * kBlk, "transpose staging fits the block scratch");

// Index of lower tile (i, j), j <= i, in row order, and of strictly-lower tile (i, j), j < i.
__host__ __device__ constexpr int low_t(int i, int j) { return i * (i + 1) / 2 + j; }
__host__ __device__ constexpr int off_t(int i, int j) { return i * (i - 1) / 2 + j; }

__device__ __forceinline__ float pick4(const f32x4& v, int e) {
    return e == 0 ? v[0] : (e == 1 ? v[1] : (e == 2 ? v[2] : v[3]));
}
// X (R layout) times Y (C layout) plus Z, 16 x 16 x 16 in fp32.
__device__ __forceinline__ f32x4 mma16(const f32x4& x, const f32x4& y, f32x4 z) {
#pragma unroll
    for (int s = 0; s < 4; ++s) z = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], y[s], z, 0, 0, 0);
    return z;
}
// This wave's LDS writes are complete (and the compiler keeps LDS accesses in
// program order around it); the wave's later LDS reads see them.
// 64 lanes x 16 bytes from rsrc + voffset (+ soffset) to LDS dst + 16 lane
// (an inactive lane neither loads nor writes)
__device__ __forceinline__ void dma16(rsrc_t r, unsigned char* dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void wave_lds_sync() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Operand fragment of one row: eight consecutive elements (any assignment of
// contraction indices to slots works as long as both operands share it, and
// both come from rows loaded the same way). Rows past the chunk lie outside
// the buffer resource and read as zero.
template <typename T> struct RowFrag;
template <> struct RowFrag<bf16> {
    static __device__ __forceinline__ bf16x8 load(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
};
template <> struct RowFrag<float> {
    static __device__ __forceinline__ f32x8 load(rsrc_t r, uint32_t off) {
        const f32x4 lo = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        const f32x4 hi = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

template <typename T>
__device__ __forceinline__ typename Mma<T>::Frag pack_frag(const f32x4& lo, const f32x4& hi) {
    const f32x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    if constexpr (sizeof(typename Mma<T>::Frag) == 16) return __builtin_convertvector(v, bf16x8);
    else return v;
}

// Forward substitution rows R.. of a unit-lower-triangular 16 x 16 solve
// (I + A) x = e_c, with -A's row r held in `arow` by lane r of the lane's
// 16-lane row: x[r] = [r == c] + sum_{s<r} (-A)[r][s] x[s].
template <int R>
__device__ __forceinline__ void subst_rows(const float (&arow)[16], float (&x)[16], int c) {
    if constexpr (R < 16) {
        float acc = R == c ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < R; ++s) acc += dpp_mov<kDppRowBcast + R>(arow[s]) * x[s];
        x[R] = acc;
        subst_rows<R + 1>(arow, x, c);
    }
}

// Inputs of the whole-prefill forms of chunk_prep. GATES: the gates are
// formed here from a and b (the same formulas as the gate kernel) instead of
// being read from g and beta. CONV (with GATES): qp / kp point at the raw q /
// k rows before the short convolution, which is applied here; the convolved
// rows go to `qk` for the scan, one contiguous block per (chunk, key head),
// so that every store covers whole cache lines.
struct PrepFused {
    const bf16* a;        // [token][head], row strides as / bs
    const bf16* b;
    int64_t as, bs;
    const float* A_log;
    const float* dt_bias;
    const bf16* wq;       // conv taps [channel][4] of q channel 0 of key head 0 (k: wk)
    const bf16* wk;
    const bf16* bq;       // conv bias of the same channels, or null
    const bf16* bk;
    unsigned char* qk;    // convolved rows out, in (chunk, key head) blocks:
                          // [q, k][32-column slice][64 rows][64 bytes]
};

// Bytes of one block of convolved q (or k) rows: 64 rows x KD bf16.
template <int KD>
constexpr uint32_t qk_block_bytes() { return (uint32_t)kChunk * KD * 2; }

// LDS staging of the CONV form: per 32-column slice of the raw rows (one
// contraction block), the three rows before the chunk and then its 64 rows
// (slot r + 3 for chunk row r), 64 bytes each, for k and for q, in two
// buffers (the next slice lands while this one is used); the taps and biases
// of the item's channels. It shares the wave's LDS with PrepLds, which is
// first used after the last slice. The four 16-byte segments of slot s are
// stored XOR-ed with (s / 4) % 4: 16 consecutive slots then cover every
// (bank group, segment) pair once, so the 16 lanes of a read that take one
// segment of 16 consecutive rows hit distinct banks.
template <int KD>
struct PrepStage {
    static constexpr int kRowB = 64;                    // bytes of a row's 32-column slice
    static constexpr int kSlice = (3 + kChunk) * kRowB;
    unsigned char rows[2][2][kSlice];                   // [buffer][k, q]
    unsigned char taps[2][KD * 4 * 2];                  // [k, q][channel][4 taps] bf16
    unsigned char bias[2][KD * 2];                      // [k, q][channel] bf16
};

__device__ __forceinline__ int stage_seg(int slot, int seg) { return seg ^ ((slot >> 2) & 3); }

template <int KD, bool CONV>
constexpr size_t prep_lds_bytes() {
    return CONV && sizeof(PrepStage<KD>) > sizeof(PrepLds) ? sizeof(PrepStage<KD>) : sizeof(PrepLds);
}

// Convolved rows of row tile i of one 32-column slice, from the staged rows
// `sl` (row r of the chunk at slot r + 3): lane (c, g) forms row 16 i + c,
// columns 8 g .. 8 g + 7 of the slice, with the slice's taps and biases at
// `tp` and `bp` (8 columns per lane group); rows at or past L are zero.
__device__ __forceinline__ bf16x8 conv_rows(const unsigned char* sl, const unsigned char* tp,
                                            const unsigned char* bp, int i, int c, int g, int L)
{
    typedef PrepStage<128> PS;   // (the row layout does not depend on KD)
    const int r = 16 * i + c;
    auto row = [&](int s) {   // segment g of slot s
        return *reinterpret_cast<const u32x4*>(sl + s * PS::kRowB + 16 * stage_seg(s, g));
    };
    const u32x4 x0 = row(r + 3);   // rows r, r - 1, r - 2, r - 3: two columns to a word
    const u32x4 x1 = row(r + 2);
    const u32x4 x2 = row(r + 1);
    const u32x4 x3 = row(r);
    const f32x8 bf = __builtin_convertvector(*reinterpret_cast<const bf16x8*>(bp + 16 * g), f32x8);
    uint32_t wp[16];   // column e: (w0, w1) in word 2 e, (w2, w3) in word 2 e + 1
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(tp + 64 * g + 16 * j);
#pragma unroll
        for (int d = 0; d < 4; ++d) wp[4 * j + d] = u[d];
    }
    f32x8 out;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float a0 = conv_taps4_bf16(wp[4 * d], wp[4 * d + 1], bf[2 * d],
                                         pair_lo(x3[d], x2[d]), pair_lo(x1[d], x0[d]));
        const float a1 = conv_taps4_bf16(wp[4 * d + 2], wp[4 * d + 3], bf[2 * d + 1],
                                         pair_hi(x3[d], x2[d]), pair_hi(x1[d], x0[d]));
        out[2 * d] = r < L ? conv_silu(a0) : 0.f;
        out[2 * d + 1] = r < L ? conv_silu(a1) : 0.f;
    }
    return __builtin_convertvector(out, bf16x8);
}

// Two waves per SIMD: registers sized for it.
template <typename T, int KD, bool GATES, bool CONV>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2)))
void chunk_prep_kernel(
    const T* __restrict__ qp, const T* __restrict__ kp, int64_t qk_stride,
    const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ offsets, int n_seqs, int T_len,
    int H, int Hk, float scale, int l2norm, unsigned char* __restrict__ ws_rec, int n_items,
    PrepFused gz)
{
    static_assert(!GATES || sizeof(T) == 2, "the whole-prefill forms run on bf16 rows");
    static_assert(!CONV || GATES, "the convolving form also forms the gates");
    typedef Mma<T> MT;
    typedef typename MT::Frag Frag;
    typedef Rec<T> RC;
    constexpr int ES = (int)sizeof(T);
    __shared__ __align__(16) unsigned char smem_raw[prep_lds_bytes<KD, CONV>()];
    PrepLds& sm = *reinterpret_cast<PrepLds*>(smem_raw);

    // XCD-aware order: the key heads of one tile run on the same XCD (blockIdx
    // % 8) one after another, so the tile's gate rows are fetched into that
    // XCD's L2 once
    const int bx = blockIdx.x >> 3;
    const int tile = (bx / Hk) * 8 + (blockIdx.x & 7);
    const int hk = bx - (bx / Hk) * Hk;
    const int it = tile * Hk + hk;
    if (it >= n_items) return;
    ChunkLoc loc;
    if (!locate_tile(tile, cu, offsets, n_seqs, T_len, loc)) return;   // packed: past the last chunk
    const int L = loc.L;
    const int per = H / Hk;
    const int lane = threadIdx.x;
    const int c = lane & 15;
    const int gq = lane >> 4;
    const bool live = lane < L;
    const int lr = min(lane, L - 1);
    const uint32_t row_bytes = (uint32_t)(qk_stride * ES);

    // gate values of value head h (lane = row): read (given, or a and b), then
    // formed from a and b in the whole-prefill forms
    auto gate_in = [&](int h, float& gv, float& bv) {
        const int64_t row = loc.tok0 + lr;
        if constexpr (GATES) {
            gv = to_f32(gz.a[row * gz.as + h]);
            bv = to_f32(gz.b[row * gz.bs + h]);
        } else {
            gv = g[row * H + h];
            bv = beta[row * H + h];
        }
    };
    auto gate_form = [&](int h, float& gv, float& bv) {
        if constexpr (GATES) {
            gv = gate_g(gv, gz.A_log[h], gz.dt_bias[h]);
            bv = gate_beta(bv);
        }
    };
    auto gate_of = [&](int h, float& gv, float& bv) {
        gate_in(h, gv, bv);
        gate_form(h, gv, bv);
    };
    // those of the first value head, requested before the rows (after the
    // staging copies in the convolving form, formed once the rows are used)
    float gh = 0.f, bh = 0.f;
    if constexpr (!CONV) gate_of(hk * per, gh, bh);

    // ---- S = K K^T and Q K^T (lower tiles, R layout), diagonal tiles of Q Q^T
    const int64_t base = (int64_t)loc.tok0 * qk_stride + (int64_t)hk * KD;
    const uint32_t span = (uint32_t)(L - 1) * row_bytes + KD * ES;
    const rsrc_t rsk = make_rsrc(kp + base, span);
    const rsrc_t rsq = make_rsrc(qp + base, span);
    f32x4 skk[kLowerTiles], sqk[kLowerTiles], sqq[4];
#pragma unroll
    for (int t = 0; t < kLowerTiles; ++t) { skk[t] = zero4(); sqk[t] = zero4(); }
#pragma unroll
    for (int i = 0; i < 4; ++i) sqq[i] = zero4();
    // CONV: staging of the raw rows (three before the chunk, none at a sequence
    // start, where the taps read zero), taps, biases, and the convolved rows'
    // destination
    PrepStage<KD>* stg = reinterpret_cast<PrepStage<KD>*>(smem_raw);
    rsrc_t rhk = rsk, rhq = rsq, rok = rsk, roq = rsk;
    // lane l lands at position l % 4 of slot l / 4 (+ the piece's first slot),
    // so it fetches the segment stored there
    auto stage_slice = [&](int kb, int buf) {
        const uint32_t col = (uint32_t)(64 * kb);
        if (lane < 12) {
            const int slot = lane >> 2;
            const uint32_t off = (uint32_t)slot * row_bytes + col + 16 * stage_seg(slot, lane & 3);
            dma16(rhk, stg->rows[buf][0], off, 0);
            dma16(rhq, stg->rows[buf][1], off, 0);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = 16 * p + (lane >> 2);
            const uint32_t off = (uint32_t)r * row_bytes + col + 16 * stage_seg(r + 3, lane & 3);
            dma16(rsk, stg->rows[buf][0] + 3 * PrepStage<KD>::kRowB + 1024 * p, off, 0);
            dma16(rsq, stg->rows[buf][1] + 3 * PrepStage<KD>::kRowB + 1024 * p, off, 0);
        }
    };
    constexpr int kSliceLoads = 2 + 2 * 4;   // copies per slice (k, q: halo + four pieces)
    constexpr int kStores = 8;               // convolved-row stores per slice
    if constexpr (CONV) {
        const uint32_t hspan = loc.first ? 0u : 2 * row_bytes + KD * ES;
        rhk = make_rsrc(kp + base - 3 * qk_stride, hspan);
        rhq = make_rsrc(qp + base - 3 * qk_stride, hspan);
        constexpr uint32_t tb = qk_block_bytes<KD>();
        unsigned char* blk = gz.qk + ((int64_t)tile * Hk + hk) * 2 * tb;
        roq = make_rsrc(blk, tb);
        rok = make_rsrc(blk + tb, tb);
        // taps and biases of the item's channels (no bias: zero-length, read as zero)
        const int64_t ch = (int64_t)hk * KD;
        constexpr int tl = KD * 8 / 16, bl = KD * 2 / 16;   // lanes of 16 bytes
        if (lane < tl) {
            dma16(make_rsrc(gz.wk + ch * 4, KD * 8), stg->taps[0], lane * 16, 0);
            dma16(make_rsrc(gz.wq + ch * 4, KD * 8), stg->taps[1], lane * 16, 0);
        }
        if (lane < bl) {
            dma16(make_rsrc(gz.bk ? gz.bk + ch : gz.wk, gz.bk ? KD * 2 : 0), stg->bias[0], lane * 16, 0);
            dma16(make_rsrc(gz.bq ? gz.bq + ch : gz.wq, gz.bq ? KD * 2 : 0), stg->bias[1], lane * 16, 0);
        }
        stage_slice(0, 0);
        stage_slice(1, 1);
        gate_in(hk * per, gh, bh);
    }
    // bf16 rows read from q and k: every fragment of the item is requested
    // before the first product, so the loads overlap one another instead of
    // waiting slice by slice (fp32 rows would not fit in registers)
    constexpr bool kAhead = !CONV && sizeof(T) == 2;
    Frag kall[kAhead ? KD / 32 : 1][4], qall[kAhead ? KD / 32 : 1][4];
    if constexpr (kAhead) {
#pragma unroll
        for (int kb = 0; kb < KD / 32; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t off = (uint32_t)(16 * i + c) * row_bytes + (32 * kb + 8 * gq) * ES;
                kall[kb][i] = RowFrag<T>::load(rsk, off);
                qall[kb][i] = RowFrag<T>::load(rsq, off);
            }
        __builtin_amdgcn_sched_barrier(0);   // keep them ahead of the products
    }
#pragma unroll
    for (int kb = 0; kb < KD / 32; ++kb) {
        Frag kf[4], qf[4];
        if constexpr (CONV) {
            // slice kb has landed once only younger accesses are outstanding: at
            // kb 0 slice 1's copies and the two gate-input loads, later the
            // previous slice's stores (the counter retires in issue order)
            static_assert(KD / 32 > 1, "two slices at least");
            if (kb == 0) wait_vmcnt<kSliceLoads + 2>();
            else wait_vmcnt<kStores>();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (kb >= 1 && kb + 1 < KD / 32) {
                stage_slice(kb + 1, (kb + 1) & 1);   // its buffer was read by slice kb - 1
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
            }
            const unsigned char* sk = stg->rows[kb & 1][0];
            const unsigned char* sq = stg->rows[kb & 1][1];
            const int cb = 32 * kb;   // first channel of the slice within the head
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kf[i] = conv_rows(sk, stg->taps[0] + cb * 8, stg->bias[0] + cb * 2, i, c, gq, L);
                qf[i] = conv_rows(sq, stg->taps[1] + cb * 8, stg->bias[1] + cb * 2, i, c, gq, L);
            }
            wave_lds_sync();   // this slice's rows are read: its buffer may be refilled
            // (one store: 16 whole rows of the slice, 1 KiB contiguous; rows past
            // the chunk are written as zero)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t off = (uint32_t)(kChunk * 64 * kb + 64 * (16 * i + c) + 16 * gq);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, kf[i]), rok, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, qf[i]), roq, off, 0, 0);
            }
        } else if constexpr (kAhead) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kf[i] = kall[kb][i];
                qf[i] = qall[kb][i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t off = (uint32_t)(16 * i + c) * row_bytes + (32 * kb + 8 * gq) * ES;
                kf[i] = RowFrag<T>::load(rsk, off);
                qf[i] = RowFrag<T>::load(rsq, off);
            }
        }
        // C(K_j X_i^T) = R(X_i K_j^T): tile (i, j) of S with the K rows first
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j <= i; ++j) {
                skk[low_t(i, j)] = MT::mma(kf[j], kf[i], skk[low_t(i, j)]);
                sqk[low_t(i, j)] = MT::mma(kf[j], qf[i], sqk[low_t(i, j)]);
            }
            sqq[i] = MT::mma(qf[i], qf[i], sqq[i]);
        }
    }
    if constexpr (CONV) gate_form(hk * per, gh, bh);
    // row norms from the diagonals: element c & 3 of the lanes with g == c / 4
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float kk = pick4(skk[low_t(i, i)], c & 3);
        const float qq = pick4(sqq[i], c & 3);
        if (gq == (c >> 2)) {   // (v_rsq_f32, ~1 ulp)
            sm.rk[16 * i + c] = l2norm ? __builtin_amdgcn_rsqf(kk + 1e-6f) : 1.f;
            sm.rq[16 * i + c] = l2norm ? __builtin_amdgcn_rsqf(qq + 1e-6f) : 1.f;
        }
    }

    for (int hv = 0; hv < per; ++hv) {
        const int h = hk * per + hv;
        unsigned char* rec = ws_rec + ((int64_t)tile * H + h) * RC::bytes;
        if (hv > 0) gate_of(h, gh, bh);
        // ---- cumsum and the per-row factors (lane = row)
        const float G2 = wave_inclusive_scan(live ? gh : 0.f) * kLog2e;
        const float GL2 = lane_value(G2, kWave - 1);
        sm.G2[lane] = G2;
        sm.beta[lane] = live ? bh : 0.f;
        wave_lds_sync();   // (also orders the norms written above)
        {
            const float rkl = sm.rk[lane];
            const float gam = __builtin_amdgcn_exp2f(G2);
            float* fac = reinterpret_cast<float*>(rec + RC::fac);
            fac[0 * kChunk + lane] = live ? gam * rkl : 0.f;
            fac[1 * kChunk + lane] = live ? scale * gam * sm.rq[lane] : 0.f;
            fac[2 * kChunk + lane] = live ? __builtin_amdgcn_exp2f(GL2 - G2) * rkl : 0.f;
            fac[3 * kChunk + lane] = __builtin_amdgcn_exp2f(GL2);
        }

        // ---- -A (strictly lower) and P (lower), R layout, row r = 16 i + c and
        // column s = 16 j + 4 g + e. The decay exp(G_r - G_s) is shared by both;
        // its exponent is zeroed above the diagonal before exponentiating.
        f32x4 aR[6];    // R(-A_ij), i > j
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * i + c;
            const float Gr = sm.G2[r];
            const float fa = -sm.beta[r] * sm.rk[r];
            const float fp = scale * sm.rq[r];
            f32x4 pt[4];
#pragma unroll
            for (int j = 0; j <= i; ++j) {
                const f32x4 Gs = *reinterpret_cast<const f32x4*>(&sm.G2[16 * j + 4 * gq]);
                const f32x4 ks = *reinterpret_cast<const f32x4*>(&sm.rk[16 * j + 4 * gq]);
                const int t = low_t(i, j);
                f32x4 a, p;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x = Gr - Gs[e];
                    if (i == j) x = (4 * gq + e <= c) ? x : 0.f;
                    const float w = ks[e] * __builtin_amdgcn_exp2f(x);
                    a[e] = fa * w * skk[t][e];
                    p[e] = fp * w * sqk[t][e];
                    if (i == j) {
                        a[e] = (4 * gq + e < c) ? a[e] : 0.f;
                        p[e] = (4 * gq + e <= c) ? p[e] : 0.f;
                    }
                }
                pt[j] = p;
                if (i == j) *reinterpret_cast<f32x4*>(&sm.blk[kBlk * i + 16 * c + 4 * gq]) = a;
                else aR[off_t(i, j)] = a;
            }
            // P fragments of row tile i: (tile 2 kb, tile 2 kb + 1), zero above the diagonal
#pragma unroll
            for (int kb = 0; 2 * kb <= i; ++kb) {
                const f32x4 lo = pt[2 * kb];
                const f32x4 hi = 2 * kb + 1 <= i ? pt[2 * kb + 1] : zero4();
                const int f = tri_frag(i, kb);
                *reinterpret_cast<Frag*>(rec + RC::pfrag + (f * kWave + lane) * RC::frag_bytes) =
                    pack_frag<T>(lo, hi);
            }
        }
        wave_lds_sync();

        // ---- diagonal blocks of N = (I + A)^-1 by forward substitution: lane
        // (c, g) holds row c of -A_gg and solves column c of block g; the
        // entry -A_gg[r][s] comes from lane r of the same 16-lane row
        {
            float arow[16], x[16];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const f32x4 av = *reinterpret_cast<const f32x4*>(sm.blk + kBlk * gq + 16 * c + 4 * s4);
#pragma unroll
                for (int e = 0; e < 4; ++e) arow[4 * s4 + e] = av[e];
            }
            subst_rows<0>(arow, x, c);
            float* Nb = sm.blk + 4 * kBlk + kBlk * gq;
#pragma unroll
            for (int r = 0; r < 16; ++r) Nb[16 * r + c] = x[r];
        }
        wave_lds_sync();
        f32x4 Rd[4], Od[4];   // R(N_ii), C(N_ii)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float* Nb = sm.blk + 4 * kBlk + kBlk * i;
            Rd[i] = *reinterpret_cast<const f32x4*>(Nb + 16 * c + 4 * gq);
#pragma unroll
            for (int e = 0; e < 4; ++e) Od[i][e] = Nb[16 * (4 * gq + e) + c];
        }

        // ---- off-diagonal blocks by block rows: N_iw = N_ii sum_{k=w}^{i-1} (-A_ik) N_kw
        f32x4 nO[6];    // C(N_iw), i > w
#pragma unroll
        for (int i = 1; i < 4; ++i) {
#pragma unroll
            for (int w = 0; w < i; ++w) {
                f32x4 X = zero4();
#pragma unroll
                for (int k = w; k < i; ++k) X = mma16(aR[off_t(i, k)], k == w ? Od[w] : nO[off_t(k, w)], X);
                nO[off_t(i, w)] = mma16(Rd[i], X, zero4());
            }
        }
        // C -> R through LDS (the diagonal blocks are no longer read)
#pragma unroll
        for (int b = 0; b < 6; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.blk[kTrBlk * b + kTrRow * (4 * gq + e) + c] = nO[b][e];
        wave_lds_sync();

        // ---- T = N diag(beta) fragments: (tile 2 kb, tile 2 kb + 1) of row tile i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 tt[4];
#pragma unroll
            for (int j = 0; j <= i; ++j) {
                const f32x4 bs = *reinterpret_cast<const f32x4*>(&sm.beta[16 * j + 4 * gq]);
                const f32x4 n = i == j ? Rd[i]
                                       : *reinterpret_cast<const f32x4*>(&sm.blk[kTrBlk * off_t(i, j) + kTrRow * c + 4 * gq]);
                tt[j] = n * bs;
            }
#pragma unroll
            for (int kb = 0; 2 * kb <= i; ++kb) {
                const f32x4 lo = tt[2 * kb];
                const f32x4 hi = 2 * kb + 1 <= i ? tt[2 * kb + 1] : zero4();
                const int f = tri_frag(i, kb);
                *reinterpret_cast<Frag*>(rec + RC::tfrag + (f * kWave + lane) * RC::frag_bytes) =
                    pack_frag<T>(lo, hi);
            }
        }
        wave_lds_sync();   // the next head rewrites the scratch
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


// The same B operand, built by converting each tile to bf16 first and then
// swapping whole dwords in groups 2 and 3 (4 selects per operand instead of 8);
// identical bits.
__device__ __forceinline__ bf16x8 state_frag_bf16(const f32x4& t0, const f32x4& t1, int grp) {
    const u32x2 a = __builtin_bit_cast(u32x2, __builtin_convertvector(t0, bf16x4));
    const u32x2 b = __builtin_bit_cast(u32x2, __builtin_convertvector(t1, bf16x4));
    const bool sw = grp >= 2;
    u32x4 r;
    r[0] = sw ? b[0] : a[0];
    r[1] = sw ? b[1] : a[1];
    r[2] = sw ? a[0] : b[0];
    r[3] = sw ? a[1] : b[1];
    return __builtin_bit_cast(bf16x8, r);
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
    // blocked K / Q (whole-prefill form): bytes of one chunk's block (0: rows
    // of qk_row bytes instead) and from one chunk's blocks to the next's
    uint32_t qk_blk;
    uint64_t kq_step;
};

// Prefetch of later chunks into L2: the waves of a unit (nwu of them) split the
// 64-byte sectors of the unit's K, Q, value and record data, one dword per
// sector, loaded into a per-wave LDS scratch word that nothing reads. By the
// time a chunk is staged into LDS its data is on chip, which keeps far more of
// the sequence's HBM traffic in flight than the LDS ring can hold.
constexpr int kPrefetchSlots = 2;      // prefetch loads per wave per chunk
constexpr int kPfSector = 128;         // bytes per prefetch touch (one L2 line)
constexpr int kPrefetchAhead = 2;      // chunks beyond the furthest staged one

// Per-wave prefetch plan, fixed for the kernel: slot s reads sector lane of
// block `sub` of tensor sel (0 K, 1 Q, 2 values, 3 record, 4 none).
template <typename T, int KD, int NW>
struct PrefetchPlan {
    uint64_t base[kPrefetchSlots];     // chunk-0 address of the slot's tensor block
    uint64_t step[kPrefetchSlots];     // bytes from one chunk to the next
    uint32_t row[kPrefetchSlots];      // bytes per row (0: one contiguous block; ~0u: unused slot)
    uint32_t blk[kPrefetchSlots];      // bytes of a contiguous block
    uint32_t off[kPrefetchSlots];      // this lane's byte offset in the chunk's block
    __device__ __forceinline__ void init(const ScanArgs<T, KD, NW>& a, int wu, int nwu) {
        constexpr int ES = (int)sizeof(T);
        constexpr int kq_sh = __builtin_ctz(KD * ES / kPfSector);     // log2 sectors per K/Q row
        constexpr int kq_spr = 1 << kq_sh;
        constexpr int rec_slots = (Rec<T>::bytes / kPfSector + kWave - 1) / kWave;
        // value rows: the unit's V * ES bytes, whole power-of-two sectors only
        const int v_spr0 = a.V * ES / kPfSector;
        const int v_sh = v_spr0 > 0 ? 31 - __builtin_clz(v_spr0) : 0;
        const int v_spr = v_spr0 > 0 ? 1 << v_sh : 0;
#pragma unroll
        for (int i = 0; i < kPrefetchSlots; ++i) {
            const int j = wu + i * nwu;                        // slot (wave-uniform)
            const int t = j < kq_spr ? 0 : j < 2 * kq_spr ? 1 : j < 2 * kq_spr + v_spr ? 2
                        : j < 2 * kq_spr + v_spr + rec_slots ? 3 : 4;
            const int sub = j - (t == 0 ? 0 : t == 1 ? kq_spr : t == 2 ? 2 * kq_spr : 2 * kq_spr + v_spr);
            // (a chunk's blocked K or Q is as many sectors as its rows)
            const bool kq_blk = t <= 1 && a.qk_blk != 0;
            base[i] = t == 0 ? a.k0 : t == 1 ? a.q0 : t == 2 ? a.v0 : a.r0;
            step[i] = t <= 1 ? (kq_blk ? a.kq_step : (uint64_t)kChunk * a.qk_row)
                             : t == 2 ? (uint64_t)kChunk * a.v_row : (uint64_t)a.H * Rec<T>::bytes;
            row[i] = kq_blk ? 0u : t <= 1 ? a.qk_row : t == 2 ? a.v_row : t == 3 ? 0u : ~0u;
            blk[i] = kq_blk ? a.qk_blk : (uint32_t)Rec<T>::bytes;
            const int sct = sub * kWave + a.lane;
            const int sh = t == 2 ? v_sh : kq_sh;
            off[i] = t >= 3 || kq_blk ? (uint32_t)sct * kPfSector
                                      : (uint32_t)(sct >> sh) * row[i] + (uint32_t)(sct & ((1 << sh) - 1)) * kPfSector;
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
    const uint64_t kq_step = a.qk_blk ? a.kq_step : (uint64_t)kChunk * a.qk_row;
    r.k = a.k0 + (uint64_t)cc * kq_step;
    r.q = a.q0 + (uint64_t)cc * kq_step;
    r.v = a.v0 + (uint64_t)cc * (kChunk * a.v_row) + vcol * ES;
    r.r = a.r0 + (uint64_t)cc * (uint32_t)(a.H * Rec<T>::bytes);
    r.kq_bytes = a.qk_blk ? (valid ? a.qk_blk : 0u) : (uint32_t)L * a.qk_row;
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
            const uint32_t bytes = !pvalid || rb == ~0u ? 0u : rb == 0u ? plan.blk[i] : pL * rb;
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

    // XCD-aware block order: the (sequence, q/k head) pairs go round the 8
    // XCDs (blockIdx % 8), and on its XCD each pair runs all column groups of
    // every value head that shares its q/k head, one after another. A unit's
    // groups and its GQA siblings read the K and Q rows and the records
    // through one L2, while consecutive pairs, of unequal packed lengths,
    // spread over the XCDs.
    const int bid = blockIdx.x;
    const int rest = bid >> 3;
    const int cgrp = rest % groups;
    const int per = H / Hk;                    // value heads per q/k head
    const int sib = (rest / groups) % per;
    const int kv = (rest / groups / per) * 8 + (bid & 7);   // (sequence, q/k head) pair
    const int u = kv * per + sib;
    if (kv >= units / per) return;
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
    a.qk_blk = 0;
    a.kq_step = 0;

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

// ------------------------------------------------------------ chunk_scan, role-split waves (bf16)
//
// One workgroup per (sequence, value head, 16 NT value columns) with NT + 2
// waves, one per SIMD (2 NT + 2 in the whole-prefill form, see below):
//   chain t owns the fp32 state of column tile t (16 columns) and runs the
//           dependent part of a chunk: X = K h, U = T (V - a o X), h' =
//           gamma_L h + K^T (c o U);
//   output  forms O^T = b o (h^T Q^T) + U^T P^T for the same columns (the
//           state and U fragments are A operands as they stand, the raw Q
//           rows and P fragments B operands) and stores O rows straight from
//           its accumulators;
//   copy    issues every direct-to-LDS copy (two chunks ahead, half of a
//           chunk on each side of the mid-step barrier) and the L2
//           prefetch, and waits for them.
// With the work of a column group spread over SIMDs this way, each wave's
// dependent chain is short and the copy engine is kept busy through the
// whole step. The step is then set by the group's shared staging and LDS
// traffic and by the barriers between the roles, not by matrix throughput:
// a chain wave given both tiles (half the K reads, twice the products) ran
// slower, and one given half a tile's state updates ran no faster.
// The chain waves hand h (at the end of a step) and U (mid-step) to the output
// wave through LDS. A chain wave reads a chunk's operands one step ahead,
// right after the mid-step barrier by which the copy wave has seen it land;
// the output wave reads its Q rows, P fragments and factors for the next
// chunk at the end of the step, likewise after that barrier.
// In the whole-prefill form the values are staged raw and one conv wave per
// column tile convolves its slab of each chunk in place during the step
// before the chains read them, half before and half after the mid-step
// barrier, which keeps the convolution off the chains' dependent path.
template <int KD, int NT>
struct RoleHand {
    bf16x8 h[KD / 32][NT][kWave];   // h of the step's chunk: B operand per contraction block and tile
    bf16x8 u[2][NT][kWave];         // U: B operand per 32-row block and tile
};

template <int KD>
struct ChainOps {
    bf16x8 kf[4][KD / 32];      // K rows: A operand of X = K h
    bf16x8 tf[kTriFrags];       // T
    f32x4 vv[4];                // values of the wave's tile, accumulator layout
    f32x4 fa[4], fc[4];         // row factors a and c
    float gL;                   // gamma_L
};
// Short-convolution taps (w0..w3, bias) of one value column, for the
// whole-prefill form, where the values are staged as raw rows before the
// convolution.
struct ColTaps {
    uint32_t w01, w23;   // (w0, w1), (w2, w3) as bf16 pairs
    float b;
};

// Whole-prefill form: the conv wave rewrites a chunk's staged value slab of
// tile t in place, from raw rows (row r at byte 32 r) to the convolved values
// in the chain wave's operand order: row tile i of chain lane l is 4 bf16 at
// byte 8 (64 i + l), i.e. where raw rows 16 i .. 16 i + 15 were.
__device__ __forceinline__ const unsigned char* conv_slot(const unsigned char* slab, int i, int lane) {
    return slab + (i * kWave + lane) * 8;
}
__device__ __forceinline__ unsigned char* conv_slot(unsigned char* slab, int i, int lane) {
    return slab + (i * kWave + lane) * 8;
}

template <int KD, int NT, bool CONV>
__device__ __forceinline__ void chain_load(ChainOps<KD>& op,
                                                const ScanBuf<bf16, KD, NT>* __restrict__ buf,
                                                const ScanLane<bf16, KD, NT>& ln, int t, int lane)
{
    const int grp = lane >> 4;
    typedef ScanBuf<bf16, KD, NT> SB;
    typedef Rec<bf16> RC;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int kb = 0; kb < KD / 32; ++kb) op.kf[rt][kb] = ld<bf16x8>(buf->k + ln.rf[kb] + 16 * rt * SB::RB);
#pragma unroll
    for (int f = 0; f < kTriFrags; ++f) op.tf[f] = ld<bf16x8>(buf->rec + RC::tfrag + (f * kWave + lane) * RC::frag_bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (CONV) {
            op.vv[i] = __builtin_convertvector(ld<bf16x4>(conv_slot(buf->v[t], i, lane)), f32x4);
        } else {
            const s16x4 raw = lds_read_tr16(buf->v[t] + ln.vtr + i * 16 * SB::VRB);
            op.vv[i] = __builtin_convertvector(__builtin_bit_cast(bf16x4, raw), f32x4);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        op.fa[i] = ld<f32x4>(buf->rec + RC::fac + (0 * kChunk + 16 * i + 4 * grp) * 4);
        op.fc[i] = ld<f32x4>(buf->rec + RC::fac + (2 * kChunk + 16 * i + 4 * grp) * 4);
    }
    op.gL = ld<float>(buf->rec + RC::fac + 3 * kChunk * 4);
}

// Conv wave, whole-prefill form: row tile i of value tile t of a staged chunk
// is convolved in place (see conv_slot). Lane (g, col) takes rows
// 16 i + 4 g .. + 3 of column col, the chain lane's rows: conv_rows reads them
// raw (x) with the four rows before them (p: 4 rows up in the slab; for lane
// group 0 of row tile 0 a valid address whose result the caller replaces by
// the raw rows 60..63 of the previous chunk, zero at the sequence start), and
// conv_put convolves and writes them over the slot. A tile's raw rows
// 16 i - 4 .. 16 i + 15 lie in its own slot and the one before, so a set of
// tiles all read before any of them is written may be converted in any order.
template <int KD, int NT>
__device__ __forceinline__ void conv_rows(const ScanBuf<bf16, KD, NT>* __restrict__ buf,
                                               const ScanLane<bf16, KD, NT>& ln, int t, int i, int grp,
                                               u32x2& x, u32x2& p)
{
    typedef ScanBuf<bf16, KD, NT> SB;
    const unsigned char* xa = buf->v[t] + ln.vtr + i * 16 * SB::VRB;
    x = __builtin_bit_cast(u32x2, lds_read_tr16(xa));
    p = __builtin_bit_cast(u32x2, lds_read_tr16(i == 0 && grp == 0 ? xa : xa - 4 * SB::VRB));
}
template <int KD, int NT>
__device__ __forceinline__ void conv_put(ScanBuf<bf16, KD, NT>* __restrict__ buf, int t, int i, int lane,
                                              const ColTaps& cv, const u32x2& x, const u32x2& p)
{
    // rows in time order, two to a word: p = (p0, p1), (p2, p3); x = (x0, x1), (x2, x3)
    const uint32_t p12 = pair_mid(p[0], p[1]), p3x0 = pair_mid(p[1], x[0]);
    const uint32_t x12 = pair_mid(x[0], x[1]);
    f32x4 y;
    y[0] = conv_silu(conv_taps4_bf16(cv.w01, cv.w23, cv.b, p12, p3x0));
    y[1] = conv_silu(conv_taps4_bf16(cv.w01, cv.w23, cv.b, p[1], x[0]));
    y[2] = conv_silu(conv_taps4_bf16(cv.w01, cv.w23, cv.b, p3x0, x12));
    y[3] = conv_silu(conv_taps4_bf16(cv.w01, cv.w23, cv.b, x[0], x[1]));
    // the values the scan sees are the bf16 convolution outputs
    *reinterpret_cast<bf16x4*>(conv_slot(buf->v[t], i, lane)) = __builtin_convertvector(y, bf16x4);
}

template <int KD>
struct OutOps {
    bf16x8 qf[4][KD / 32];      // Q rows: B operand of h^T Q^T
    bf16x8 pf[kTriFrags];       // P rows: B operand of U^T P^T
    float fb[4];                // b of chunk row 16 rt + (lane & 15)
};
template <int KD, int NT>
__device__ __forceinline__ void out_load(OutOps<KD>& op,
                                              const ScanBuf<bf16, KD, NT>* __restrict__ buf,
                                              const ScanLane<bf16, KD, NT>& ln, int col, int lane)
{
    typedef ScanBuf<bf16, KD, NT> SB;
    typedef Rec<bf16> RC;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int kb = 0; kb < KD / 32; ++kb) op.qf[rt][kb] = ld<bf16x8>(buf->q + ln.rf[kb] + 16 * rt * SB::RB);
#pragma unroll
    for (int f = 0; f < kTriFrags; ++f) op.pf[f] = ld<bf16x8>(buf->rec + RC::pfrag + (f * kWave + lane) * RC::frag_bytes);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) op.fb[rt] = ld<float>(buf->rec + RC::fac + (1 * kChunk + 16 * rt + col) * 4);
}

// One chunk of chain wave t. `hf` holds h as B operand (made when h was
// last updated) and `op` the chunk's operands; both turn over to the next
// chunk (its operands read from `ahead`).
template <int KD, int NT, bool CONV>
__device__ __forceinline__ void role_chain(const ScanBuf<bf16, KD, NT>* __restrict__ cur,
                                           const ScanBuf<bf16, KD, NT>* __restrict__ ahead,
                                           RoleHand<KD, NT>* __restrict__ hand,
                                           const ScanLane<bf16, KD, NT>& ln, int t, int grp, int col,
                                           f32x4 (&hs)[KD / 16], bf16x8 (&hf)[KD / 32],
                                           ChainOps<KD>& op)
{
    typedef Mma<bf16> MT;
    typedef bf16x8 Frag;
    typedef ScanBuf<bf16, KD, NT> SB;
    constexpr int KB = KD / 32;
    constexpr int RT = KD / 16;
    const int lane = 16 * grp + col;
    const unsigned char* kt = cur->k;

    // K^T operands of this chunk, used once U is known
    Frag ktf[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const unsigned char* p = kt + ln.tf[rt & 1][rt >> 1] + 32 * half * SB::RB;
            const s16x4 lo = lds_read_tr16(p);
            const s16x4 hi = lds_read_tr16(p + 16 * SB::RB);
            ktf[rt][half] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }

    // ---- X = K h (row tiles interleaved), U = T (V - a o X)
    f32x4 X[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) X[rt] = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) X[rt] = MT::mma(op.kf[rt][kb], hf[kb], X[rt]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) hs[rt] *= op.gL;   // decayed state: accumulator of the update
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) X[rt] = op.vv[rt] - op.fa[rt] * X[rt];
    f32x4 U[4];
    {
        const Frag vf0 = MT::acc_frag(X[0], X[1]);
        const Frag vf1 = MT::acc_frag(X[2], X[3]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) U[rt] = MT::mma(op.tf[tri_frag(rt, 0)], vf0, zero4());
#pragma unroll
        for (int rt = 2; rt < 4; ++rt) U[rt] = MT::mma(op.tf[tri_frag(rt, 1)], vf1, U[rt]);
    }
    hand->u[0][t][lane] = MT::acc_frag(U[0], U[1]);
    hand->u[1][t][lane] = MT::acc_frag(U[2], U[3]);
    f32x4 fc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) fc[rt] = op.fc[rt];
    lds_barrier();   // U is visible to the output wave; the next chunk has landed

    // ---- the next chunk's operands, then h' = gamma_L h + K^T (c o U)
    chain_load<KD, NT, CONV>(op, ahead, ln, t, lane);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) U[rt] *= fc[rt];
    const Frag df0 = MT::acc_frag(U[0], U[1]);
    const Frag df1 = MT::acc_frag(U[2], U[3]);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) hs[rt] = MT::mma(ktf[rt][half], half ? df1 : df0, hs[rt]);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        hf[kb] = state_frag<bf16>(hs[2 * kb], hs[2 * kb + 1], grp);
        hand->h[kb][t][lane] = hf[kb];
    }
}

// One chunk of the output wave: O^T tiles (lane: chunk row 16 rt + c, value
// columns 16 t + 4 g .. + 3) stored straight to global memory. `op` holds the
// chunk's operands (read a step ahead) and turns over to the next chunk's,
// read from `ahead`.
template <int KD, int NT>
__device__ __forceinline__ void role_output(const ScanBuf<bf16, KD, NT>* __restrict__ ahead,
                                            const RoleHand<KD, NT>* __restrict__ hand,
                                            const ScanLane<bf16, KD, NT>& ln, int grp, int col,
                                            OutOps<KD>& op, rsrc_t ro, uint32_t o_row)
{
    typedef Mma<bf16> MT;
    typedef bf16x8 Frag;
    constexpr int KB = KD / 32;
    const int lane = 16 * grp + col;

    Frag hf[NT][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int t = 0; t < NT; ++t) hf[t][kb] = hand->h[kb][t][lane];
    // ---- h^T Q^T, scaled by b per chunk row
    f32x4 O[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) O[t][rt] = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int t = 0; t < NT; ++t) O[t][rt] = MT::mma(hf[t][kb], op.qf[rt][kb], O[t][rt]);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) O[t][rt] *= op.fb[rt];
    lds_barrier();   // U has been written; the next chunk has landed

    // ---- + U^T P^T, then the next chunk's operands and the stores
    Frag uf[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        uf[t][0] = hand->u[0][t][lane];
        uf[t][1] = hand->u[1][t][lane];
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            O[t][rt] = MT::mma(uf[t][0], op.pf[tri_frag(rt, 0)], O[t][rt]);
            if (rt >= 2) O[t][rt] = MT::mma(uf[t][1], op.pf[tri_frag(rt, 1)], O[t][rt]);
        }
        if constexpr (NT == 2) {
            // one 16-byte store per lane: lane (g, c) holds columns 4 g .. + 3
            // of each tile in row c; two lane swaps (32 lanes apart, then 16)
            // give lane (g, c) the workgroup's columns 8 g .. + 7 instead, so a
            // row's 64 bytes go out as one piece (half the store requests)
            const u32x2 a = __builtin_bit_cast(u32x2, __builtin_convertvector(O[0][rt], bf16x4));
            const u32x2 b = __builtin_bit_cast(u32x2, __builtin_convertvector(O[1][rt], bf16x4));
            u32x4 s;
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const auto w32 = __builtin_amdgcn_permlane32_swap(a[d], b[d], false, false);
                const auto w16 = __builtin_amdgcn_permlane16_swap(w32[0], w32[1], false, false);
                s[d] = w16[0];
                s[2 + d] = w16[1];
            }
            __builtin_amdgcn_raw_buffer_store_b128(s, ro, (uint32_t)(16 * rt + col) * o_row + 16 * grp, 0, 0);
        } else {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bf16x4 ob = __builtin_convertvector(O[t][rt], bf16x4);
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ob), ro,
                                                      (uint32_t)(16 * rt + col) * o_row + (16 * t + 4 * grp) * 2, 0, 0);
            }
        }
    }
    out_load<KD, NT>(op, ahead, ln, col, lane);   // the next chunk's (landed by the mid-step barrier)
}

// CONV (whole-prefill form): vp points at the raw value rows before the
// short convolution, whose taps and bias for value channel 0 of head 0 are at
// wv and bv (bv may be null). NT more waves, the conv waves (one per column
// tile), convolve each chunk's staged values in place (conv_rows, conv_put)
// in the step before the chain waves read them; the copy wave stages values
// one chunk further ahead than the rest, so they have landed a step before
// that. Waves go copy, output, chains, conv: with two tiles the conv waves
// share SIMDs with the copy and output waves, which leave the VALU mostly
// idle; with one, every wave has a SIMD of its own.
template <int NT, bool CONV>
constexpr int roles_waves() { return NT + 2 + (CONV ? NT : 0); }

template <int KD, int NT, int NBUF, bool CONV>
__global__ __launch_bounds__((NT + 2 + (CONV ? NT : 0)) * kWave)
__attribute__((amdgpu_waves_per_eu((NT + 5 + (CONV ? NT : 0)) / 4, (NT + 5 + (CONV ? NT : 0)) / 4)))
void chunk_scan_roles_kernel(
    const bf16* __restrict__ qp, const bf16* __restrict__ kp, int64_t qk_stride,
    const bf16* __restrict__ vp, int64_t v_stride,
    const float* __restrict__ S0, float* __restrict__ Sfin, bf16* __restrict__ o,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ offsets,
    const unsigned char* __restrict__ ws_rec,
    int T_len, int H, int Hk, int V, int units, int groups,
    const bf16* __restrict__ wv, const bf16* __restrict__ bv)
{
    typedef bf16 T;
    typedef ScanBuf<T, KD, NT> SB;
    typedef ScanLane<T, KD, NT> LN;
    typedef RoleHand<KD, NT> HD;
    static_assert(NBUF == 3, "two chunks in flight");
    constexpr int ES = SB::ES;
    constexpr int RT = KD / 16;
    constexpr int TP = SB::tile_pieces;
    constexpr int RP = SB::rec_pieces;
    constexpr int loads = 2 * TP + RP + NT * SB::v_pieces;   // copies per chunk
    static_assert(loads + 2 * kPrefetchSlots < 64, "a step's loads fit the vector-memory counter");
    extern __shared__ __align__(1024) unsigned char smem_raw[];
    SB* bufs = reinterpret_cast<SB*>(smem_raw);
    unsigned char* scratch = smem_raw + NBUF * sizeof(SB);
    HD* hand = reinterpret_cast<HD*>(smem_raw + NBUF * sizeof(SB) + 256);

    // XCD-aware block order: the (sequence, q/k head) pairs go round the 8
    // XCDs (blockIdx % 8), and on its XCD each pair runs all column groups of
    // every value head that shares its q/k head, one after another. A unit's
    // groups and its GQA siblings read the K and Q rows and the records
    // through one L2, while consecutive pairs, of unequal packed lengths,
    // spread over the XCDs.
    const int bid = blockIdx.x;
    const int rest = bid >> 3;
    const int cgrp = rest % groups;
    const int per = H / Hk;                    // value heads per q/k head
    const int sib = (rest / groups) % per;
    const int kv = (rest / groups / per) * 8 + (bid & 7);   // (sequence, q/k head) pair
    const int u = kv * per + sib;
    if (kv >= units / per) return;
    const int seq = u / H;
    const int h = u - seq * H;

    const int lane = threadIdx.x & (kWave - 1);
    // roles: 0 .. NT - 1 chain of column tile `role`; NT output; NT + 1 copy;
    // NT + 2 + t conv of tile t (whole-prefill form). Waves in that order,
    // except that with conv waves they go copy, output, chains, conv (a
    // workgroup's wave w runs on SIMD (s + w) mod 4 for some s)
    constexpr int kRoleCopy = NT + 1, kRoleConv = NT + 2;
    constexpr int nwaves = roles_waves<NT, CONV>();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int role = !CONV ? wave : wave == 0 ? kRoleCopy : wave == 1 ? NT : wave <= NT + 1 ? wave - 2 : wave;
    const int grp = lane >> 4;
    const int col = lane & 15;

    ScanArgs<T, KD, NT> a;
    a.qp = qp; a.kp = kp; a.qk_stride = qk_stride; a.vp = vp; a.v_stride = v_stride; a.op = o;
    a.ws_rec = ws_rec; a.H = H; a.V = V; a.h = h; a.hk = h / (H / Hk); a.wave = 0; a.lane = lane;
    a.c0 = cgrp * NT * 16;                       // the workgroup's first value column
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
    a.qk_row = (uint32_t)(qk_stride * ES);
    a.v_row = (uint32_t)(v_stride * ES);
    a.v0 = (uint64_t)(vp + (int64_t)a.tok_begin * v_stride + h * V);
    a.r0 = (uint64_t)(ws_rec + ((int64_t)a.tile0 * H + h) * Rec<T>::bytes);
    if constexpr (CONV) {
        // q and k in (chunk, key head) blocks from qp: [q, k][slice][row][64 B]
        constexpr uint32_t tb = qk_block_bytes<KD>();
        a.qk_blk = tb;
        a.kq_step = (uint64_t)Hk * 2 * tb;
        a.q0 = (uint64_t)qp + ((uint64_t)a.tile0 * Hk + a.hk) * 2 * tb;
        a.k0 = a.q0 + tb;
    } else {
        a.k0 = (uint64_t)(kp + (int64_t)a.tok_begin * qk_stride + a.hk * KD);
        a.q0 = (uint64_t)(qp + (int64_t)a.tok_begin * qk_stride + a.hk * KD);
        a.qk_blk = 0;
        a.kq_step = 0;
    }

    // operand offsets (chain and output waves)
    LN ln;
#pragma unroll
    for (int kb = 0; kb < LN::KB; ++kb) {
        ln.rf[kb] = (uint32_t)tile_off<T, KD, NT>(col, 32 * kb + 8 * grp);
#pragma unroll
        for (int par = 0; par < 2; ++par)
            ln.tf[par][kb] = (uint32_t)tile_off<T, KD, NT>(4 * grp + (col >> 2), state_row(2 * kb + par, col & 3, 0));
    }
    ln.vtr = (uint32_t)((4 * grp + (col >> 2)) * SB::VRB + (col & 3) * 8);

    // A partial last chunk leaves the rows past the sequence unfetched: start
    // them at zero so they hold finite values (their factors are zero).
    if ((a.tok_end - a.tok_begin) % kChunk != 0) {
        const f32x4 z = zero4();
        for (int i = threadIdx.x * 16; i < NBUF * (int)sizeof(SB); i += nwaves * kWave * 16)
            *reinterpret_cast<f32x4*>(smem_raw + i) = z;
        lds_barrier();
    }

    if (role < NT) {
        // ---------------- chain of column tile t
        const int t = role;
        const int vc = a.c0 + 16 * t + col;
        f32x4 hs[RT];
        const int64_t sbase = ((int64_t)seq * H + h) * KD * V;
        if (S0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) hs[rt][e] = S0[sbase + (int64_t)state_row(rt, grp, e) * V + vc];
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) hs[rt] = zero4();
        }
        bf16x8 hf[LN::KB];
#pragma unroll
        for (int kb = 0; kb < LN::KB; ++kb) {
            hf[kb] = state_frag<T>(hs[2 * kb], hs[2 * kb + 1], grp);
            hand->h[kb][t][lane] = hf[kb];
        }
        lds_barrier();
        if constexpr (CONV) lds_barrier();   // chunk 0's values are convolved
        ChainOps<KD> op;
        chain_load<KD, NT, CONV>(op, &bufs[0], ln, t, lane);
        int b = 0;
        for (int c = 0; c < nchunks; ++c) {
            const int bn = b == NBUF - 1 ? 0 : b + 1;
            role_chain<KD, NT, CONV>(&bufs[b], &bufs[bn], hand, ln, t, grp, col, hs, hf, op);
            lds_barrier();
            b = bn;
        }
        if (Sfin) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) Sfin[sbase + (int64_t)state_row(rt, grp, e) * V + vc] = hs[rt][e];
        }
    } else if (role == NT) {
        // ---------------- output
        const int64_t HV = (int64_t)H * V;
        const uint32_t o_row = (uint32_t)(HV * ES);
        lds_barrier();
        if constexpr (CONV) lds_barrier();
        OutOps<KD> op;
        out_load<KD, NT>(op, &bufs[0], ln, col, lane);
        int b = 0;
        for (int c = 0; c < nchunks; ++c) {
            const int bn = b == NBUF - 1 ? 0 : b + 1;
            const int tok0 = a.tok_begin + c * kChunk;
            const int L = min(kChunk, a.tok_end - tok0);
            const rsrc_t ro = make_rsrc(o + (int64_t)tok0 * HV + (int64_t)h * V + a.c0, (uint32_t)L * o_row);
            role_output<KD, NT>(&bufs[bn], hand, ln, grp, col, op, ro, o_row);
            lds_barrier();
            b = bn;
        }
    } else if (role == kRoleCopy) {
        // ---------------- copy
        uint32_t tsrc[TP];
#pragma unroll
        for (int j = 0; j < TP; ++j) {
            const int row = j * SB::RPI + lane / SB::SPR;
            const int s = (lane % SB::SPR) ^ tile_mask<T, KD, NT>(row);
            // (blocked: segment s of a row is segment s % 4 of 32-column slice s / 4)
            tsrc[j] = CONV ? (uint32_t)((s >> 2) * (kChunk * 64) + row * 64 + (s & 3) * 16)
                           : (uint32_t)(row * (int64_t)a.qk_row + s * 16);
        }
        uint32_t vsrc[SB::v_pieces];
#pragma unroll
        for (int p = 0; p < SB::v_pieces; ++p)
            vsrc[p] = (uint32_t)((p * SB::RPV + lane / SB::LPR) * a.v_row + (lane % SB::LPR) * 16);
        PrefetchPlan<T, KD, NT> plan;
        plan.init(a, cgrp, groups);
        // A chunk's copies go out in two parts, one on each side of the
        // mid-step barrier, so that the copy engine works through the whole
        // step: part A (the K tile, the values and the prefetch of chunk cp)
        // and part B (the Q tile and the record). In the whole-prefill form the
        // values go out on their own, after the mid-step barrier of the step
        // two chunks earlier (issue_v).
        constexpr int nv = NT * SB::v_pieces;
        constexpr int partA = TP + (CONV ? 0 : nv) + kPrefetchSlots;
        auto issue_v = [&](int cs, SB* __restrict__ dst) {
            const ChunkSpan sp = chunk_span<T, KD, NT>(cs, a, a.c0);
            const rsrc_t rv = make_rsrc((const void*)sp.v, sp.v_bytes);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int p = 0; p < SB::v_pieces; ++p) dma16(rv, dst->v[t] + p * 1024, vsrc[p], t * 16 * ES);
        };
        auto issue_a = [&](int cs, int cp, SB* __restrict__ dst) {
            const ChunkSpan sp = chunk_span<T, KD, NT>(cs, a, a.c0);
            const rsrc_t rk = make_rsrc((const void*)sp.k, sp.kq_bytes);
#pragma unroll
            for (int j = 0; j < TP; ++j) dma16(rk, dst->k + j * 1024, tsrc[j], 0);
            if constexpr (!CONV) issue_v(cs, dst);
            const bool pvalid = cp < nchunks;
            const int pc = pvalid ? cp : 0;
            const uint32_t pL = pvalid ? (uint32_t)min(kChunk, a.tok_end - (a.tok_begin + cp * kChunk)) : 0u;
#pragma unroll
            for (int i = 0; i < kPrefetchSlots; ++i) {
                const uint32_t rb = plan.row[i];
                const uint32_t bytes = !pvalid || rb == ~0u ? 0u : rb == 0u ? plan.blk[i] : pL * rb;
                const rsrc_t pr = make_rsrc((const void*)(plan.base[i] + (uint64_t)pc * plan.step[i]), bytes);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(pr, (lds_ptr_t)scratch, 4, plan.off[i], 0, 0, 0);
            }
        };
        auto issue_b = [&](int cs, SB* __restrict__ dst) {
            const ChunkSpan sp = chunk_span<T, KD, NT>(cs, a, a.c0);
            const rsrc_t rq = make_rsrc((const void*)sp.q, sp.kq_bytes);
            const rsrc_t rr = make_rsrc((const void*)sp.r, sp.r_bytes);
#pragma unroll
            for (int j = 0; j < TP; ++j) dma16(rq, dst->q + j * 1024, tsrc[j], 0);
#pragma unroll
            for (int j = 0; j < RP; ++j) dma16(rr, dst->rec + j * 1024, lane * 16, j * 1024);
        };
        if constexpr (CONV) {
            // chunk 0 and chunk 1's values must land before the loop (the conv
            // wave takes them in the prologue), chunk 2's by the first mid-step
            issue_v(0, &bufs[0]);
            issue_a(0, NBUF - 1, &bufs[0]);
            issue_b(0, &bufs[0]);
            issue_v(1, &bufs[1]);
            issue_a(1, NBUF, &bufs[1]);
            issue_b(1, &bufs[1]);
            issue_v(2, &bufs[2]);
            wait_vmcnt<partA + TP + RP + nv>();   // younger: chunk 1's other copies, chunk 2's values
            lds_barrier();
            lds_barrier();   // chunk 0's values (and half of chunk 1's) are convolved
        } else {
            issue_a(0, NBUF - 1, &bufs[0]);
            issue_b(0, &bufs[0]);
            issue_a(1, NBUF, &bufs[1]);
            issue_b(1, &bufs[1]);
            wait_vmcnt<loads + kPrefetchSlots>();   // chunk 0 has landed (younger: chunk 1's copies)
            lds_barrier();
        }
        int b = 0;
        for (int c = 0; c < nchunks; ++c) {
            const int bp = b == 0 ? NBUF - 1 : b - 1;
            issue_a(c + NBUF - 1, c + NBUF - 1 + kPrefetchAhead, &bufs[bp]);
            // chunk c + 1 has landed (younger: this step's part A); with CONV
            // also chunk c + 2's values, issued a step ago
            wait_vmcnt<partA>();
            lds_barrier();         // mid-step
            // (CONV: chunk c's values were read by the chains a step ago)
            if constexpr (CONV) issue_v(c + NBUF, &bufs[b]);
            issue_b(c + NBUF - 1, &bufs[bp]);
            lds_barrier();         // end of step
            b = b == NBUF - 1 ? 0 : b + 1;
        }
        wait_vmcnt<0>();   // no copy into LDS may outlive the workgroup
    } else if constexpr (CONV) {
        // ---------------- conv of column tile t (whole-prefill form)
        // A chunk's value slab of tile t is convolved in two halves, row tiles
        // 3 and 2, then 1 and 0: chunk c + 2's first half after the mid-step
        // barrier of step c, its second half before the mid-step barrier of
        // step c + 1, by which the chain waves read it.
        const int t = role - kRoleConv;
        ColTaps cv;
        {
            const int64_t chn = (int64_t)h * V + a.c0 + 16 * t + col;
            const u32x2 tw = *reinterpret_cast<const u32x2*>(wv + chn * 4);
            cv.w01 = tw[0];
            cv.w23 = tw[1];
            cv.b = bv ? (float)bv[chn] : 0.f;
        }
        // raw rows 60..63 of the chunk before (cur; zero before the first) and
        // of this chunk (nxt), as held by lane group 3
        u32x2 cur = u32x2{0u, 0u}, nxt = u32x2{0u, 0u};
        const int from = (48 + col) * 4;   // byte index of lane (3, col)
        // a half's two row tiles are both read, then both convolved and
        // written (their dependent arithmetic interleaves). Row tile i reads
        // the last four raw rows of row tile i - 1, so the halves go from the
        // last rows to the first: tiles 3 and 2 (which read rows 28 .. 63)
        // before tiles 1 and 0 overwrite rows 0 .. 31
        auto convert = [&](int cc, int half) {
            if (cc >= nchunks) return;
            SB* __restrict__ buf = &bufs[cc % NBUF];
            u32x2 xs[2], ps[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) conv_rows<KD, NT>(buf, ln, t, 3 - 2 * half - n, grp, xs[n], ps[n]);
            if (half == 0) {
                nxt = xs[0];
            } else {
                u32x2 halo;
                halo[0] = (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)cur[0]);
                halo[1] = (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)cur[1]);
                if (grp == 0) ps[1] = halo;
                cur = nxt;
            }
#pragma unroll
            for (int n = 0; n < 2; ++n) conv_put<KD, NT>(buf, t, 3 - 2 * half - n, lane, cv, xs[n], ps[n]);
        };
        lds_barrier();
        convert(0, 0);
        convert(0, 1);
        convert(1, 0);
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            convert(c + 1, 1);
            lds_barrier();   // mid-step
            convert(c + 2, 0);
            lds_barrier();   // end of step
        }
    }
}

// ------------------------------------------------------------ chunk_scan, wide workgroups (bf16)
//
// One workgroup per (sequence, value head) unit holding ALL of the unit's V
// value columns, so a chunk's K and Q tiles and its record are staged into LDS
// once per unit instead of once per column group. NT / TPW compute waves:
// wave w owns the TPW column tiles TPW w .. TPW w + TPW - 1 (16 columns each,
// V = 16 NT) and runs the whole chunk step for them, the dependent
// chain X = K h, U = T (V - a o X), h' = gamma_L h + K^T (c o U) and the
// output O^T = b o (h^T Q^T) + U^T P^T (as the role-split kernel's output
// wave forms it, so each lane stores consecutive columns of one row), with no
// hand-off between waves. With two compute waves per SIMD (one tile each),
// one wave's VALU work and LDS waits overlap the other's matrix ops, and the
// compute waves issue the copies of the next chunk themselves (a wave stalled
// getting its share into the vector-memory pipe leaves its SIMD to the other);
// with one compute wave per SIMD (two tiles each) a copy wave issues every
// direct-to-LDS copy of the next chunk at the start of a step (61 KiB at
// K = V = 128: 61 copies, which fit its vector-memory counter) and waits for
// them at the end, so the compute waves never stall getting copies into the
// vector-memory pipe (a compute wave that issues a quarter of them itself
// spends a large part of its step there). Two buffers: chunk c + 1 lands while
// chunk c is computed; one barrier per chunk. Inside a step each phase's LDS
// operands are requested during the phase before, so their latency hides
// behind matrix ops.
//
// Whole-prefill form (CONV): four compute waves of NT / 4 tiles and four
// auxiliary waves, one per compute wave. Auxiliary wave a issues a quarter of
// the copies (the K / Q blocks and record of chunk c + 1 into one of two
// buffers, the raw value rows of chunk c + 2 into a ring of three) and, in
// step c, convolves compute wave a's value slabs of chunk c + 1 in place, as
// the column-group form's conv waves do; the compute waves read the convolved
// values in their operand order.
template <int KD, int NTILES>
struct WideBuf {
    static constexpr int RB = KD * 2;                       // bytes per K / Q row
    static constexpr int SPR = RB / 16;                     // 16-byte segments per row
    static constexpr int RPI = 1024 / RB;                   // rows per 1 KiB piece
    static constexpr int tile_pieces = kChunk * RB / 1024;
    static constexpr int rec_pieces = Rec<bf16>::bytes / 1024;
    static constexpr int NT = NTILES;                       // column tiles of the unit
    static constexpr int VRB = 32;                          // bytes per row of a tile slab
    static constexpr int v_pieces = NT * kChunk * VRB / 1024;
    static constexpr int copies = 2 * tile_pieces + v_pieces + rec_pieces;
    static_assert(copies < 64, "a chunk's copies fit the vector-memory counter");
    unsigned char k[kChunk * RB];
    unsigned char q[kChunk * RB];
    unsigned char rec[Rec<bf16>::bytes];
    unsigned char v[NT][kChunk * VRB];
};

// The direct-to-LDS copies of one chunk, pieces p = wave, wave + NW, ... of
// the list [K tile][Q tile][value slabs][record] (1 KiB each), issued by NW
// waves: the copy wave alone (NW = 1), or every compute wave. Per piece this
// lane's source offset and the piece's place in the buffer; the tensor of a
// piece is wave-uniform.
template <int KD, int NT, int NW>
struct WideCopies {
    typedef WideBuf<KD, NT> WB;
    static constexpr int total = WB::copies;
    static constexpr int per = (total + NW - 1) / NW;
    uint32_t src[per];
    uint32_t dst[per];
    int tensor[per];          // 0 K, 1 Q, 2 values, 3 record, 4 none
    __device__ __forceinline__ void init(int wave, int lane, uint32_t qk_row, uint32_t v_row) {
#pragma unroll
        for (int i = 0; i < per; ++i) {
            const int p = wave + NW * i;
            int t = 4, j = 0;
            if (p < WB::tile_pieces) { t = 0; j = p; }
            else if (p < 2 * WB::tile_pieces) { t = 1; j = p - WB::tile_pieces; }
            else if (p < 2 * WB::tile_pieces + WB::v_pieces) { t = 2; j = p - 2 * WB::tile_pieces; }
            else if (p < total) { t = 3; j = p - 2 * WB::tile_pieces - WB::v_pieces; }
            tensor[i] = t;
            if (t <= 1) {
                // rows RPI j .., each lane fetching the logical segment stored at its LDS position
                const int row = j * WB::RPI + lane / WB::SPR;
                const int sg = (lane % WB::SPR) ^ tile_mask<bf16, KD, 1>(row);
                src[i] = (uint32_t)row * qk_row + (uint32_t)sg * 16;
                dst[i] = (t == 0 ? offsetof(WB, k) : offsetof(WB, q)) + j * 1024;
            } else if (t == 2) {
                // rows 32 (j % 2) .. of slab j / 2
                const int row = 32 * (j & 1) + lane / 2;
                src[i] = (uint32_t)row * v_row + (uint32_t)(j >> 1) * 32 + (uint32_t)(lane & 1) * 16;
                dst[i] = offsetof(WB, v) + (j >> 1) * (kChunk * WB::VRB) + (j & 1) * 1024;
            } else {
                src[i] = (uint32_t)j * 1024 + lane * 16;
                dst[i] = offsetof(WB, rec) + j * 1024;
            }
        }
    }
    __device__ __forceinline__ void issue(unsigned char* buf, rsrc_t rk, rsrc_t rq, rsrc_t rv,
                                          rsrc_t rr) const {
#pragma unroll
        for (int i = 0; i < per; ++i) {
            const int t = tensor[i];
            if (t == 4) continue;
            const rsrc_t r = t == 0 ? rk : t == 1 ? rq : t == 2 ? rv : rr;
            dma16(r, buf + dst[i], src[i], 0);
        }
    }
};

// Whole-prefill form (CONV): the K and Q tiles and the record of a chunk in
// two buffers, its value slabs in a ring of three (a slab is copied raw two
// chunks ahead and convolved in place one chunk ahead).
template <int KD>
struct WideKQR {
    unsigned char k[kChunk * KD * 2];
    unsigned char q[kChunk * KD * 2];
    unsigned char rec[Rec<bf16>::bytes];
};
template <int NT>
struct WideVal {
    unsigned char v[NT][kChunk * 32];
};
template <int KD, int NT, bool CONV>
constexpr size_t wide_lds_bytes() {
    return CONV ? 2 * sizeof(WideKQR<KD>) + 3 * sizeof(WideVal<NT>) : 2 * sizeof(WideBuf<KD, NT>);
}

// The copies of a whole-prefill chunk step as pieces of 1 KiB, [K tile][Q
// tile][record][value slabs], auxiliary wave a taking pieces a, a + 4, ...:
// each piece's tensor, index in its tensor and LDS destination, at compile
// time.
template <int KD, int NT>
struct WideAuxPieces {
    typedef WideKQR<KD> KQR;
    static constexpr int TPc = kChunk * KD * 2 / 1024;     // pieces of a K / Q tile
    static constexpr int RPc = Rec<bf16>::bytes / 1024;
    static constexpr int VPc = NT * 2;                      // value pieces (2 per slab)
    static constexpr int total = 2 * TPc + RPc + VPc;
    static constexpr int per = (total + 3) / 4;
    // 0 K, 1 Q, 2 record, 3 values, 4 none
    static constexpr int tensor(int pc) {
        return pc < TPc ? 0 : pc < 2 * TPc ? 1 : pc < 2 * TPc + RPc ? 2 : pc < total ? 3 : 4;
    }
    static constexpr int index(int pc) {
        return pc < TPc ? pc : pc < 2 * TPc ? pc - TPc : pc < 2 * TPc + RPc ? pc - 2 * TPc
                                                                               : pc - 2 * TPc - RPc;
    }
    static constexpr uint32_t dst(int pc) {
        return tensor(pc) == 0 ? (uint32_t)offsetof(KQR, k) + index(pc) * 1024
             : tensor(pc) == 1 ? (uint32_t)offsetof(KQR, q) + index(pc) * 1024
             : tensor(pc) == 2 ? (uint32_t)offsetof(KQR, rec) + index(pc) * 1024
             : (uint32_t)(index(pc) >> 1) * (kChunk * 32) + (index(pc) & 1) * 1024;
    }
};

// f(std::integral_constant<int, i>) for i = 0 .. N - 1, unrolled
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// compute waves of a unit of NT column tiles with TPW tiles each; after them
// a copy wave (COPYW), or (CONV) four auxiliary waves that issue the copies
// and convolve the values, one per compute wave
template <int NT, int TPW>
constexpr int wide_waves() { return NT / TPW; }
template <int NT, int TPW, bool COPYW, bool CONV>
constexpr int wide_block() { return (wide_waves<NT, TPW>() + (CONV ? 4 : COPYW ? 1 : 0)) * kWave; }

// CONV (whole-prefill form): qp points at the blocked convolved q / k rows
// of the per-chunk solve ([q, k][32-column slice][64 rows][64 B] per (chunk,
// key head)), vp at the raw value rows, wv / bv at the value channels' taps
// and bias (bv may be null).
template <int KD, int NT, int TPW, bool COPYW, bool CONV>
__global__ __launch_bounds__((wide_block<NT, TPW, COPYW, CONV>()))
__attribute__((amdgpu_waves_per_eu((wide_block<NT, TPW, COPYW, CONV>() / kWave + 3) / 4,
                                   (wide_block<NT, TPW, COPYW, CONV>() / kWave + 3) / 4)))
void chunk_scan_wide_kernel(
    const bf16* __restrict__ qp, const bf16* __restrict__ kp, int64_t qk_stride,
    const bf16* __restrict__ vp, int64_t v_stride,
    const float* __restrict__ S0, float* __restrict__ Sfin, bf16* __restrict__ o,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ order,
    const unsigned char* __restrict__ ws_rec, int T_len, int H, int Hk, int units,
    const bf16* __restrict__ wv, const bf16* __restrict__ bv)
{
    typedef WideBuf<KD, NT> WB;
    typedef WideKQR<KD> KQR;
    typedef WideVal<NT> WV;
    constexpr int kWideWaves = wide_waves<NT, TPW>();
    static_assert(!CONV || kWideWaves == 4, "one auxiliary wave per compute wave");
    typedef Mma<bf16> MT;
    typedef bf16x8 Frag;
    typedef Rec<bf16> RC;
    constexpr int V = 16 * WB::NT;
    constexpr int KB = KD / 32;
    constexpr int RT = KD / 16;
    extern __shared__ __align__(1024) unsigned char smem_raw[];
    WB* bufs = reinterpret_cast<WB*>(smem_raw);
    KQR* kqrs = reinterpret_cast<KQR*>(smem_raw);
    WV* vring = reinterpret_cast<WV*>(smem_raw + 2 * sizeof(KQR));

    // Dense batches: XCD-aware order, the value heads that share a q/k head run
    // on one XCD (blockIdx % 8), one after another, so their K and Q rows come
    // from its L2. Packed sequences: longest first (order from the plan), so
    // the last workgroups to start are the shortest and the tail is short.
    const int bid = blockIdx.x;
    const int u = cu ? bid : (bid & 7) * ((units + 7) >> 3) + (bid >> 3);
    if (u >= units) return;
    const int rank = u / H;
    const int h = u - rank * H;
    const int seq = cu ? order[rank] : rank;
    const int hk = h / (H / Hk);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int grp = lane >> 4;
    const int col = lane & 15;

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
    const int nchunks = (tok_end - tok_begin + kChunk - 1) / kChunk;

    // A partial last chunk leaves the rows past the sequence unfetched: start
    // them at zero so they hold finite values (their factors are zero).
    if ((tok_end - tok_begin) % kChunk != 0) {
        const f32x4 z = zero4();
        for (int i = threadIdx.x * 16; i < (int)wide_lds_bytes<KD, NT, CONV>(); i += wide_block<NT, TPW, COPYW, CONV>() * 16)
            *reinterpret_cast<f32x4*>(smem_raw + i) = z;
        lds_barrier();
    }

    // ---- copies: chunk c + 1 into buffer (c + 1) % 2 during step c
    const uint32_t qk_row = (uint32_t)(qk_stride * 2);
    const uint32_t v_row = (uint32_t)(v_stride * 2);
    const uint64_t k0 = (uint64_t)(kp + (int64_t)tok_begin * qk_stride + hk * KD);
    const uint64_t q0 = (uint64_t)(qp + (int64_t)tok_begin * qk_stride + hk * KD);
    const uint64_t v0 = (uint64_t)(vp + (int64_t)tok_begin * v_stride + h * V);
    const uint64_t r0 = (uint64_t)(ws_rec + ((int64_t)tile0 * H + h) * RC::bytes);
    const uint64_t rstep = (uint64_t)H * RC::bytes;
    constexpr int NW = COPYW ? 1 : kWideWaves;
    WideCopies<KD, NT, NW> cp;
    if (!CONV && (!COPYW || wave == kWideWaves)) cp.init(COPYW ? 0 : wave, lane, qk_row, v_row);
    auto issue = [&](int c) {
        const bool valid = c < nchunks;
        const int cc = valid ? c : 0;
        const uint32_t L = valid ? (uint32_t)min(kChunk, tok_end - (tok_begin + cc * kChunk)) : 0u;
        cp.issue(reinterpret_cast<unsigned char*>(&bufs[c & 1]),
                 make_rsrc((const void*)(k0 + (uint64_t)cc * kChunk * qk_row), L * qk_row),
                 make_rsrc((const void*)(q0 + (uint64_t)cc * kChunk * qk_row), L * qk_row),
                 make_rsrc((const void*)(v0 + (uint64_t)cc * kChunk * v_row), L * v_row),
                 make_rsrc((const void*)(r0 + (uint64_t)cc * rstep), valid ? (uint32_t)RC::bytes : 0u));
    };

    if (CONV && wave >= kWideWaves) {
        // ---------------- auxiliary wave a: a quarter of the copies (K, Q and
        // record of chunk c + 1, raw values of chunk c + 2) and the
        // convolution of compute wave a's value slabs of chunk c + 1, in step c
        // (one instance per a, so every piece's tensor and LDS destination are
        // constants)
      auto aux = [&](auto a_c) {
        constexpr int a = decltype(a_c)::value;
        typedef WideAuxPieces<KD, NT> AP;
        constexpr uint32_t tb = qk_block_bytes<KD>();
        constexpr int SPR = KD * 2 / 16, RPI = 1024 / (KD * 2);
        const uint64_t qb0 = (uint64_t)qp + ((uint64_t)tile0 * Hk + hk) * 2 * tb;   // chunk 0's q block
        const uint64_t kqstep = (uint64_t)Hk * 2 * tb;
        uint32_t src[AP::per];   // this lane's source offset per piece
        static_for<AP::per>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            constexpr int pc = a + 4 * i, t = AP::tensor(pc), j = AP::index(pc);
            if constexpr (t <= 1) {
                // (blocked: logical segment sg of a row is segment sg % 4 of slice sg / 4)
                const int row = j * RPI + lane / SPR;
                const int sg = (lane % SPR) ^ tile_mask<bf16, KD, 1>(row);
                src[i] = (uint32_t)((sg >> 2) * (kChunk * 64) + row * 64 + (sg & 3) * 16);
            } else if constexpr (t == 2) {
                src[i] = (uint32_t)j * 1024 + lane * 16;
            } else if constexpr (t == 3) {
                const int row = 32 * (j & 1) + lane / 2;
                src[i] = (uint32_t)row * v_row + (uint32_t)(j >> 1) * 32 + (uint32_t)(lane & 1) * 16;
            } else {
                src[i] = 0u;
            }
        });
        auto chunk_rows = [&](int c) {
            return c < nchunks ? (uint32_t)min(kChunk, tok_end - (tok_begin + c * kChunk)) : 0u;
        };
        // K, Q and record of chunk c into kqrs[c % 2], values of chunk cv into vring[cv % 3]
        auto issue_aux = [&](int c, int cv, bool kqr, bool val) {
            const bool valid = c < nchunks;
            const int cc = valid ? c : 0;
            const uint64_t qb = qb0 + (uint64_t)cc * kqstep;
            const rsrc_t rq = make_rsrc((const void*)qb, valid ? tb : 0u);
            const rsrc_t rk = make_rsrc((const void*)(qb + tb), valid ? tb : 0u);
            const rsrc_t rr = make_rsrc((const void*)(r0 + (uint64_t)cc * rstep), valid ? (uint32_t)RC::bytes : 0u);
            const int cvv = cv < nchunks ? cv : 0;
            const rsrc_t rv = make_rsrc((const void*)(v0 + (uint64_t)cvv * kChunk * v_row), chunk_rows(cv) * v_row);
            unsigned char* kb_ = reinterpret_cast<unsigned char*>(&kqrs[c & 1]);
            unsigned char* vb_ = reinterpret_cast<unsigned char*>(&vring[cv % 3]);
            static_for<AP::per>([&](auto i_c) {
                constexpr int i = decltype(i_c)::value;
                constexpr int pc = a + 4 * i, t = AP::tensor(pc);
                constexpr uint32_t d = AP::dst(pc);
                if constexpr (t <= 2) {
                    if (kqr) dma16(t == 0 ? rk : t == 1 ? rq : rr, kb_ + d, src[i], 0);
                } else if constexpr (t == 3) {
                    if (val) dma16(rv, vb_ + d, src[i], 0);
                }
            });
        };
        // the taps and bias of this lane's column in each of compute wave a's tiles
        ColTaps cv[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int64_t chn = (int64_t)h * V + 16 * (TPW * a + t) + col;
            const u32x2 tw = *reinterpret_cast<const u32x2*>(wv + chn * 4);
            cv[t].w01 = tw[0];
            cv[t].w23 = tw[1];
            cv[t].b = bv ? (float)bv[chn] : 0.f;
        }
        // raw rows 60 .. 63 of the previous chunk per tile (as lane group 3 holds
        // them; zero before the sequence's first chunk)
        u32x2 prev[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) prev[t] = u32x2{0u, 0u};
        const uint32_t vtr_a = (uint32_t)((4 * grp + (col >> 2)) * 32 + (col & 3) * 8);
        const int from = (48 + col) * 4;   // byte index of lane (3, col) for ds_bpermute
        // the value slabs of chunk cc, in place: every row tile read (x: its 16
        // rows; p: the 4 rows before them) before any is written
        auto convert = [&](int cc) {
            if (cc >= nchunks) return;
            WV* __restrict__ vb = &vring[cc % 3];
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                unsigned char* slab = vb->v[TPW * a + t];
                u32x2 xs[4], ps[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const unsigned char* xa = slab + vtr_a + i * 16 * 32;
                    xs[i] = __builtin_bit_cast(u32x2, lds_read_tr16(xa));
                    ps[i] = __builtin_bit_cast(u32x2, lds_read_tr16(i == 0 && grp == 0 ? xa : xa - 4 * 32));
                }
                u32x2 halo;
                halo[0] = (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)prev[t][0]);
                halo[1] = (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)prev[t][1]);
                if (grp == 0) ps[0] = halo;
                prev[t] = xs[3];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x2 x = xs[i], pp = ps[i];
                    const uint32_t p12 = pair_mid(pp[0], pp[1]), p3x0 = pair_mid(pp[1], x[0]);
                    const uint32_t x12 = pair_mid(x[0], x[1]);
                    f32x4 y;
                    y[0] = conv_silu(conv_taps4_bf16(cv[t].w01, cv[t].w23, cv[t].b, p12, p3x0));
                    y[1] = conv_silu(conv_taps4_bf16(cv[t].w01, cv[t].w23, cv[t].b, pp[1], x[0]));
                    y[2] = conv_silu(conv_taps4_bf16(cv[t].w01, cv[t].w23, cv[t].b, p3x0, x12));
                    y[3] = conv_silu(conv_taps4_bf16(cv[t].w01, cv[t].w23, cv[t].b, x[0], x[1]));
                    *reinterpret_cast<bf16x4*>(conv_slot(slab, i, lane)) = __builtin_convertvector(y, bf16x4);
                }
            }
        };
        issue_aux(0, 0, true, true);
        issue_aux(0, 1, false, true);
        wait_vmcnt<0>();
        lds_barrier();
        convert(0);
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            issue_aux(c + 1, c + 2, true, true);
            convert(c + 1);
            wait_vmcnt<0>();
            lds_barrier();
        }
      };
        switch (wave - kWideWaves) {
        case 0: aux(std::integral_constant<int, 0>{}); break;
        case 1: aux(std::integral_constant<int, 1>{}); break;
        case 2: aux(std::integral_constant<int, 2>{}); break;
        default: aux(std::integral_constant<int, 3>{}); break;
        }
        return;
    }

    if (COPYW && wave == kWideWaves) {
        // ---------------- copy wave: the copies of chunk c + 1 in step c (an L2
        // prefetch of later chunks from this wave measured slower: its one-line
        // loads congest the CU's vector-memory pipe)
        issue(0);
        wait_vmcnt<0>();
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            issue(c + 1);
            wait_vmcnt<0>();
            lds_barrier();
        }
        return;
    }

    // ---------------- compute wave
    uint32_t rf[KB], tf[2][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        rf[kb] = (uint32_t)tile_off<bf16, KD, 1>(col, 32 * kb + 8 * grp);
#pragma unroll
        for (int par = 0; par < 2; ++par)
            tf[par][kb] = (uint32_t)tile_off<bf16, KD, 1>(4 * grp + (col >> 2), state_row(2 * kb + par, col & 3, 0));
    }
    const uint32_t vtr = (uint32_t)((4 * grp + (col >> 2)) * WB::VRB + (col & 3) * 8);

    const int64_t sbase = ((int64_t)seq * H + h) * KD * V;
    f32x4 hs[TPW][RT];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int vc = 16 * (TPW * wave + t) + col;
        if (S0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) hs[t][rt][e] = S0[sbase + (int64_t)state_row(rt, grp, e) * V + vc];
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) hs[t][rt] = zero4();
        }
    }
    Frag hf[TPW][KB];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) hf[t][kb] = state_frag_bf16(hs[t][2 * kb], hs[t][2 * kb + 1], grp);

    const int64_t HV = (int64_t)H * V;
    const uint32_t o_row = (uint32_t)(HV * 2);
    if constexpr (!COPYW && !CONV) {
        issue(0);
        wait_vmcnt<0>();
    }
    lds_barrier();   // chunk 0 has landed
    if constexpr (CONV) lds_barrier();   // chunk 0's values are convolved

    int vslot = 0;   // CONV: the value ring slot of chunk c
    for (int c = 0; c < nchunks; ++c) {
        if constexpr (!COPYW && !CONV) issue(c + 1);
        const unsigned char* kt;
        const unsigned char* qt;
        const unsigned char* rec;
        const unsigned char* vsl[TPW];
        if constexpr (CONV) {
            const KQR* __restrict__ cur = &kqrs[c & 1];
            kt = cur->k;
            qt = cur->q;
            rec = cur->rec;
#pragma unroll
            for (int t = 0; t < TPW; ++t) vsl[t] = vring[vslot].v[TPW * wave + t];
            vslot = vslot == 2 ? 0 : vslot + 1;
        } else {
            const WB* __restrict__ cur = &bufs[c & 1];
            kt = cur->k;
            qt = cur->q;
            rec = cur->rec;
#pragma unroll
            for (int t = 0; t < TPW; ++t) vsl[t] = cur->v[TPW * wave + t];
        }
        auto row_frag = [&](const unsigned char* tile, int rt, int kb) -> Frag {
            return ld<Frag>(tile + rf[kb] + 16 * rt * WB::RB);
        };
        auto fac4 = [&](int which, int rt) -> f32x4 {
            return ld<f32x4>(rec + RC::fac + (which * kChunk + 16 * rt + 4 * grp) * 4);
        };
        auto kt_frag = [&](int rt, int half) -> Frag {
            const unsigned char* p = kt + tf[rt & 1][rt >> 1] + 32 * half * WB::RB;
            const s16x4 lo = lds_read_tr16(p);
            const s16x4 hi = lds_read_tr16(p + 16 * WB::RB);
            return __builtin_bit_cast(Frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };

        // Each phase's LDS operands are requested in the phase before it, and
        // each phase carries VALU work that does not depend on its own matrix
        // ops, so the two overlap: the state decay and the value conversion
        // beside X, U's operand packing beside Y, the outputs' packing and
        // stores and the next step's state operands beside the h' products.

        // ---- operands of X (row tiles 0, 1), the values, a and gamma_L
        Frag ka[2][KB], kb2[2][KB];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) ka[r][kb] = row_frag(kt, r, kb);
        s16x4 vraw[TPW][4];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                // (CONV: convolved in place in this lane's operand order)
                if constexpr (CONV) vraw[t][rt] = ld<s16x4>(conv_slot(vsl[t], rt, lane));
                else vraw[t][rt] = lds_read_tr16(vsl[t] + vtr + rt * 16 * WB::VRB);
            }
        f32x4 fa[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) fa[rt] = fac4(0, rt);
        const float gL = ld<float>(rec + RC::fac + 3 * kChunk * 4);
        SCAN_FENCE();

        // ---- X = K h, row tiles 0, 1 (loads: K row tiles 2, 3 and T; VALU:
        // the first half of the decayed state gamma_L h, the accumulator of h')
        f32x4 X[TPW][4];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                X[t][r] = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) X[t][r] = MT::mma(ka[r][kb], hf[t][kb], X[t][r]);
            }
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) kb2[r][kb] = row_frag(kt, 2 + r, kb);
        Frag tfr[kTriFrags];
#pragma unroll
        for (int f = 0; f < kTriFrags; ++f) tfr[f] = ld<Frag>(rec + RC::tfrag + (f * kWave + lane) * RC::frag_bytes);
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int rt = 0; rt < RT / 2; ++rt) hs[t][rt] *= gL;
        SCAN_FENCE();

        // ---- X, row tiles 2, 3 (loads: Q row tiles 0, 1; VALU: the other
        // half of gamma_L h, the values to fp32)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                X[t][2 + r] = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) X[t][2 + r] = MT::mma(kb2[r][kb], hf[t][kb], X[t][2 + r]);
            }
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) ka[r][kb] = row_frag(qt, r, kb);
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int rt = RT / 2; rt < RT; ++rt) hs[t][rt] *= gL;
        SCAN_FENCE();

        // ---- U = T (V - a o X) (loads: Q row tiles 2, 3)
        f32x4 U[TPW][4];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const f32x4 vv = __builtin_convertvector(__builtin_bit_cast(bf16x4, vraw[t][rt]), f32x4);
                X[t][rt] = vv - fa[rt] * X[t][rt];
            }
            const Frag vf0 = MT::acc_frag(X[t][0], X[t][1]);
            const Frag vf1 = MT::acc_frag(X[t][2], X[t][3]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) U[t][rt] = MT::mma(tfr[tri_frag(rt, 0)], vf0, zero4());
#pragma unroll
            for (int rt = 2; rt < 4; ++rt) U[t][rt] = MT::mma(tfr[tri_frag(rt, 1)], vf1, U[t][rt]);
        }
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) kb2[r][kb] = row_frag(qt, 2 + r, kb);
        SCAN_FENCE();

        // ---- Y^T = h^T Q^T, row tiles 0, 1 (loads: b, c)
        f32x4 Y[TPW][4];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                Y[t][r] = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) Y[t][r] = MT::mma(hf[t][kb], ka[r][kb], Y[t][r]);
            }
        float fb[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) fb[rt] = ld<float>(rec + RC::fac + (1 * kChunk + 16 * rt + col) * 4);
        f32x4 fc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) fc[rt] = fac4(2, rt);
        SCAN_FENCE();

        // ---- Y^T, row tiles 2, 3 (loads: P; VALU: the operands of U and of
        // c o U, b o Y^T of row tiles 0, 1)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                Y[t][2 + r] = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) Y[t][2 + r] = MT::mma(hf[t][kb], kb2[r][kb], Y[t][2 + r]);
            }
        Frag pfr[kTriFrags];
#pragma unroll
        for (int f = 0; f < kTriFrags; ++f) pfr[f] = ld<Frag>(rec + RC::pfrag + (f * kWave + lane) * RC::frag_bytes);
        Frag uf[TPW][2], df[TPW][2];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            uf[t][0] = MT::acc_frag(U[t][0], U[t][1]);
            uf[t][1] = MT::acc_frag(U[t][2], U[t][3]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) U[t][rt] *= fc[rt];
            df[t][0] = MT::acc_frag(U[t][0], U[t][1]);
            df[t][1] = MT::acc_frag(U[t][2], U[t][3]);
            Y[t][0] *= fb[0];
            Y[t][1] *= fb[1];
        }
        SCAN_FENCE();

        // ---- O^T = b o Y^T + U^T P^T (loads: K^T of state tiles 0, 1)
        Frag ktf[2][2][2];   // [pair parity][tile of the pair][half]
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int half = 0; half < 2; ++half) ktf[0][i][half] = kt_frag(i, half);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                Y[t][rt] = MT::mma(uf[t][0], pfr[tri_frag(rt, 0)], rt >= 2 ? Y[t][rt] * fb[rt] : Y[t][rt]);
                if (rt >= 2) Y[t][rt] = MT::mma(uf[t][1], pfr[tri_frag(rt, 1)], Y[t][rt]);
            }
        }
        SCAN_FENCE();

        // ---- h' = gamma_L h + K^T (c o U), two state tiles at a time, the K^T
        // operands of the next two requested before the current products; the
        // outputs packed and stored, and the next step's state operands built,
        // beside them
        const int tok0 = tok_begin + c * kChunk;
        const uint32_t L = (uint32_t)min(kChunk, tok_end - tok0);
        const rsrc_t ro = make_rsrc(o + (int64_t)tok0 * HV + (int64_t)h * V + 16 * TPW * wave, L * o_row);
        auto store_rows = [&](int rt) {
            if constexpr (TPW == 2) {
                // lane swaps give lane (g, c) the wave's columns 8 g .. + 7 of row c
                const u32x2 a = __builtin_bit_cast(u32x2, __builtin_convertvector(Y[0][rt], bf16x4));
                const u32x2 b = __builtin_bit_cast(u32x2, __builtin_convertvector(Y[1][rt], bf16x4));
                u32x4 sv;
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const auto w32 = __builtin_amdgcn_permlane32_swap(a[d], b[d], false, false);
                    const auto w16 = __builtin_amdgcn_permlane16_swap(w32[0], w32[1], false, false);
                    sv[d] = w16[0];
                    sv[2 + d] = w16[1];
                }
                __builtin_amdgcn_raw_buffer_store_b128(sv, ro, (uint32_t)(16 * rt + col) * o_row + 16 * grp, 0, 0);
            } else {
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const bf16x4 ob = __builtin_convertvector(Y[t][rt], bf16x4);
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ob), ro,
                                                          (uint32_t)(16 * rt + col) * o_row + (16 * t + 4 * grp) * 2, 0, 0);
                }
            }
        };
#pragma unroll
        for (int rp = 0; rp < RT / 2; ++rp) {
            if (rp + 1 < RT / 2) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int half = 0; half < 2; ++half)
                        ktf[(rp + 1) & 1][i][half] = kt_frag(2 * (rp + 1) + i, half);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const int rt = 2 * rp + i;
                    const f32x4 acc = MT::mma(ktf[rp & 1][i][0], df[t][0], hs[t][rt]);
                    hs[t][rt] = MT::mma(ktf[rp & 1][i][1], df[t][1], acc);
                }
            if (rp < 4) store_rows(rp);
            if (rp >= 1) {
#pragma unroll
                for (int t = 0; t < TPW; ++t) hf[t][rp - 1] = state_frag_bf16(hs[t][2 * rp - 2], hs[t][2 * rp - 1], grp);
            }
            SCAN_FENCE();
        }
#pragma unroll
        for (int rt = RT / 2; rt < 4; ++rt) store_rows(rt);
#pragma unroll
        for (int t = 0; t < TPW; ++t) hf[t][KB - 1] = state_frag_bf16(hs[t][RT - 2], hs[t][RT - 1], grp);
        if constexpr (!COPYW && !CONV) wait_vmcnt<0>();   // this wave's copies of chunk c + 1 (and its stores)
        lds_barrier();   // every wave is done with this buffer; chunk c + 1 has landed
    }

    if (Sfin) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int vc = 16 * (TPW * wave + t) + col;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) Sfin[sbase + (int64_t)state_row(rt, grp, e) * V + vc] = hs[t][rt][e];
        }
    }
}

// ------------------------------------------------------------ launchers

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static inline int64_t tiles_upper_bound(int B, int T_len, int n_seqs, bool packed) {
    if (!packed) return (int64_t)B * ((T_len + kChunk - 1) / kChunk);
    return ((int64_t)T_len + (int64_t)(kChunk - 1) * n_seqs) / kChunk;
}

// Workspace header: the packed sequences' chunk offsets (n_seqs + 1) and their
// longest-first order (n_seqs), then the records.
static inline size_t plan_bytes(int n_seqs) { return align256(sizeof(int32_t) * (size_t)(2 * n_seqs + 1)); }

size_t chunk_workspace_bytes(int B, int T_len, int H, int n_seqs, bool packed, bool use_bf16) {
    const int64_t tiles = tiles_upper_bound(B, T_len, n_seqs, packed);
    const size_t rec = use_bf16 ? Rec<bf16>::bytes : Rec<float>::bytes;
    return plan_bytes(n_seqs) + rec * (size_t)tiles * H;
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
    const int upad = (units / (H / Hk) + 7) / 8 * 8 * (H / Hk);   // 8 XCDs x whole (sequence, q/k head) pairs
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

template <int KD, int NT, bool CONV = false>
static hipError_t launch_scan_roles(const void* q, const void* k, int64_t qks, const void* v,
                                   int64_t vs, const float* S0, float* Sf, void* o,
                                   const int32_t* cu, const int32_t* offsets,
                                   const unsigned char* wsrec, int T_len, int H, int Hk, int V,
                                   int N, hipStream_t stream, const void* wv = nullptr,
                                   const void* bv = nullptr)
{
    const int units = N * H;
    const int groups = V / (16 * NT);
    const int upad = (units / (H / Hk) + 7) / 8 * 8 * (H / Hk);   // 8 XCDs x whole (sequence, q/k head) pairs
    typedef ScanBuf<bf16, KD, NT> SB;
    constexpr int NBUF = 3;
    constexpr size_t smem = NBUF * sizeof(SB) + 256 + sizeof(RoleHand<KD, NT>);
    static_assert(smem <= 160 * 1024, "scan staging fits in LDS");
    auto kern = chunk_scan_roles_kernel<KD, NT, NBUF, CONV>;
    hipError_t err = set_smem(kern, smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3((unsigned)(upad * groups)), dim3(roles_waves<NT, CONV>() * kWave), smem, stream,
                       (const bf16*)q, (const bf16*)k, qks, (const bf16*)v, vs, S0, Sf, (bf16*)o,
                       cu, offsets, wsrec, T_len, H, Hk, V, units, groups, (const bf16*)wv,
                       (const bf16*)bv);
    return hipGetLastError();
}

template <int KD, int NT, int TPW, bool COPYW, bool CONV = false>
static hipError_t launch_scan_wide(const void* q, const void* k, int64_t qks, const void* v,
                                   int64_t vs, const float* S0, float* Sf, void* o,
                                   const int32_t* cu, const int32_t* offsets, const int32_t* order,
                                   const unsigned char* wsrec, int T_len, int H, int Hk, int N,
                                   hipStream_t stream, const void* wv = nullptr,
                                   const void* bv = nullptr)
{
    const int units = N * H;
    const int u8 = (units + 7) / 8;
    constexpr size_t smem = wide_lds_bytes<KD, NT, CONV>();
    static_assert(smem <= 160 * 1024, "wide scan staging fits in LDS");
    auto kern = chunk_scan_wide_kernel<KD, NT, TPW, COPYW, CONV>;
    hipError_t err = set_smem(kern, smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3((unsigned)(8 * u8)), dim3(wide_block<NT, TPW, COPYW, CONV>()), smem,
                       stream, (const bf16*)q, (const bf16*)k, qks, (const bf16*)v, vs, S0, Sf,
                       (bf16*)o, cu, offsets, order, wsrec, T_len, H, Hk, units, (const bf16*)wv,
                       (const bf16*)bv);
    return hipGetLastError();
}

struct ChunkWs {
    int32_t* offsets;
    int32_t* order;
    unsigned char* rec;
};

static inline ChunkWs carve(void* ws, int n_seqs) {
    ChunkWs w;
    w.offsets = (int32_t*)ws;
    w.order = w.offsets + (n_seqs + 1);
    w.rec = (unsigned char*)ws + plan_bytes(n_seqs);
    return w;
}

template <typename T, int KD, bool GATES = false, bool CONV = false>
static hipError_t launch_prepare_t(const void* q, const void* k, int64_t qks, const float* g,
                                   const float* beta, const int32_t* cu, int n_seqs, int B,
                                   int T_len, int H, int Hk, float scale, int l2norm, void* ws,
                                   hipStream_t stream, const PrepFused& gz = PrepFused{})
{
    const bool packed = cu != nullptr;
    const int64_t tiles = tiles_upper_bound(B, T_len, n_seqs, packed);
    const ChunkWs w = carve(ws, n_seqs);
    if (packed) {
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(256), 0, stream, cu, n_seqs, w.offsets,
                           w.order);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (tiles > 0) {
        // one single-wave workgroup per (tile, key head) item (tiles padded to
        // a multiple of the 8 XCDs)
        const int64_t items = tiles * Hk;
        const int64_t blocks = (tiles + 7) / 8 * 8 * Hk;
        auto kern = chunk_prep_kernel<T, KD, GATES, CONV>;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kWave), 0, stream,
                           (const T*)q, (const T*)k, qks, g, beta, cu, w.offsets, n_seqs, T_len, H,
                           Hk, scale, l2norm, w.rec, (int)items, gz);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Column tiles (of 16 value columns) per scan workgroup. bf16 (role-split
// kernel): two where that still gives a workgroup per CU, else one; fp32: four
// (shared staging) when there is parallelism to spare, else one (a 2-tile
// instance does not get through the gfx950 backend). The tuning knob
// overrides the choice with any value valid for the dtype.
// Scan form for bf16 operands: whole-unit workgroups when the call has
// enough (sequence, head) units to fill the chip twice over with one
// workgroup each (their per-unit copies are a quarter of the column groups',
// but a unit runs on one CU), else column groups. The knob overrides.
constexpr int kWideMinUnits = 512;
static inline bool scan_wide(int64_t units) {
    const int f = tune_knob[kTuneScanForm];
    if (f == 1 || f == 2) return f == 2;
    return units >= kWideMinUnits;
}

static inline int scan_tiles(int64_t units, int slabs, bool bf16_ops) {
    const int k = tune_knob[kTuneScanTiles];
    if (bf16_ops) {
        if (k == 1 || k == 2) return k;
        return units * (slabs / 2) >= 256 ? 2 : 1;
    }
    if (k == 1 || (k == 4 && slabs % 4 == 0)) return k;
    return units * (slabs / 4) >= 512 && slabs % 4 == 0 ? 4 : 1;
}

template <typename T, int KD>
static hipError_t launch_scan_t(const void* q, const void* k, int64_t qks, const void* v,
                                int64_t vs, const float* S0, float* Sf, void* o, const int32_t* cu,
                                int n_seqs, int B, int T_len, int H, int Hk, int V, const void* ws,
                                hipStream_t stream)
{
    const int N = cu ? n_seqs : B;
    const ChunkWs w = carve(const_cast<void*>(ws), n_seqs);
    const int units = N * H;
    const int slabs = V / 16;
    const int tiles = scan_tiles(units, slabs, sizeof(T) == 2);
    if constexpr (sizeof(T) == 2) {
        // bf16 operands: whole-unit workgroups when chosen, else the split-role step
        if (scan_wide(units)) {
            // V = 128: four compute waves of two tiles and a copy wave, or
            // (GDN_TUNE_SCAN_TILES = 1) eight compute waves of one tile
            // issuing the copies themselves; V = 64: four of one tile
            if (V == 128 && tune_knob[kTuneScanTiles] == 1)
                return launch_scan_wide<KD, 8, 1, false>(q, k, qks, v, vs, S0, Sf, o, cu, w.offsets, w.order, w.rec, T_len, H, Hk, N, stream);
            if (V == 128)
                return launch_scan_wide<KD, 8, 2, true>(q, k, qks, v, vs, S0, Sf, o, cu, w.offsets, w.order, w.rec, T_len, H, Hk, N, stream);
            return launch_scan_wide<KD, 4, 1, true>(q, k, qks, v, vs, S0, Sf, o, cu, w.offsets, w.order, w.rec, T_len, H, Hk, N, stream);
        }
        if (tiles == 2)
            return launch_scan_roles<KD, 2>(q, k, qks, v, vs, S0, Sf, o, cu, w.offsets, w.rec, T_len, H, Hk, V, N, stream);
        return launch_scan_roles<KD, 1>(q, k, qks, v, vs, S0, Sf, o, cu, w.offsets, w.rec, T_len, H, Hk, V, N, stream);
    } else {
        // fp32 operands (the small parity workloads)
        if (tiles == 4)
            return launch_scan<T, KD, 4>(q, k, qks, v, vs, S0, Sf, o, cu, w.offsets, w.rec, T_len, H, Hk, V, N, stream);
        return launch_scan<T, KD, 1>(q, k, qks, v, vs, S0, Sf, o, cu, w.offsets, w.rec, T_len, H, Hk, V, N, stream);
    }
}

hipError_t launch_chunk_prepare(const void* q, const void* k, int64_t qks, const float* g,
                                const float* beta, const int32_t* cu, int n_seqs, int B, int T_len,
                                int H, int Hk, int K, float scale, int l2norm, bool use_bf16,
                                void* ws, hipStream_t stream)
{
    if (!cu) n_seqs = 0;   // dense: the workspace holds no sequence offsets
    if (use_bf16)
        return K == 128 ? launch_prepare_t<bf16, 128>(q, k, qks, g, beta, cu, n_seqs, B, T_len, H, Hk, scale, l2norm, ws, stream)
                        : launch_prepare_t<bf16, 64>(q, k, qks, g, beta, cu, n_seqs, B, T_len, H, Hk, scale, l2norm, ws, stream);
    return K == 128 ? launch_prepare_t<float, 128>(q, k, qks, g, beta, cu, n_seqs, B, T_len, H, Hk, scale, l2norm, ws, stream)
                    : launch_prepare_t<float, 64>(q, k, qks, g, beta, cu, n_seqs, B, T_len, H, Hk, scale, l2norm, ws, stream);
}

// Whole prefill in two launches (prepare and scan phases): chunk_prep
// convolving the raw q and k rows and forming the gates itself (the
// convolved rows go to the workspace, after the records, for the scan), then
// the role-split scan convolving the value rows as it reads them. Equal, bit
// for bit, to conv1d + gate_prepare + chunk_prepare + chunk_scan (role-split)
// on the same inputs; y, g and beta are never written.
size_t prefill_workspace_bytes(int B, int T_len, int H, int Hk, int K, int n_seqs, bool packed) {
    const int64_t tiles = tiles_upper_bound(B, T_len, n_seqs, packed);
    return align256(chunk_workspace_bytes(B, T_len, H, n_seqs, packed, true)) +
           (size_t)tiles * Hk * 2 * kChunk * K * sizeof(bf16);
}

// The q / k blocks of the whole-prefill form: after the records in the workspace.
static inline unsigned char* prefill_qk(void* ws, int B, int T_len, int H, int n_seqs) {
    return (unsigned char*)ws + align256(chunk_workspace_bytes(B, T_len, H, n_seqs, n_seqs > 0, true));
}

template <int KD>
static hipError_t launch_prefill_prepare_t(const bf16* x, int64_t xs, const bf16* cw,
                                           const bf16* cb, const bf16* a, int64_t as,
                                           const bf16* b, int64_t bs, const float* A_log,
                                           const float* dt_bias, const int32_t* cu, int n_seqs,
                                           int B, int T_len, int H, int Hk, float scale,
                                           int l2norm, void* ws, hipStream_t stream)
{
    const int64_t qkc = (int64_t)Hk * KD;             // channels of q (and of k)
    PrepFused gz;
    gz.a = a; gz.as = as;
    gz.b = b; gz.bs = bs;
    gz.A_log = A_log;
    gz.dt_bias = dt_bias;
    gz.wq = cw;
    gz.wk = cw + qkc * 4;
    gz.bq = cb;
    gz.bk = cb ? cb + qkc : nullptr;
    gz.qk = prefill_qk(ws, B, T_len, H, n_seqs);
    return launch_prepare_t<bf16, KD, true, true>(x, x + qkc, xs, nullptr, nullptr, cu, n_seqs, B,
                                                  T_len, H, Hk, scale, l2norm, ws, stream, gz);
}

template <int KD>
static hipError_t launch_prefill_scan_t(const bf16* x, int64_t xs, const bf16* cw, const bf16* cb,
                                        const float* S0, float* Sf, void* o, const int32_t* cu,
                                        int n_seqs, int B, int T_len, int H, int Hk, int V,
                                        void* ws, hipStream_t stream)
{
    const int64_t qkc = (int64_t)Hk * KD;
    const bf16* qk = (const bf16*)prefill_qk(ws, B, T_len, H, n_seqs);   // blocked q / k
    const int N = cu ? n_seqs : B;
    const ChunkWs w = carve(ws, n_seqs);
    const int slabs = V / 16;
    const bf16* wv = cw + 2 * qkc * 4;
    const bf16* bv = cb ? cb + 2 * qkc : nullptr;
    if (scan_wide((int64_t)N * H)) {
        if (V == 128)
            return launch_scan_wide<KD, 8, 2, false, true>(qk, qk, 0, x + 2 * qkc, xs, S0, Sf, o, cu,
                                                           w.offsets, w.order, w.rec, T_len, H, Hk, N,
                                                           stream, wv, bv);
        return launch_scan_wide<KD, 4, 1, false, true>(qk, qk, 0, x + 2 * qkc, xs, S0, Sf, o, cu,
                                                       w.offsets, w.order, w.rec, T_len, H, Hk, N,
                                                       stream, wv, bv);
    }
    if (scan_tiles((int64_t)N * H, slabs, true) == 2)
        return launch_scan_roles<KD, 2, true>(qk, qk, 0, x + 2 * qkc, xs, S0, Sf, o, cu, w.offsets,
                                              w.rec, T_len, H, Hk, V, N, stream, wv, bv);
    return launch_scan_roles<KD, 1, true>(qk, qk, 0, x + 2 * qkc, xs, S0, Sf, o, cu, w.offsets,
                                          w.rec, T_len, H, Hk, V, N, stream, wv, bv);
}

hipError_t launch_prefill_prepare(const void* x, int64_t xs, const void* cw, const void* cb,
                                  const void* a, int64_t as, const void* b, int64_t bs,
                                  const float* A_log, const float* dt_bias, const int32_t* cu,
                                  int n_seqs, int B, int T_len, int H, int Hk, int K, float scale,
                                  int l2norm, void* ws, hipStream_t stream)
{
    if (!cu) n_seqs = 0;
    if (K == 128)
        return launch_prefill_prepare_t<128>((const bf16*)x, xs, (const bf16*)cw, (const bf16*)cb,
                                             (const bf16*)a, as, (const bf16*)b, bs, A_log, dt_bias,
                                             cu, n_seqs, B, T_len, H, Hk, scale, l2norm, ws, stream);
    return launch_prefill_prepare_t<64>((const bf16*)x, xs, (const bf16*)cw, (const bf16*)cb,
                                        (const bf16*)a, as, (const bf16*)b, bs, A_log, dt_bias, cu,
                                        n_seqs, B, T_len, H, Hk, scale, l2norm, ws, stream);
}

hipError_t launch_prefill_scan(const void* x, int64_t xs, const void* cw, const void* cb,
                               const float* S0, float* Sf, void* o, const int32_t* cu, int n_seqs,
                               int B, int T_len, int H, int Hk, int K, int V, void* ws,
                               hipStream_t stream)
{
    if (!cu) n_seqs = 0;
    if (K == 128)
        return launch_prefill_scan_t<128>((const bf16*)x, xs, (const bf16*)cw, (const bf16*)cb, S0,
                                          Sf, o, cu, n_seqs, B, T_len, H, Hk, V, ws, stream);
    return launch_prefill_scan_t<64>((const bf16*)x, xs, (const bf16*)cw, (const bf16*)cb, S0, Sf,
                                     o, cu, n_seqs, B, T_len, H, Hk, V, ws, stream);
}

hipError_t launch_chunk_scan(const void* q, const void* k, int64_t qks, const void* v, int64_t vs,
                             const float* S0, float* Sf, void* o, const int32_t* cu, int n_seqs,
                             int B, int T_len, int H, int Hk, int K, int V, bool use_bf16,
                             const void* ws, hipStream_t stream)
{
    if (!cu) n_seqs = 0;
    if (use_bf16)
        return K == 128 ? launch_scan_t<bf16, 128>(q, k, qks, v, vs, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, ws, stream)
                        : launch_scan_t<bf16, 64>(q, k, qks, v, vs, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, ws, stream);
    return K == 128 ? launch_scan_t<float, 128>(q, k, qks, v, vs, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, ws, stream)
                    : launch_scan_t<float, 64>(q, k, qks, v, vs, S0, Sf, o, cu, n_seqs, B, T_len, H, Hk, V, ws, stream);
}

}  // namespace gdn
