// gdn_common.hpp -- device helpers for the gfx950 (CDNA4) kernels.
//
// Element types, 16-byte vector access, wave64 reductions, and the MFMA
// fragment conventions used by the chunk kernels.
//
// MFMA conventions (v_mfma_f32_16x16x32_bf16 for bf16 operands and
// v_mfma_f32_16x16x4f32, eight times, for fp32 operands), for lane l with
// grp = l >> 4 and col = l & 15:
//   * accumulator D (16 x 16 fp32): lane holds D[4*grp + e][col], e = 0..3;
//   * A operand (16 rows x 32 contraction): lane supplies row `col`;
//   * B operand (32 contraction x 16 cols): lane supplies column `col`.
// Inside one 32-wide contraction block a lane's eight operand slots stand for
// the contraction indices  4*grp + {0,1,2,3}  and  16 + 4*grp + {0,1,2,3}.
// The product only needs A and B to agree on that assignment, and with it a
// pair of accumulator tiles covering contraction rows [0,16) and [16,32) IS a
// B operand: no LDS round trip is needed to feed a result (the state h, the
// corrected values U) into the next product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kChunk = 64;      // timesteps per chunk ([ZZ] item 2: 64-timestep chunks)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// 16 bytes of elements: 8 x bf16 or 4 x fp32.
template <typename T> struct V16;
template <> struct V16<bf16> {
    static constexpr int n = 8;
    typedef bf16x8 type;
    typedef f32x8 ftype;
    static __device__ __forceinline__ ftype to_float(type v) { return __builtin_convertvector(v, f32x8); }
    static __device__ __forceinline__ type from_float(ftype v) { return __builtin_convertvector(v, bf16x8); }
};
template <> struct V16<float> {
    static constexpr int n = 4;
    typedef f32x4 type;
    typedef f32x4 ftype;
    static __device__ __forceinline__ ftype to_float(type v) { return v; }
    static __device__ __forceinline__ type from_float(ftype v) { return v; }
};

// Lane moves within the wave that stay in the VALU (no LDS round trip): DPP
// patterns inside 4-, 8- and 16-lane rows, and gfx950's row / half-wave swaps.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141; // lane i of each 8 <- lane 7 - i
constexpr int kDppRowMirror = 0x140;  // lane i of each 16 <- lane 15 - i
constexpr int kDppRowBcast = 0x150;   // + n (row_newbcast): every lane of each 16 <- lane n of it

// Sum over aligned groups of `width` lanes (width a power of two <= 64); every
// lane of a group ends with the same value.
template <int width>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(width >= 1 && width <= 64 && (width & (width - 1)) == 0, "group width");
    if constexpr (width >= 2) v += dpp_mov<kDppQuadSwap1>(v);
    if constexpr (width >= 4) v += dpp_mov<kDppQuadSwap2>(v);
    if constexpr (width >= 8) v += dpp_mov<kDppHalfMirror>(v);
    if constexpr (width >= 16) v += dpp_mov<kDppRowMirror>(v);
    if constexpr (width >= 32) {
        // after the swap the two results hold rows (0, 0, 2, 2) and (1, 1, 3, 3)
        const int b = __builtin_bit_cast(int, v);
        const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
        v = __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
    }
    if constexpr (width >= 64) {
        const int b = __builtin_bit_cast(int, v);
        const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
        v = __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<kWave>(v); }

// Inclusive prefix sum over the 64 lanes (Hillis-Steele inside 16-lane rows,
// then the row totals carried across rows with row broadcasts).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
    const int r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, true);
    return v + __builtin_bit_cast(float, r);
}
__device__ __forceinline__ float wave_inclusive_scan(float v) {
    v = dpp_add<0x111, 0xf>(v);   // row_shr:1
    v = dpp_add<0x112, 0xf>(v);   // row_shr:2
    v = dpp_add<0x114, 0xf>(v);   // row_shr:4
    v = dpp_add<0x118, 0xf>(v);   // row_shr:8
    v = dpp_add<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}
__device__ __forceinline__ float lane_value(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// ---------------------------------------------------------------- MFMA

template <typename T> struct Mma;

template <> struct Mma<bf16> {
    typedef bf16x8 Frag;
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // Operand fragment of a row-major LDS matrix: row `row`, contraction block
    // starting at column c0; slots as described at the top of this file.
    static __device__ __forceinline__ Frag lds_frag(const bf16* m, int ld, int row, int c0, int grp) {
        const bf16* p = m + row * ld + c0 + 4 * grp;
        bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
        bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // B operand from two accumulator tiles covering contraction rows [0,16), [16,32).
    static __device__ __forceinline__ Frag acc_frag(f32x4 lo, f32x4 hi) {
        f32x8 f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_convertvector(f, bf16x8);
    }
};

template <> struct Mma<float> {
    typedef f32x8 Frag;
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
#pragma unroll
        for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ Frag lds_frag(const float* m, int ld, int row, int c0, int grp) {
        const float* p = m + row * ld + c0 + 4 * grp;
        f32x4 lo = *reinterpret_cast<const f32x4*>(p);
        f32x4 hi = *reinterpret_cast<const f32x4*>(p + 16);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    static __device__ __forceinline__ Frag acc_frag(f32x4 lo, f32x4 hi) {
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

// Gates of Megatron-Core API docs, "core.ssm.ops.gdp.decode_prepare"
// (introduction and the "softplus" entry): softplus is log1p(exp(x)) in fp32,
// the identity once x exceeds 20; beta = sigmoid(b); g = -exp(A_log) *
// softplus(a + dt_bias). Accurate device exp / log1p and IEEE division; every
// kernel that forms a gate uses these, so their results agree bit for bit.
__device__ __forceinline__ float gate_softplus(float x) { return x > 20.f ? x : log1pf(expf(x)); }
__device__ __forceinline__ float gate_beta(float b) { return 1.f / (1.f + expf(-b)); }
__device__ __forceinline__ float gate_g(float a, float A_log, float dt_bias) {
    return -expf(A_log) * gate_softplus(a + dt_bias);
}

// Short causal convolution of "ZzCompute" (PyTorch Helion Hackathon gallery),
// item 1 "Causal Conv1d", width 4: the taps w0..w3 multiply x[t-3] .. x[t]
// and are accumulated onto the bias in that order with fused multiply-adds;
// SiLU is z / (1 + exp(-z)) with the reciprocal from v_rcp_f32 (~1 ulp).
// Every kernel that applies the convolution uses these two, so they agree bit
// for bit.
__device__ __forceinline__ float conv_taps4(float w0, float w1, float w2, float w3, float bias,
                                            float xm3, float xm2, float xm1, float x0) {
    float acc = bias;
    acc = fmaf(w0, xm3, acc);
    acc = fmaf(w1, xm2, acc);
    acc = fmaf(w2, xm1, acc);
    acc = fmaf(w3, x0, acc);
    return acc;
}
__device__ __forceinline__ float conv_silu(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

// bf16 inputs and taps: the four products summed onto the bias as two
// two-term dot products (v_dot2_f32_bf16; a product of two bf16 values is
// exact in fp32). x01 packs (x[t-3], x[t-2]) and x23 (x[t-1], x[t]) as bf16
// pairs (low half first); w01 and w23 pack (w0, w1) and (w2, w3), which is how
// a channel's four taps lie in memory. Every bf16 kernel that applies the
// convolution uses this, so they agree bit for bit.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float conv_taps4_bf16(uint32_t w01, uint32_t w23, float bias,
                                                 uint32_t x01, uint32_t x23) {
    const float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x01),
                                                      __builtin_bit_cast(bf16x2, w01), bias, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x23),
                                           __builtin_bit_cast(bf16x2, w23), acc, false);
}
// (lo, hi) bf16 pair from the low (pair_lo) or high (pair_hi) halves of two
// words, each holding two channels: the same channel at two times
__device__ __forceinline__ uint32_t pair_lo(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}
// (lo's high half, hi's low half): the pair straddling two words of a
// sequence of bf16 values packed in time order
__device__ __forceinline__ uint32_t pair_mid(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_perm(hi, lo, 0x05040302u);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Index of the packed sequence containing token t: the largest i with
// cu[i] <= t (binary search over cu[0..n]); requires cu[0] <= t < cu[n].
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int n, int t) {
    int lo = 0, hi = n;  // invariant: cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
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

// Launch-configuration knobs (gdn_tune_set): 0 = automatic. They change how
// work is scheduled, never the arithmetic, so every setting gives the same
// bits. Read by the launchers on the host.
enum TuneKnob { kTuneScanTiles = 0, kTuneConvRun = 1, kTuneConvThreads = 2, kTuneScanForm = 3, kTuneKnobs = 4 };
extern int tune_knob[kTuneKnobs];

}  // namespace gdn
