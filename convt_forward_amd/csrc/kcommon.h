// Device helpers shared by the kernels: element conversions, MFMA operand
// types, the phase/tap decoding of the plan tables, and the block-id remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "convt_internal.h"

namespace convt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// bfloat16 values travel as their 16-bit patterns.
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
    return __uint_as_float((uint32_t)v << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }

template <> __device__ __forceinline__ float to_f32<_Float16>(_Float16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) { return f32_to_bf16(v); }
// float32 -> IEEE half, round to nearest even
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float v) { return (_Float16)v; }

// Two-byte element types travel as 16-bit patterns; E (__bf16 or _Float16)
// is the arithmetic type they hold. Conversions round to nearest even.
template <typename E> __device__ __forceinline__ float half_to_f32(uint16_t v) {
    return (float)__builtin_bit_cast(E, v);
}
template <typename E> __device__ __forceinline__ uint16_t f32_to_half(float v) {
    return __builtin_bit_cast(uint16_t, (E)v);
}
// two float32 -> two E (RNE) in one word, the first value in the low half
template <typename E> __device__ __forceinline__ uint32_t pack_half2(float a, float b) {
    typedef E e2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, e2));
}

// 1 / (1 + e^-v) from e^-v = 2^(-v * log2 e) on the hardware exp2 and
// reciprocal instructions (each within about 1 ulp); the relative error of
// the result grows like |v| * 2^-24 through the product, below the
// pre-activation error the outputs already carry for any |v| it matters at.
__device__ __forceinline__ float logistic(float v) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
}

// tanh from e = e^(-2|v|) in (0, 1] (hardware exp2 and reciprocal):
// tanh|v| = (1 - e) / (1 + e), the sign restored. Nothing overflows; near 0
// the absolute error is a few units of 2^-24.
__device__ __forceinline__ float tanh_exp2(float v) {
    const float e = __builtin_amdgcn_exp2f(fabsf(v) * -2.8853900817779268f);  // -2 log2(e)
    return copysignf((1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e), v);
}

// erf by the rational approximation of Abramowitz and Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (due to Hastings): for x >= 0,
// erf x = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) e^(-x^2) with
// t = 1 / (1 + p x), absolute error at most 1.5e-7; odd in x.
__device__ __forceinline__ float erf_as7126(float x) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
    const float poly =
        t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float e = __builtin_amdgcn_exp2f(ax * ax * -1.4426950408889634f);  // e^(-x^2)
    return copysignf(1.0f - poly * e, x);
}

// The activation applied to an output after its bias (convt_activation),
// in float32. LOWP: the output is then rounded to a two-byte type (relative
// step 2^-8 or 2^-11), so tanh and erf take the short forms above, whose
// errors (below 1.5e-7 absolute) vanish in that rounding; float32 outputs
// use the device library's tanhf / erff. The short forms matter where
// outputs are cheap: an HBM-bound kernel has a few dozen VALU cycles per
// wave-wide output instruction.
template <bool LOWP = false>
__device__ __forceinline__ float activate(int act, float v) {
    switch (act) {
        case CONVT_ACT_RELU: return v > 0.0f ? v : 0.0f;
        case CONVT_ACT_SIGMOID: return logistic(v);
        case CONVT_ACT_TANH:
            if constexpr (LOWP)
                return tanh_exp2(v);
            else
                return tanhf(v);
        case CONVT_ACT_SILU: return v * logistic(v);
        case CONVT_ACT_GELU:
            if constexpr (LOWP)
                return 0.5f * v * (1.0f + erf_as7126(v * 0.7071067811865476f));
            else
                return 0.5f * v * (1.0f + erff(v * 0.7071067811865476f));
        default: return v;
    }
}

// The 8 XCDs take hardware block ids round-robin. With the remap, XCD k runs
// logical blocks [k*n/8, (k+1)*n/8), so blocks that share input tiles or
// weight slices share one L2. Requires n % 8 == 0.
__device__ __forceinline__ int remap_block(int bid, int n, int enable) {
    return enable ? (bid % 8) * (n / 8) + bid / 8 : bid;
}

// Phase P (lexicographic over the per-axis residues) of a plan, unpacked
// from its table record (one scalar load).
struct PhaseDesc {
    int r[3];      // residue per axis
    int n[3];      // taps per axis
    int qn[3];     // q count per axis
    int off0[3];   // first (smallest) input offset per axis
    int ntaps;     // product of n
    int tapbase;   // index of the phase's first tap in the reordered weights
};

__device__ __forceinline__ PhaseDesc phase_desc(const DevParams &p, int P) {
    const PhaseRec rec = p.ph[P];
    PhaseDesc ph;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        ph.r[a] = rec.rn[a] & 0xff;
        ph.n[a] = rec.rn[a] >> 8;
        ph.qn[a] = rec.qo[a] & 0xffff;
        ph.off0[a] = rec.qo[a] >> 16;  // arithmetic shift keeps the sign
    }
    ph.ntaps = rec.ntaps;
    ph.tapbase = rec.tapbase;
    return ph;
}

// Index, in the reordered weights, of the tap (k0, k1, k2) of the forward
// kernel: its phase's tapbase plus its rank within the phase.
__device__ __forceinline__ int tap_global(const DevParams &p, int k0, int k1, int k2) {
    int kk[3] = {k0, k1, k2};
    int r[3], j[3], n[3], cum[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const DevAxis &ax = p.ax[a];
        // residue of the outputs this tap reaches: r = (kk*d - p) mod s
        int v = (kk[a] * ax.D - ax.P) % ax.S;
        r[a] = v < 0 ? v + ax.S : v;
        j[a] = (ax.kk0[r[a]] - kk[a]) / ax.kstep;
        n[a] = ax.n[r[a]];
        cum[a] = ax.cum[r[a]];
    }
    const int tapbase = cum[0] * p.ax[1].K * p.ax[2].K + n[0] * (cum[1] * p.ax[2].K + n[1] * cum[2]);
    return tapbase + (j[0] * n[1] + j[1]) * n[2] + j[2];
}

// Index of tap (k0, k1, k2) when phase P's taps start at ph[P].tapbase (the
// phase GEMM's layout, where each phase is padded to whole tap groups).
__device__ __forceinline__ int tap_in_table(const DevParams &p, int k0, int k1, int k2) {
    int kk[3] = {k0, k1, k2};
    int r[3], j[3], n[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const DevAxis &ax = p.ax[a];
        int v = (kk[a] * ax.D - ax.P) % ax.S;
        r[a] = v < 0 ? v + ax.S : v;
        j[a] = (ax.kk0[r[a]] - kk[a]) / ax.kstep;
        n[a] = ax.n[r[a]];
    }
    const int P = (r[0] * p.ax[1].S + r[1]) * p.ax[2].S + r[2];
    return p.ph[P].tapbase + (j[0] * n[1] + j[1]) * n[2] + j[2];
}

// Element offset in W of the weight from input channel ci (global) to output
// channel ocl of ci's group at forward tap kk (row-major over K0, K1, K2),
// for the filter layouts of convt.h; Ci, Co, Cig, Cog are the forward
// problem's channel counts.
__device__ __forceinline__ int64_t w_offset(int layout, int flip, int Ci, int Co, int Cig, int Cog,
                                            int K0, int K1, int K2, int ci, int ocl, int kk) {
    if (flip) {
        const int k2 = kk % K2, k1 = (kk / K2) % K1, k0 = kk / (K1 * K2);
        kk = ((K0 - 1 - k0) * K1 + (K1 - 1 - k1)) * K2 + (K2 - 1 - k2);
    }
    const int ktot = K0 * K1 * K2;
    if (layout == CONVT_FILTER_K_CI_CO) return ((int64_t)kk * Ci + ci) * Cog + ocl;
    if (layout == CONVT_FILTER_K_CO_CI) {
        const int g = ci / Cig;
        return ((int64_t)kk * Co + (int64_t)g * Cog + ocl) * Cig + (ci - g * Cig);
    }
    return ((int64_t)ci * Cog + ocl) * ktot + kk;
}
// The same for a forward problem's parameters.
__device__ __forceinline__ int64_t w_offset(const DevParams &p, int ci, int ocl, int kk) {
    return w_offset(p.w_layout, p.w_flip, p.Ci, p.Co, p.Cig, p.Cog, p.ax[0].K, p.ax[1].K, p.ax[2].K,
                    ci, ocl, kk);
}
// Whether W is in the default layout and orientation (the vector paths).
__device__ __forceinline__ bool w_plain(const DevParams &p) {
    return p.w_layout == CONVT_FILTER_CI_CO_K && !p.w_flip;
}

// ---- raw buffers and global -> LDS copies (phase GEMM, grouped kernel) ----

// Buffer resource word 3 for gfx9-family raw buffers.
constexpr uint32_t kRsrcWord3 = 0x00020000u;
// A byte offset that is out of range for every resource used here (each
// covers less than 2^31 bytes), also after adding a tap or chunk offset.
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             (int)kRsrcWord3);
}

// A resource whose base and size are the same in every lane, built from
// lane 0's words so that the compiler holds it in scalar registers (else a
// resource it cannot prove uniform is kept in vector registers and each
// access loops over the lanes' resources). The words are taken unsigned: a
// signed low word would be sign-extended into the high one.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void *base, uint32_t bytes,
                                                                    int word3 = (int)kRsrcWord3) {
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | (uint64_t)lo), (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), word3);
}

// The same resource as four scalar words, for the copy instructions below.
__device__ __forceinline__ u32x4 rsrc_words(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = kRsrcWord3;
    return r;
}


// Global -> LDS copies: every lane reads BYTES at its offset in the resource
// and writes them at lds + lane * max(BYTES, 4). Out-of-range reads write
// zeros. Issued as plain instructions so that the compiler neither waits for
// them nor reorders them with the barriers; completion is awaited by the
// counts of stage_barrier. They set M0, a register the compiler reserves and
// does not otherwise use in the kernels that call these.
template <int BYTES>
__device__ __forceinline__ void copy_to_lds(uint32_t lds, uint32_t voff, const u32x4 &rs) {
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     ::"s"(lds), "v"(voff), "s"(rs));
    else if constexpr (BYTES == 4)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                     ::"s"(lds), "v"(voff), "s"(rs));
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_ushort %1, %2, 0 offen lds"
                     ::"s"(lds), "v"(voff), "s"(rs));
}

// Wait until at most N vector-memory operations of this wave are in flight
// and its LDS operations are done, then join the block's barrier. The
// memory clobber keeps the compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void stage_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// The same with a wave-uniform count n (clamped to MAXN).
template <int MAXN>
__device__ __forceinline__ void stage_barrier_n(int n) {
    if constexpr (MAXN > 0) {
        if (n >= MAXN) {
            stage_barrier<MAXN>();
            return;
        }
        stage_barrier_n<MAXN - 1>(n);
    } else {
        stage_barrier<0>();
    }
}

// 32-bit words of two-byte elements: the low halves of a and b, or their
// high halves, as one word (a's in the low half).
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// a / b for 0 <= a < 2^22 and 0 < b < 2^16 through a float32 reciprocal,
// corrected to the exact quotient (the estimate is within one of it).
__device__ __forceinline__ int div_small(int a, int b) {
    int q = (int)((float)a * __builtin_amdgcn_rcpf((float)b));
    if (q * b > a) --q;
    else if ((q + 1) * b <= a) ++q;
    return q;
}

// The box position (within a 32-position operand fragment) that lane i
// (0..31) reads when the box rows are 16 positions long, so that a fragment
// covers two box rows: lanes 0-7 and 24-31 the first (columns 0-7, 8-15),
// lanes 8-23 the second. With the rows 24 x 16 bytes apart in LDS, a wave's
// 16-byte reads of such a fragment then meet no bank conflict (measured on
// gfx950 with an LDS probe under rocprofv3: lanes 0-15 on the first row
// conflict two-way at every row pitch that is not a multiple of 16 rows).
__device__ __forceinline__ int frag16_pos(int i) {
    const int q = i >> 3;
    return ((q == 1 || q == 2) ? 16 : 0) + (i & 7) + ((q >> 1) << 3);
}

// n / d for any 32-bit n through the multiplier the planner derives for d
// (FastDiv): q = (mulhi(n, m) + n) >> s in 33-bit arithmetic.
__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
    const uint64_t t = (uint64_t)__umulhi(n, f.m) + n;
    return (uint32_t)(t >> f.s);
}

}  // namespace convt
