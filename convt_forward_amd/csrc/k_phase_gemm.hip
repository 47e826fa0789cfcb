// Stride-phase implicit-gather GEMM on MFMA (gfx950).
//
// Splitting the scatter y[i*s - p + kk*d] += x[i]*w[kk] by output residue
// turns each stride phase into a dense correlation over q (output s*q + r
// gathers x[q + off(kk)] * w[kk] over the phase's taps), so no zero-inserted
// input is formed and no scatter pass runs. For one phase P, batch b and
// group g this is the GEMM
//     D[co][q] = sum over (tap, ci) of Wr[g][P][tap][co][ci] * x[b][g*Cig+ci][q + off(tap)]
// whose reduction spans the full in-channel-by-tap depth, with out-of-range
// inputs read as zero (the implicit padding). This is the implicit-gather
// GEMM the huggingface ai.onnx.ConvTranspose page describes for its stride-1
// variant ("ncdhw3d_implicit_sgmat": input windows read directly, outputs
// stored directly, no column matrix), extended here to every stride through
// the phase split its stride-phase variants name.
//
// Block: 256 threads (4 waves, 2 x 2), BM output channels x BN positions of
// one phase. The BN positions form a (td, th, tw) box in q space; for each
// chunk of BK input channels the block stages the box's input halo (the box
// grown by the phase's tap span) in LDS, transposed to channel-contiguous
// rows, and reuses it for every tap of the phase: tap t reads the halo rows
// shifted by its offset. Weight tiles [BM][BK] per (tap, chunk) stream
// through a second LDS buffer. Both are double-buffered: the halo of chunk
// c+1 is requested when chunk c starts, the weight tile of the next stage
// one stage ahead; one barrier per (tap, chunk) stage.
//
// Loads and stores go through raw buffer resources, whose range check
// returns zero for reads (and drops writes) past the resource's size: x is
// read through a resource that ends at the last input channel of the group,
// so a ragged channel chunk reads zeros, and positions outside the input use
// an offset of 2^31, always out of range. Every per-lane offset is a
// 32-bit byte offset fixed per block; the per-stage parts are uniform.
//
// MFMA: bfloat16 inputs use v_mfma_f32_32x32x16_bf16 (each lane supplies 8
// consecutive channels of one row of each operand), float32 inputs use
// v_mfma_f32_32x32x2_f32 (each lane reads 4 consecutive channels and feeds
// them to 4 MFMAs; A and B pair the same channel in every lane, so the sum
// is the full reduction). Operand A is the weight tile (rows = co), operand B
// the gathered inputs (columns = positions), so the accumulator columns are
// positions and each store instruction writes runs of consecutive outputs.
//
// Epilogue: acc + bias[co] in float32, one rounding to the output type
// (v_cvt_pk_bf16_f32 rounds to nearest even), stored to
// y[b][g*Cog+co][s*q + r]; outputs beyond the phase's q range or past Cog
// fall outside the store resource and are dropped.
#include "kcommon.h"
#include "launch.h"

namespace convt {

template <typename T, int CFG> struct GemmCfg {
    static constexpr int BM = tiles::kGemmCfg[CFG].bm, BN = tiles::kGemmCfg[CFG].bn;
    static constexpr int BK = tiles::kGemmCfg[CFG].bk, HALO = tiles::kGemmCfg[CFG].halo;
    static constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte vector
    static_assert(BK == (sizeof(T) == 2 ? 32 : 16), "tile config does not match the element type");
};

// Buffer resource word 3 for gfx9-family raw buffers.
constexpr int kRsrcWord3 = 0x00020000;
// A byte offset that is out of range for every resource used here (each
// covers less than 2^31 bytes), also after adding a channel offset.
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

template <typename T, int CFG>
__global__ __launch_bounds__(256) void phase_gemm_kernel(DevParams p, const T *__restrict__ x,
                                                         const T *__restrict__ wr,
                                                         const T *__restrict__ bias,
                                                         T *__restrict__ y) {
    using C = GemmCfg<T, CFG>;
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, VEC = C::VEC;
    constexpr int ES = (int)sizeof(T);
    constexpr int LDK = BK + VEC;  // LDS row: BK channels + 16 bytes of padding
    constexpr int NKV = BK / VEC;  // 16-byte vectors per row
    constexpr int HALO = C::HALO;
    constexpr int XITEMS = (HALO * NKV + 255) / 256;
    constexpr int WVEC = BM * NKV / 256;
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MT = WM / 32, NT = WN / 32;
    static_assert(WVEC * 256 == BM * NKV, "weight tile must split evenly over the block");

    __shared__ __attribute__((aligned(16))) T xs[2][HALO * LDK];
    __shared__ __attribute__((aligned(16))) T ws[2][BM * LDK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int wm = wave >> 1, wn = wave & 1;

    int bid = remap_block(blockIdx.x, p.n_blocks, p.xcd_remap);
    const int co_t = bid % p.n_co_tiles;
    bid /= p.n_co_tiles;
    const int P = bid % p.nphase;
    bid /= p.nphase;
    const int tw_i = bid % p.nt_w;
    bid /= p.nt_w;
    const int th_i = bid % p.nt_h;
    bid /= p.nt_h;
    const int td_i = bid % p.nt_d;
    bid /= p.nt_d;
    const int g = bid % p.G;
    const int b = bid / p.G;

    const PhaseDesc ph = phase_desc(p, P);
    const DevAxis &a0 = p.ax[0], &a1 = p.ax[1], &a2 = p.ax[2];
    const int T0 = p.td, T1 = p.th, T2 = p.tw;
    const int q00 = td_i * T0, q01 = th_i * T1, q02 = tw_i * T2;
    // this phase's halo box: the q box grown by its tap span, starting at the
    // phase's smallest input offset
    const int E0 = T0 + (ph.n[0] > 0 ? (ph.n[0] - 1) * a0.ostep : 0);
    const int E1 = T1 + (ph.n[1] > 0 ? (ph.n[1] - 1) * a1.ostep : 0);
    const int E2 = T2 + (ph.n[2] > 0 ? (ph.n[2] - 1) * a2.ostep : 0);
    const int hsz = E0 * E1 * E2;
    const int h00 = q00 + ph.off0[0];
    const int h01 = q01 + ph.off0[1];
    const int h02 = q02 + ph.off0[2];

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.0f;

    const int ntaps = ph.ntaps;
    const int nchunks = p.cig_pad / BK;
    const int Cig = p.Cig;
    const uint32_t xpl_bytes = (uint32_t)p.x_plane * ES;

    if (ntaps > 0) {
        // --- per-thread halo items: (row, 16-byte channel vector) pairs ---
        // xoff: byte offset of the item's first channel at its position,
        // relative to the chunk's first channel; out of range outside the input.
        const int nitems = hsz * NKV;
        uint32_t xoff[XITEMS];
        int lds_off[XITEMS];
#pragma unroll
        for (int i = 0; i < XITEMS; ++i) {
            const int it = tid + 256 * i;
            lds_off[i] = -1;
            xoff[i] = kOutOfRange;
            if (it < nitems) {
                const int kv = it / hsz, row = it - kv * hsz;
                const int c2 = row % E2, c1 = (row / E2) % E1, c0 = row / (E2 * E1);
                const int i0 = h00 + c0, i1 = h01 + c1, i2 = h02 + c2;
                lds_off[i] = row * LDK + kv * VEC;
                if (i0 >= 0 && i0 < a0.I && i1 >= 0 && i1 < a1.I && i2 >= 0 && i2 < a2.I)
                    xoff[i] = (uint32_t)(kv * VEC) * xpl_bytes +
                              (uint32_t)((i0 * a1.I + i1) * a2.I + i2) * ES;
            }
        }
        const T *xslice = x + ((int64_t)b * p.Ci + (int64_t)g * Cig) * p.x_plane;
        u32x4 xr[XITEMS];
        auto load_x = [&](int chunk) __attribute__((always_inline)) {
            // resource from the chunk's first channel to the group's last one
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(xslice + (int64_t)chunk * BK * p.x_plane,
                          (uint32_t)(Cig - chunk * BK) * xpl_bytes);
#pragma unroll
            for (int i = 0; i < XITEMS; ++i) {
                if (i * 256 < nitems) {  // uniform: skip items no lane holds
                    if constexpr (ES == 2) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
                                rs, xoff[i] + (2 * e) * xpl_bytes, 0, 0);
                            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
                                rs, xoff[i] + (2 * e + 1) * xpl_bytes, 0, 0);
                            xr[i][e] = lo | (hi << 16);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            xr[i][e] =
                                __builtin_amdgcn_raw_buffer_load_b32(rs, xoff[i] + e * xpl_bytes, 0, 0);
                    }
                }
            }
        };
        auto store_x = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < XITEMS; ++i)
                if (i * 256 < nitems && lds_off[i] >= 0) *(u32x4 *)&xs[buf][lds_off[i]] = xr[i];
        };

        // --- weight tiles: lanes take 16-byte vectors row by row ---
        const uint32_t tap_bytes = (uint32_t)p.cog_pad * p.cig_pad * ES;
        const __amdgpu_buffer_rsrc_t wrs =
            make_rsrc(wr + (int64_t)(g * p.ktot + ph.tapbase) * p.cog_pad * p.cig_pad,
                      (uint32_t)ntaps * tap_bytes);
        uint32_t woff[WVEC];
        int wlds[WVEC];
#pragma unroll
        for (int i = 0; i < WVEC; ++i) {
            const int v = tid + 256 * i, m = v / NKV, kv = v % NKV;
            woff[i] = (uint32_t)((co_t * BM + m) * p.cig_pad + kv * VEC) * ES;
            wlds[i] = m * LDK + kv * VEC;
        }
        u32x4 wrg[WVEC];
        auto load_w = [&](int t, int chunk) __attribute__((always_inline)) {
            const uint32_t soff = (uint32_t)t * tap_bytes + (uint32_t)(chunk * BK * ES);
#pragma unroll
            for (int i = 0; i < WVEC; ++i)
                wrg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, woff[i], soff, 0));
        };
        auto store_w = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < WVEC; ++i) *(u32x4 *)&ws[buf][wlds[i]] = wrg[i];
        };

        // --- operand rows of this lane ---
        int brow[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n = wn * WN + nt * 32 + (lane & 31);
            const int c2 = n % T2, c1 = (n / T2) % T1, c0 = n / (T2 * T1);
            brow[nt] = ((c0 * E1 + c1) * E2 + c2) * LDK + (lane >> 5) * VEC;
        }
        const int arow = (wm * WM + (lane & 31)) * LDK + (lane >> 5) * VEC;
        const int n1 = ph.n[1], n2 = ph.n[2];
        const int dstep2 = a2.ostep * LDK, dstep1 = a1.ostep * E2 * LDK,
                  dstep0 = a0.ostep * E1 * E2 * LDK;

        auto compute = [&](int xbuf, int wbuf, int delta) __attribute__((always_inline)) {
            const T *xsb = xs[xbuf] + delta;
            const T *wsb = ws[wbuf] + arow;
            if constexpr (ES == 2) {
#pragma unroll
                for (int ks = 0; ks < BK / 16; ++ks) {
                    bf16x8 A[MT], Bv[NT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        A[mt] = __builtin_bit_cast(bf16x8,
                                                   *(const u32x4 *)&wsb[mt * 32 * LDK + ks * 16]);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        Bv[nt] = __builtin_bit_cast(bf16x8, *(const u32x4 *)&xsb[brow[nt] + ks * 16]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[mt], Bv[nt],
                                                                                  acc[mt][nt], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int kq = 0; kq < BK / 8; ++kq) {
                    f32x4 A[MT], Bv[NT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        A[mt] = *(const f32x4 *)&wsb[mt * 32 * LDK + kq * 8];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        Bv[nt] = *(const f32x4 *)&xsb[brow[nt] + kq * 8];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                            for (int nt = 0; nt < NT; ++nt)
                                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                    A[mt][i], Bv[nt][i], acc[mt][nt], 0, 0, 0);
                }
            }
        };

        // --- pipeline over (chunk, tap) stages ---
        load_x(0);
        load_w(0, 0);
        store_x(0);
        store_w(0);
        __syncthreads();
        int chunk = 0, t = 0, j0 = 0, j1 = 0, j2 = 0, sb = 0;
        for (;;) {
            // next stage
            int t1 = t + 1, c1 = chunk;
            if (t1 == ntaps) {
                t1 = 0;
                ++c1;
            }
            const bool has_next = c1 < nchunks;
            const bool new_chunk_next = has_next && t1 == 0;
            if (t == 0 && chunk + 1 < nchunks) load_x(chunk + 1);
            if (has_next) load_w(t1, c1);
            compute(chunk & 1, sb, j0 * dstep0 + j1 * dstep1 + j2 * dstep2);
            if (has_next) store_w(sb ^ 1);
            if (new_chunk_next) store_x(c1 & 1);
            __syncthreads();
            if (!has_next) break;
            // tap counters of the next stage (taps in (j0, j1, j2) order)
            if (t1 == 0) {
                j0 = j1 = j2 = 0;
            } else if (++j2 == n2) {
                j2 = 0;
                if (++j1 == n1) {
                    j1 = 0;
                    ++j0;
                }
            }
            t = t1;
            chunk = c1;
            sb ^= 1;
        }
    }

    // --- epilogue: bias, one rounding, strided stores ---
    // per position: byte offset in the output plane, out of range if masked
    uint32_t yoff[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = wn * WN + nt * 32 + (lane & 31);
        const int c2 = n % T2, c1 = (n / T2) % T1, c0 = n / (T2 * T1);
        const int qd = q00 + c0, qh = q01 + c1, qw = q02 + c2;
        yoff[nt] = kOutOfRange;
        if (qd < ph.qn[0] && qh < ph.qn[1] && qw < ph.qn[2]) {
            const int o0 = a0.S * qd + ph.r[0], o1 = a1.S * qh + ph.r[1], o2 = a2.S * qw + ph.r[2];
            yoff[nt] = (uint32_t)((o0 * a1.O + o1) * a2.O + o2) * ES;
        }
    }
    const int co_w = co_t * BM + wm * WM;  // first output channel of this wave
    const uint32_t ypl_bytes = (uint32_t)p.y_plane * ES;
    // the group's output planes from this wave's first channel to Cog
    const int co_left = p.Cog - co_w;
    if (co_left > 0) {
        const __amdgpu_buffer_rsrc_t ys = make_rsrc(
            y + ((int64_t)b * p.Co + (int64_t)g * p.Cog + co_w) * p.y_plane,
            (uint32_t)co_left * ypl_bytes);
        const __amdgpu_buffer_rsrc_t bs =
            make_rsrc(bias + g * p.Cog + co_w, p.has_bias ? (uint32_t)co_left * ES : 0u);
        const uint32_t lane_co = 4 * (lane >> 5);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                // this lane's channel: mt*32 + 8*(j/4) + 4*(lane/32) + j%4
                const uint32_t co_u = mt * 32 + 8 * (j >> 2) + (j & 3);
                float bv;
                if constexpr (ES == 2)
                    bv = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(bs, (co_u + lane_co) * 2, 0, 0));
                else
                    bv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bs, (co_u + lane_co) * 4, 0, 0));
                const uint32_t cbytes = (co_u + lane_co) * ypl_bytes;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const float v = acc[mt][nt][j] + bv;
                    const uint32_t off = yoff[nt] + cbytes;
                    if constexpr (ES == 2)
                        __builtin_amdgcn_raw_buffer_store_b16(
                            __builtin_bit_cast(uint16_t, (__bf16)v), ys, off, 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ys, off, 0, 0);
                }
            }
        }
    }
}

template <typename T, int CFG>
static void launch_cfg(const DevParams &p, const void *x, const void *wr, const void *bias, void *y,
                       hipStream_t stream) {
    hipLaunchKernelGGL((phase_gemm_kernel<T, CFG>), dim3(p.n_blocks), dim3(256), 0, stream, p,
                       (const T *)x, (const T *)wr, (const T *)bias, (T *)y);
}

hipError_t launch_phase_gemm(const Plan &pl, const void *x, const void *wr, const void *bias,
                             void *y, hipStream_t stream) {
    const DevParams &p = pl.dp;
    if (p.n_blocks <= 0) return hipSuccess;
    switch (p.gemm_cfg) {
        case 0: launch_cfg<uint16_t, 0>(p, x, wr, bias, y, stream); break;
        case 1: launch_cfg<uint16_t, 1>(p, x, wr, bias, y, stream); break;
        case 2: launch_cfg<uint16_t, 2>(p, x, wr, bias, y, stream); break;
        case 3: launch_cfg<float, 3>(p, x, wr, bias, y, stream); break;
        case 4: launch_cfg<float, 4>(p, x, wr, bias, y, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace convt
