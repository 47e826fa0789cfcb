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
// through a second LDS buffer. Both are double-buffered with a register
// prefetch, one barrier per (tap, chunk) stage.
//
// MFMA: bfloat16 inputs use v_mfma_f32_32x32x16_bf16 (each lane supplies 8
// consecutive channels of one row of each operand), float32 inputs use
// v_mfma_f32_32x32x2_f32 (each lane reads 4 consecutive channels and feeds
// them to 4 MFMAs; A and B pair the same channel in every lane, so the sum
// is the full reduction). Operand A is the weight tile (rows = co), operand B
// the gathered inputs (columns = positions), so the accumulator columns are
// positions and each store instruction writes runs of consecutive outputs.
//
// Epilogue: acc + bias[co] in float32, one rounding to the output type,
// stored to y[b][g*Cog+co][s*q + r] (masked to the phase's q range).
#include "kcommon.h"
#include "launch.h"

namespace convt {

template <typename T> struct GemmCfg;
template <> struct GemmCfg<uint16_t> {
    static constexpr int BM = tiles::kGemmBM_bf16, BN = tiles::kGemmBN, BK = tiles::kGemmBK_bf16;
    static constexpr int VEC = 8;  // elements per 16-byte vector
};
template <> struct GemmCfg<float> {
    static constexpr int BM = tiles::kGemmBM_f32, BN = tiles::kGemmBN, BK = tiles::kGemmBK_f32;
    static constexpr int VEC = 4;
};

template <typename T>
__global__ __launch_bounds__(256, 2) void phase_gemm_kernel(DevParams p, const T *__restrict__ x,
                                                            const T *__restrict__ wr,
                                                            const T *__restrict__ bias,
                                                            T *__restrict__ y) {
    using C = GemmCfg<T>;
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, VEC = C::VEC;
    constexpr int LDK = BK + VEC;  // LDS row: BK channels + 16 bytes of padding
    constexpr int NKV = BK / VEC;  // 16-byte vectors per row
    constexpr int HALO = tiles::kGemmHaloMax;
    constexpr int XITEMS = (HALO * NKV + 255) / 256;
    constexpr int WVEC = BM * NKV / 256;
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MT = WM / 32, NT = WN / 32;
    static_assert(WVEC * 256 == BM * NKV, "weight tile must split evenly over the block");

    __shared__ __attribute__((aligned(16))) T xs[2][HALO * LDK];
    __shared__ __attribute__((aligned(16))) T ws[2][BM * LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    const int h00 = q00 + a0.off0[ph.r[0]];
    const int h01 = q01 + a1.off0[ph.r[1]];
    const int h02 = q02 + a2.off0[ph.r[2]];

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.0f;

    const int ntaps = ph.ntaps;
    const int nchunks = p.cig_pad / BK;
    const int nst = ntaps * nchunks;

    if (nst > 0) {
        // --- per-thread halo items: (row, 16-byte channel vector) pairs ---
        int lds_off[XITEMS], in_off[XITEMS], kvv[XITEMS];
#pragma unroll
        for (int i = 0; i < XITEMS; ++i) {
            const int it = tid + 256 * i;
            lds_off[i] = -1;
            in_off[i] = -1;
            kvv[i] = 0;
            if (it < hsz * NKV) {
                const int kv = it / hsz, row = it - kv * hsz;
                const int c2 = row % E2, c1 = (row / E2) % E1, c0 = row / (E2 * E1);
                const int i0 = h00 + c0, i1 = h01 + c1, i2 = h02 + c2;
                lds_off[i] = row * LDK + kv * VEC;
                kvv[i] = kv * VEC;
                if (i0 >= 0 && i0 < a0.I && i1 >= 0 && i1 < a1.I && i2 >= 0 && i2 < a2.I)
                    in_off[i] = (i0 * a1.I + i1) * a2.I + i2;
            }
        }
        const T *xg = x + ((int64_t)b * p.Ci + (int64_t)g * p.Cig) * p.x_plane;
        const int64_t xpl = p.x_plane;
        const int Cig = p.Cig;
        u32x4 xr[XITEMS];
        auto load_x = [&](int chunk) {
#pragma unroll
            for (int i = 0; i < XITEMS; ++i) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (in_off[i] >= 0) {
                    const int cb = chunk * BK + kvv[i];
                    const T *src = xg + (int64_t)cb * xpl + in_off[i];
                    if constexpr (sizeof(T) == 2) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t lo = (cb + 2 * e < Cig) ? (uint32_t)src[(2 * e) * xpl] : 0u;
                            const uint32_t hi =
                                (cb + 2 * e + 1 < Cig) ? (uint32_t)src[(2 * e + 1) * xpl] : 0u;
                            v[e] = lo | (hi << 16);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = (cb + e < Cig) ? __float_as_uint((float)src[e * xpl]) : 0u;
                    }
                }
                xr[i] = v;
            }
        };
        auto store_x = [&](int buf) {
#pragma unroll
            for (int i = 0; i < XITEMS; ++i)
                if (lds_off[i] >= 0) *(u32x4 *)&xs[buf][lds_off[i]] = xr[i];
        };

        // --- weight tiles ---
        const T *wb = wr + ((int64_t)(g * p.ktot + ph.tapbase) * p.cog_pad + co_t * BM) * p.cig_pad;
        const int64_t tap_stride = (int64_t)p.cog_pad * p.cig_pad;
        u32x4 wrg[WVEC];
        auto load_w = [&](int t, int chunk) {
            const T *src = wb + (int64_t)t * tap_stride + chunk * BK;
#pragma unroll
            for (int i = 0; i < WVEC; ++i) {
                const int v = tid + 256 * i, m = v / NKV, kv = v % NKV;
                wrg[i] = *(const u32x4 *)(src + (int64_t)m * p.cig_pad + kv * VEC);
            }
        };
        auto store_w = [&](int buf) {
#pragma unroll
            for (int i = 0; i < WVEC; ++i) {
                const int v = tid + 256 * i, m = v / NKV, kv = v % NKV;
                *(u32x4 *)&ws[buf][m * LDK + kv * VEC] = wrg[i];
            }
        };

        // --- operand rows of this lane ---
        int brow[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n = wn * WN + nt * 32 + (lane & 31);
            const int c2 = n % T2, c1 = (n / T2) % T1, c0 = n / (T2 * T1);
            brow[nt] = (c0 * E1 + c1) * E2 + c2;
        }
        const int kofs = (lane >> 5) * VEC;
        const int n1 = ph.n[1], n2 = ph.n[2];
        const int os0 = a0.ostep, os1 = a1.ostep, os2 = a2.ostep;

        auto compute = [&](int xbuf, int wbuf, int t) {
            const int j2 = t % n2, j1 = (t / n2) % n1, j0 = t / (n2 * n1);
            const int delta = ((j0 * os0) * E1 + j1 * os1) * E2 + j2 * os2;
            const T *xsb = xs[xbuf];
            const T *wsb = ws[wbuf];
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int ks = 0; ks < BK / 16; ++ks) {
                    bf16x8 A[MT], Bv[NT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        A[mt] = __builtin_bit_cast(
                            bf16x8, *(const u32x4 *)&wsb[(wm * WM + mt * 32 + (lane & 31)) * LDK +
                                                         ks * 16 + kofs]);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        Bv[nt] = __builtin_bit_cast(
                            bf16x8, *(const u32x4 *)&xsb[(brow[nt] + delta) * LDK + ks * 16 + kofs]);
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
                        A[mt] = *(const f32x4 *)&wsb[(wm * WM + mt * 32 + (lane & 31)) * LDK +
                                                     kq * 8 + kofs];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        Bv[nt] = *(const f32x4 *)&xsb[(brow[nt] + delta) * LDK + kq * 8 + kofs];
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
        for (int s = 0; s < nst; ++s) {
            const int chunk = s / ntaps, t = s - chunk * ntaps;
            const int s1 = s + 1;
            const bool has_next = s1 < nst;
            int c1 = 0;
            bool new_chunk = false;
            if (has_next) {
                c1 = s1 / ntaps;
                const int t1 = s1 - c1 * ntaps;
                new_chunk = (t1 == 0);
                load_w(t1, c1);
                if (new_chunk) load_x(c1);
            }
            compute(chunk & 1, s & 1, t);
            if (has_next) {
                store_w(s1 & 1);
                if (new_chunk) store_x(c1 & 1);
            }
            __syncthreads();
        }
    }

    // --- epilogue: bias, one rounding, masked strided stores ---
    int yoff[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = wn * WN + nt * 32 + (lane & 31);
        const int c2 = n % T2, c1 = (n / T2) % T1, c0 = n / (T2 * T1);
        const int qd = q00 + c0, qh = q01 + c1, qw = q02 + c2;
        yoff[nt] = -1;
        if (qd < a0.qn[ph.r[0]] && qh < a1.qn[ph.r[1]] && qw < a2.qn[ph.r[2]]) {
            const int o0 = a0.S * qd + ph.r[0], o1 = a1.S * qh + ph.r[1], o2 = a2.S * qw + ph.r[2];
            yoff[nt] = (o0 * a1.O + o1) * a2.O + o2;
        }
    }
    T *yb = y + ((int64_t)b * p.Co + (int64_t)g * p.Cog) * p.y_plane;
    const int co_base = co_t * BM + wm * WM;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int co = co_base + mt * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            if (co < p.Cog) {
                const float bv = p.has_bias ? to_f32(bias[g * p.Cog + co]) : 0.0f;
                T *yp = yb + (int64_t)co * p.y_plane;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    if (yoff[nt] >= 0) yp[yoff[nt]] = from_f32<T>(acc[mt][nt][j] + bv);
            }
        }
    }
}

hipError_t launch_phase_gemm(const Plan &pl, const void *x, const void *wr, const void *bias,
                             void *y, hipStream_t stream) {
    const DevParams &p = pl.dp;
    if (p.n_blocks <= 0) return hipSuccess;
    if (pl.elem_bytes == 2)
        hipLaunchKernelGGL(phase_gemm_kernel<uint16_t>, dim3(p.n_blocks), dim3(256), 0, stream, p,
                           (const uint16_t *)x, (const uint16_t *)wr, (const uint16_t *)bias,
                           (uint16_t *)y);
    else
        hipLaunchKernelGGL(phase_gemm_kernel<float>, dim3(p.n_blocks), dim3(256), 0, stream, p,
                           (const float *)x, (const float *)wr, (const float *)bias, (float *)y);
    return hipGetLastError();
}

}  // namespace convt
