// Weight reorder (phase GEMM layouts), the channel-chunked input copy, bias
// fill, the one-thread-per-output gather kernels and the small-channel direct
// kernels.
#include "kcommon.h"
#include "launch.h"

namespace convt {

// ---------------------------------------------------------------------------
// Weight reorder for the phase GEMM:
//     W[g*Cig + ci][co][kk] -> Wr[g][tap][chunk][co][32 bytes of ci]
// where tap is kk's index in the plan's tap order (phase by phase, each phase
// padded with zero taps to whole groups of gemm_gs), chunk = ci / BK (BK =
// 16 bfloat16 or 8 float32 channels), and the two 16-byte halves of a row
// swap places where bit 3 of co is set. Channels past Cig and rows past Cog
// are zero.
//
// A block owns one chunk, CO output channels and KT consecutive taps kk of
// W: it reads the BK runs W[ci][co0 .. co0 + CO)[kk0 .. kk0 + KT) with
// consecutive lanes on consecutive elements into LDS, then each lane
// assembles 16-byte destination halves (VEC channels of one (tap, co)) and
// stores them, consecutive lanes on consecutive co. The blocks of the first
// tap range also zero the padding taps of their (chunk, co) tile, and block P
// writes phase P's part of the per-tap halo shift table the GEMM reads (the
// grid may be smaller than the phase count: blocks then take every gridDim-th
// phase): entry tapbase(P) + t
// holds, for tap t of phase P in (j0, j1, j2) order, the shift of its input
// window within the phase's halo box in box positions,
// (j0 * ostep0 * E1 + j1 * ostep1) * E2 + j2 * ostep2 (E1, E2: the box
// extents of that phase), and 0 for the padding taps.
// ---------------------------------------------------------------------------
// (block `blk` of `nblk`; lds_raw: 32 * CO * KT + 4 * KT bytes)
template <typename T>
__device__ __forceinline__ void reorder_chunked_block(const DevParams &p, const T *__restrict__ w,
                                                      T *__restrict__ wr, int32_t *__restrict__ tab,
                                                      int CO, int KT, int vec_runs, int blk, int nblk,
                                                      unsigned char *lds_raw) {
    constexpr int VEC = 16 / sizeof(T), BK = 2 * VEC;
    const int ktot = p.ktot;
    const int nchunks = p.cig_pad / BK;
    const int nco = (p.cog_pad + CO - 1) / CO;
    const int nkt = (ktot + KT - 1) / KT;
    int bid = blk;
    const int kb = bid % nkt;
    bid /= nkt;
    const int cb = bid % nco;
    bid /= nco;
    const int c = bid % nchunks;
    const int g = bid / nchunks;
    const int co0 = cb * CO, kk0 = kb * KT;
    const int nk = ktot - kk0 < KT ? ktot - kk0 : KT;  // taps of this block
    T *brick = (T *)lds_raw;                              // [BK][CO][KT]
    int *dst_tap = (int *)(lds_raw + (size_t)BK * CO * KT * sizeof(T));
    const int K1 = p.ax[1].K, K2 = p.ax[2].K;
    // each tap's index in the plan order; computed while a lane's first
    // loads are in flight (the lookups are chains of dependent parameter
    // reads)
    auto tap_lookup = [&]() __attribute__((always_inline)) {
        for (int k = threadIdx.x; k < nk; k += 256) {
            const int kk = kk0 + k;
            dst_tap[k] = tap_in_table(p, kk / (K1 * K2), (kk / K2) % K1, kk % K2);
        }
    };
    // 1. load. With vec_runs (KT == ktot, whole 16-byte aligned runs, the
    // block's channels inside or wholly outside Cog), each channel's run
    // [co0, co0 + CO) x [0, ktot) moves as 16-byte vectors, 4 per lane in
    // flight; otherwise elements, 8 per lane in flight.
    const int n_in = BK * CO * nk;
    if (vec_runs) {
        const int nvr = CO * ktot * (int)sizeof(T) / 16;  // vectors of one channel's run
        const int nv = BK * nvr;
        auto load = [&](int v0, u32x4 *v) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int vi = v0 + 256 * u;
                const int i = vi / nvr, r = vi - i * nvr;
                const int ci = c * BK + i;
                v[u] = u32x4{0u, 0u, 0u, 0u};
                if (vi < nv && ci < p.Cig && co0 < p.Cog)
                    v[u] = ((const u32x4 *)(w + (((int64_t)g * p.Cig + ci) * p.Cog + co0) * ktot))[r];
            }
        };
        u32x4 v[4];
        load(threadIdx.x, v);
        tap_lookup();
        for (int v0 = threadIdx.x; v0 < nv; v0 += 256 * 4) {
            if (v0 != (int)threadIdx.x) load(v0, v);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int vi = v0 + 256 * u;
                if (vi < nv) {
                    const int i = vi / nvr, r = vi - i * nvr;
                    ((u32x4 *)(brick + (size_t)i * CO * KT))[r] = v[u];
                }
            }
        }
    } else {
        auto load = [&](int e0, T *v) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = e0 + 256 * u;
                const int i = e / (CO * nk), r = e - i * (CO * nk);
                const int col = r / nk, k = r - col * nk;
                const int ci = c * BK + i, co = co0 + col;
                const bool ok = e < n_in && ci < p.Cig && co < p.Cog;
                v[u] = w[ok ? w_offset(p, g * p.Cig + ci, co, kk0 + k) : 0];
                if (!ok) v[u] = from_f32<T>(0.0f);
            }
        };
        T v[8];
        load(threadIdx.x, v);
        tap_lookup();
        for (int e0 = threadIdx.x; e0 < n_in; e0 += 256 * 8) {
            if (e0 != (int)threadIdx.x) load(e0, v);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = e0 + 256 * u;
                if (e < n_in) {
                    const int i = e / (CO * nk), r = e - i * (CO * nk);
                    brick[(i * CO + r / nk) * KT + r % nk] = v[u];
                }
            }
        }
    }
    __syncthreads();
    // 2. destination halves: v = (k * CO + col) * 2 + half
    const int64_t chunk_elems = (int64_t)p.cog_pad * BK;
    T *wg = wr + (int64_t)g * p.ktot_pad * nchunks * chunk_elems + (int64_t)c * chunk_elems;
    const int n_out = nk * CO * 2;
    for (int v = threadIdx.x; v < n_out; v += 256) {
        const int half = v & 1, col = (v >> 1) % CO, k = (v >> 1) / CO;
        const int co = co0 + col;
        if (co >= p.cog_pad) continue;
        u32x4 out;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i0 = half * VEC + 2 * e;
                out[e] = (uint32_t)brick[(i0 * CO + col) * KT + k] |
                         ((uint32_t)brick[((i0 + 1) * CO + col) * KT + k] << 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = __float_as_uint((float)brick[((half * VEC + e) * CO + col) * KT + k]);
        }
        const int phys = half ^ ((co >> 3) & 1);
        *(u32x4 *)&wg[(int64_t)dst_tap[k] * nchunks * chunk_elems + (int64_t)co * BK + phys * VEC] = out;
    }
    // 3. padding taps of this (chunk, co) tile (none when every phase's tap
    // count is a whole number of groups)
    if (kb == 0 && p.ktot_pad != p.ktot) {
        const int gs = p.gemm_gs;
        for (int P = 0; P < p.nphase; ++P) {
            const int nt = p.ph[P].ntaps;
            const int npad = (nt + gs - 1) / gs * gs - nt;
            for (int v = threadIdx.x; v < npad * CO * 2; v += 256) {
                const int co = co0 + (v >> 1) % CO;
                if (co < p.cog_pad)
                    *(u32x4 *)&wg[(int64_t)(p.ph[P].tapbase + nt + (v >> 1) / CO) * nchunks * chunk_elems +
                                  (int64_t)co * BK + (v & 1) * VEC] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    // 4. the halo shift table: block P writes phase P's entries
    {
        const int gs = p.gemm_gs;
        for (int P = blk; P < p.nphase; P += nblk) {
            const PhaseDesc ph = phase_desc(p, P);
            const int padded = (ph.ntaps + gs - 1) / gs * gs;
            const int n1 = ph.n[1], n2 = ph.n[2];
            const int E1 = p.th + (n1 > 0 ? (n1 - 1) * p.ax[1].ostep : 0);
            const int E2 = p.tw + (n2 > 0 ? (n2 - 1) * p.ax[2].ostep : 0);
            for (int t = threadIdx.x; t < padded; t += 256) {
                int v = 0;
                if (t < ph.ntaps) {
                    const int j2 = t % n2, j1 = (t / n2) % n1, j0 = t / (n1 * n2);
                    v = (j0 * p.ax[0].ostep * E1 + j1 * p.ax[1].ostep) * E2 + j2 * p.ax[2].ostep;
                }
                tab[ph.tapbase + t] = v;
            }
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void reorder_chunked_kernel(DevParams p, const T *__restrict__ w,
                                                              T *__restrict__ wr,
                                                              int32_t *__restrict__ tab, int CO,
                                                              int KT, int vec_runs) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    reorder_chunked_block<T>(p, w, wr, tab, CO, KT, vec_runs, blockIdx.x, gridDim.x, lds_raw);
}

// Launch shape of a chunked weight reorder (forward or backward layout):
// the per-block extents (CO output channels or OCB channel columns, KT
// taps), whether whole runs move as 16-byte vectors, the grid and the LDS.
struct ReorderGrid {
    int a, KT, vec_runs;
    int64_t blocks;
    size_t lds;
};

static hipError_t reorder_chunked_grid(const Plan &pl, const void *w, ReorderGrid *r) {
    const DevParams &p = pl.dp;
    const int bk = 32 / pl.elem_bytes;
    if (p.cig_pad % bk) return hipErrorInvalidValue;
    // KT taps x CO output channels per block: at most 1024 (co, tap)
    // pairs, and CO halved while the grid has fewer than 1024 blocks
    const int KT = p.ktot < 256 ? p.ktot : 256;
    const int nkt = (p.ktot + KT - 1) / KT;
    const int64_t base = (int64_t)p.G * (p.cig_pad / bk) * nkt;
    int CO = 1024 / KT;
    if (CO < 1) CO = 1;
    if (CO > p.cog_pad) CO = p.cog_pad;
    while (CO > 1 && base * ((p.cog_pad + CO - 1) / CO) < 1024) CO /= 2;
    const int64_t run_bytes = (int64_t)CO * p.ktot * pl.elem_bytes;
    r->a = CO;
    r->KT = KT;
    r->vec_runs = p.w_layout == CONVT_FILTER_CI_CO_K && !p.w_flip && KT == p.ktot &&
                  run_bytes % 16 == 0 && ((int64_t)p.Cog * p.ktot * pl.elem_bytes) % 16 == 0 &&
                  p.Cog % CO == 0 && (uintptr_t)w % 16 == 0;
    r->blocks = base * ((p.cog_pad + CO - 1) / CO);
    r->lds = (size_t)32 * CO * KT + (size_t)4 * KT;
    if (r->blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    return hipSuccess;
}

hipError_t launch_reorder(const Plan &pl, const void *w, void *wr, hipStream_t stream) {
    const DevParams &p = pl.dp;
    if (p.wr_chunked) {
        ReorderGrid r;
        const hipError_t e = reorder_chunked_grid(pl, w, &r);
        if (e != hipSuccess) return e;
        if (r.blocks <= 0) return hipSuccess;
        int32_t *tab = (int32_t *)((char *)wr + pl.tab_offset);
        if (pl.elem_bytes == 2)
            hipLaunchKernelGGL(reorder_chunked_kernel<uint16_t>, dim3((unsigned)r.blocks), dim3(256), r.lds,
                               stream, p, (const uint16_t *)w, (uint16_t *)wr, tab, r.a, r.KT, r.vec_runs);
        else
            hipLaunchKernelGGL(reorder_chunked_kernel<float>, dim3((unsigned)r.blocks), dim3(256), r.lds,
                               stream, p, (const float *)w, (float *)wr, tab, r.a, r.KT, r.vec_runs);
        return hipGetLastError();
    }
    // every route that reorders W into the workspace uses the chunked layout
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Input re-layout for the bfloat16 phase GEMM:
//     x[b][g*Cig + ci][pos] -> xp[b][g][chunk][pos][16 channels]
// (32 bytes per position and chunk, channels past Cig zero), so that the GEMM
// copies a halo row of one chunk as two 16-byte pieces. One thread per
// (b, g, chunk, position): 16 two-byte loads, coalesced over the positions
// of a wave, and two 16-byte stores.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void pack_x_block(const DevParams &p, const uint16_t *__restrict__ x,
                                             uint16_t *__restrict__ xp, int ptiles, int blk) {
    const int nchunks = p.cig_pad / 16;
    const int64_t plane = p.x_plane;
    int bid = blk;
    const int pt = bid % ptiles;
    bid /= ptiles;
    const int c = bid % nchunks;
    bid /= nchunks;
    const int g = bid % p.G;
    const int b = bid / p.G;
    const int64_t pos = (int64_t)pt * 256 + threadIdx.x;
    if (pos >= plane) return;
    const uint16_t *src = x + ((int64_t)b * p.Ci + (int64_t)g * p.Cig + c * 16) * plane + pos;
    const int nch = p.Cig - c * 16;  // channels of this chunk inside the group (>= 1)
    uint32_t v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = e < nch ? src[e * plane] : 0u;
    u32x4 o0, o1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        o0[k] = v[2 * k] | (v[2 * k + 1] << 16);
        o1[k] = v[8 + 2 * k] | (v[9 + 2 * k] << 16);
    }
    u32x4 *dst = (u32x4 *)(xp + ((((int64_t)b * p.G + g) * nchunks + c) * plane + pos) * 16);
    dst[0] = o0;
    dst[1] = o1;
}

// The same re-layout for planes of a multiple of 8 positions (16-byte
// aligned channel rows), through LDS: a block owns (b, g, chunk) and 256
// positions; it reads the 16 channel rows with 16-byte loads (consecutive
// lanes on consecutive pieces of a row), and writes the 256 x 32-byte
// destination rows with 16-byte stores, consecutive lanes on consecutive
// 16 bytes.
constexpr int kPackRS = 256 + 2;  // LDS row stride (elements): 256 positions + 4 bytes
constexpr int kPackLdsBytes = 16 * kPackRS * 2;
__device__ __forceinline__ void pack_x8_block(const DevParams &p, const uint16_t *__restrict__ x,
                                              uint16_t *__restrict__ xp, int ptiles, int blk,
                                              uint16_t *tile) {
    constexpr int RS = kPackRS;
    const int nchunks = p.cig_pad / 16;
    const int64_t plane = p.x_plane;
    int bid = blk;
    const int pt = bid % ptiles;
    bid /= ptiles;
    const int c = bid % nchunks;
    bid /= nchunks;
    const int g = bid % p.G;
    const int64_t b = bid / p.G;
    const int64_t pos0 = (int64_t)pt * 256;
    const uint16_t *src = x + ((b * p.Ci + (int64_t)g * p.Cig + c * 16) * plane + pos0);
    const int nch = p.Cig - c * 16;  // channels of this chunk inside the group (>= 1)
    u32x4 v[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int idx = threadIdx.x + 256 * k, ch = idx / 32, pg = idx % 32;
        v[k] = ch < nch && pos0 + pg * 8 < plane ? *(const u32x4 *)(src + ch * plane + pg * 8)
                                                 : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int idx = threadIdx.x + 256 * k, ch = idx / 32, pg = idx % 32;
        uint32_t *row = (uint32_t *)&tile[ch * RS + pg * 8];  // 4-byte aligned (RS even)
#pragma unroll
        for (int e = 0; e < 4; ++e) row[e] = v[k][e];
    }
    __syncthreads();
    u32x4 *dst = (u32x4 *)(xp + (((b * p.G + g) * nchunks + c) * plane + pos0) * 16);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int idx = threadIdx.x + 256 * k, pos = idx / 2, half = idx % 2;
        if (pos0 + pos < plane) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = (uint32_t)tile[(half * 8 + 2 * e) * RS + pos] |
                       ((uint32_t)tile[(half * 8 + 2 * e + 1) * RS + pos] << 16);
            dst[idx] = o;
        }
    }
}

__global__ __launch_bounds__(256) void pack_x_kernel(DevParams p, const uint16_t *__restrict__ x,
                                                      uint16_t *__restrict__ xp, int ptiles) {
    pack_x_block(p, x, xp, ptiles, blockIdx.x);
}

__global__ __launch_bounds__(256) void pack_x8_kernel(DevParams p, const uint16_t *__restrict__ x,
                                                       uint16_t *__restrict__ xp, int ptiles) {
    __shared__ uint16_t tile[16 * kPackRS];
    pack_x8_block(p, x, xp, ptiles, blockIdx.x, tile);
}

// Launch shape of the channel-chunked copy: 256 positions of one (b, g,
// chunk) per block; x8: planes of whole 16-byte rows (the LDS variant).
struct PackGrid {
    bool x8;
    int ptiles;
    int64_t blocks;
};

static hipError_t pack_grid(const DevParams &p, const void *x, PackGrid *g) {
    g->x8 = p.x_plane % 8 == 0 && (uintptr_t)x % 16 == 0;
    const int64_t ptiles = ((int64_t)p.x_plane + 255) / 256;
    g->blocks = (int64_t)p.B * p.G * (p.cig_pad / 16) * ptiles;
    if (ptiles > 0x7fffffff || g->blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    g->ptiles = (int)ptiles;
    return hipSuccess;
}

hipError_t launch_pack_x(const Plan &pl, const void *x, void *xp, hipStream_t stream) {
    if (pl.xp_bytes == 0) return hipSuccess;
    return launch_pack_dp(pl.dp, x, xp, stream);
}

hipError_t launch_pack_dp(const DevParams &p, const void *x, void *xp, hipStream_t stream) {
    PackGrid g;
    const hipError_t e = pack_grid(p, x, &g);
    if (e != hipSuccess) return e;
    if (g.blocks <= 0) return hipSuccess;
    if (g.x8)
        hipLaunchKernelGGL(pack_x8_kernel, dim3((unsigned)g.blocks), dim3(256), 0, stream, p,
                           (const uint16_t *)x, (uint16_t *)xp, g.ptiles);
    else
        hipLaunchKernelGGL(pack_x_kernel, dim3((unsigned)g.blocks), dim3(256), 0, stream, p,
                           (const uint16_t *)x, (uint16_t *)xp, g.ptiles);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fill: y = bias (or 0). Serves problems whose sums are empty (no input
// channel or an empty input axis): every output is the bias alone.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void fill_kernel(DevParams p, const T *__restrict__ bias,
                                                    T *__restrict__ y, int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int oc = (int)((i / p.y_plane) % p.Co);
        float v = p.has_bias ? to_f32(bias[oc]) : 0.0f;
        if (p.act != CONVT_ACT_NONE) v = activate<sizeof(T) == 2>(p.act, v);
        y[i] = from_f32<T>(v);
    }
}

static unsigned grid_for(int64_t total) {
    int64_t b = (total + 255) / 256;
    return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

hipError_t launch_fill(const Plan &pl, const void *bias, void *y, hipStream_t stream) {
    return launch_fill_dp(pl.dp, pl.elem_bytes, bias, y, stream);
}

hipError_t launch_fill_dp(const DevParams &p, int elem_bytes, const void *bias, void *y,
                          hipStream_t stream) {
    const int64_t total = (int64_t)p.B * p.Co * p.y_plane;
    if (total <= 0) return hipSuccess;
    if (elem_bytes == 2 && p.f16)
        hipLaunchKernelGGL(fill_kernel<_Float16>, dim3(grid_for(total)), dim3(256), 0, stream, p,
                           (const _Float16 *)bias, (_Float16 *)y, total);
    else if (elem_bytes == 2)
        hipLaunchKernelGGL(fill_kernel<uint16_t>, dim3(grid_for(total)), dim3(256), 0, stream, p,
                           (const uint16_t *)bias, (uint16_t *)y, total);
    else
        hipLaunchKernelGGL(fill_kernel<float>, dim3(grid_for(total)), dim3(256), 0, stream, p,
                           (const float *)bias, (float *)y, total);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Naive gather: one thread per output. For output o and tap kk the input
// position is i = (o + p - kk*d) / s when that division is exact and
// 0 <= i < I. Products accumulate in float32, then the bias, then one
// rounding. Serves any stride; used where no other route applies.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void naive_kernel(DevParams p, const T *__restrict__ x,
                                                     const T *__restrict__ w,
                                                     const T *__restrict__ bias, T *__restrict__ y,
                                                     int64_t total) {
    const DevAxis &a0 = p.ax[0], &a1 = p.ax[1], &a2 = p.ax[2];
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t plane = idx / p.y_plane;
        const int o = (int)(idx % p.y_plane);
        const int oc = (int)(plane % p.Co);
        const int64_t b = plane / p.Co;
        const int o2 = o % a2.O, o1 = (o / a2.O) % a1.O, o0 = o / (a2.O * a1.O);
        const int g = oc / p.Cog, ocl = oc % p.Cog;
        float acc = 0.0f;
        for (int ci = 0; ci < p.Cig; ++ci) {
            const T *xp = x + ((int64_t)b * p.Ci + g * p.Cig + ci) * p.x_plane;
            const int cig = g * p.Cig + ci;
            for (int k0 = 0; k0 < a0.K; ++k0) {
                const int t0 = o0 + a0.P - k0 * a0.D;
                if (t0 % a0.S) continue;
                const int i0 = t0 / a0.S;
                if (i0 < 0 || i0 >= a0.I) continue;
                for (int k1 = 0; k1 < a1.K; ++k1) {
                    const int t1 = o1 + a1.P - k1 * a1.D;
                    if (t1 % a1.S) continue;
                    const int i1 = t1 / a1.S;
                    if (i1 < 0 || i1 >= a1.I) continue;
                    for (int k2 = 0; k2 < a2.K; ++k2) {
                        const int t2 = o2 + a2.P - k2 * a2.D;
                        if (t2 % a2.S) continue;
                        const int i2 = t2 / a2.S;
                        if (i2 < 0 || i2 >= a2.I) continue;
                        acc += to_f32(xp[((int64_t)i0 * a1.I + i1) * a2.I + i2]) *
                               to_f32(w[w_offset(p, cig, ocl, (k0 * a1.K + k1) * a2.K + k2)]);
                    }
                }
            }
        }
        if (p.has_bias) acc += to_f32(bias[oc]);
        if (p.act != CONVT_ACT_NONE) acc = activate<sizeof(T) == 2>(p.act, acc);
        y[idx] = from_f32<T>(acc);
    }
}

hipError_t launch_naive(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                        hipStream_t stream) {
    const DevParams &p = pl.dp;
    const int64_t total = (int64_t)p.B * p.Co * p.y_plane;
    if (total <= 0) return hipSuccess;
    if (pl.elem_bytes == 2 && p.f16)
        hipLaunchKernelGGL(naive_kernel<_Float16>, dim3(grid_for(total)), dim3(256), 0, stream, p,
                           (const _Float16 *)x, (const _Float16 *)w, (const _Float16 *)bias,
                           (_Float16 *)y, total);
    else if (pl.elem_bytes == 2)
        hipLaunchKernelGGL(naive_kernel<uint16_t>, dim3(grid_for(total)), dim3(256), 0, stream, p,
                           (const uint16_t *)x, (const uint16_t *)w, (const uint16_t *)bias,
                           (uint16_t *)y, total);
    else
        hipLaunchKernelGGL(naive_kernel<float>, dim3(grid_for(total)), dim3(256), 0, stream, p,
                           (const float *)x, (const float *)w, (const float *)bias, (float *)y,
                           total);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Direct small-channel kernel. A block owns 256 consecutive output positions
// of one (batch, group). The group's weight slab W[g*Cig .. +Cig][Cog][k...]
// is staged once in LDS (as float32). Each lane owns one output position and
// kCo output channels at a time; every input sample it gathers (through the
// phase table of its output residue, so only contributing taps are visited)
// feeds all of them. Lanes own whole outputs, so no cross-lane reduction and
// no atomics are needed. When the group's input planes fit (XS), they are
// staged in LDS after the slab as well: a lane's gathers are then LDS reads
// after one block-wide coalesced load, rather than a chain of dependent
// global loads (the taps' bounds checks keep the compiler from batching them).
// ---------------------------------------------------------------------------
constexpr int kDirPos = 256;

// c + a.lo * b.lo + a.hi * b.hi for two 16-bit values per word (bfloat16 or
// half by T), products and sum in float32 (the two-element dot instructions)
template <typename T>
__device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float c) {
    if constexpr (std::is_same<T, _Float16>::value) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
    } else {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
    }
}

template <typename T, bool ACT, bool XS>
__global__ __launch_bounds__(256) void direct_kernel(DevParams p, const T *__restrict__ x,
                                                      const T *__restrict__ w,
                                                      const T *__restrict__ bias,
                                                      T *__restrict__ y) {
    extern __shared__ float slab[];
    constexpr int kCo = tiles::kDirCoChunk;
    const int ntile = (p.y_plane + kDirPos - 1) / kDirPos;
    int bid = blockIdx.x;
    const int tile = bid % ntile;
    bid /= ntile;
    const int g = bid % p.G;
    const int b = bid / p.G;
    const int slab_n = p.Cig * p.Cog * p.ktot;
    const T *wg = w + (int64_t)g * slab_n;
    if (w_plain(p)) {
        for (int e = threadIdx.x; e < slab_n; e += 256) slab[e] = to_f32(wg[e]);
    } else {
        // slab element e = (ci * Cog + co) * ktot + kk
        for (int e = threadIdx.x; e < slab_n; e += 256) {
            const int kk = e % p.ktot, co = (e / p.ktot) % p.Cog, ci = e / (p.ktot * p.Cog);
            slab[e] = to_f32(w[w_offset(p, g * p.Cig + ci, co, kk)]);
        }
    }
    const T *xb = x + ((int64_t)b * p.Ci + (int64_t)g * p.Cig) * p.x_plane;
    float *xl = slab + slab_n;  // XS: the group's input planes [Cig][x_plane]
    if constexpr (XS) {
        const int xn = p.Cig * p.x_plane;
        for (int e = threadIdx.x; e < xn; e += 256) xl[e] = to_f32(xb[e]);
    }
    __syncthreads();
    const int o = tile * kDirPos + threadIdx.x;
    if (o >= p.y_plane) return;
    const DevAxis &a0 = p.ax[0], &a1 = p.ax[1], &a2 = p.ax[2];
    const int o2 = o % a2.O, o1 = (o / a2.O) % a1.O, o0 = o / (a2.O * a1.O);
    const int r0 = o0 % a0.S, r1 = o1 % a1.S, r2 = o2 % a2.S;
    const int q0 = o0 / a0.S, q1 = o1 / a1.S, q2 = o2 / a2.S;
    const int n0 = a0.n[r0], n1 = a1.n[r1], n2 = a2.n[r2];
    const int b0 = q0 + a0.off0[r0], b1 = q1 + a1.off0[r1], b2 = q2 + a2.off0[r2];
    const int kb0 = a0.kk0[r0], kb1 = a1.kk0[r1], kb2 = a2.kk0[r2];
    T *yb = y + ((int64_t)b * p.Co + (int64_t)g * p.Cog) * p.y_plane + o;
    for (int co0 = 0; co0 < p.Cog; co0 += kCo) {
        float acc[kCo];
#pragma unroll
        for (int c = 0; c < kCo; ++c) acc[c] = 0.0f;
        for (int ci = 0; ci < p.Cig; ++ci) {
            const T *xp = xb + (int64_t)ci * p.x_plane;
            const float *xlp = xl + ci * p.x_plane;
            const float *wc = slab + (ci * p.Cog + co0) * p.ktot;
            for (int j0 = 0; j0 < n0; ++j0) {
                const int i0 = b0 + j0 * a0.ostep;
                if (i0 < 0 || i0 >= a0.I) continue;
                const int k0 = kb0 - j0 * a0.kstep;
                for (int j1 = 0; j1 < n1; ++j1) {
                    const int i1 = b1 + j1 * a1.ostep;
                    if (i1 < 0 || i1 >= a1.I) continue;
                    const int k1 = kb1 - j1 * a1.kstep;
                    for (int j2 = 0; j2 < n2; ++j2) {
                        const int i2 = b2 + j2 * a2.ostep;
                        if (i2 < 0 || i2 >= a2.I) continue;
                        const int k2 = kb2 - j2 * a2.kstep;
                        float xv;
                        if constexpr (XS)
                            xv = xlp[(i0 * a1.I + i1) * a2.I + i2];
                        else
                            xv = to_f32(xp[((int64_t)i0 * a1.I + i1) * a2.I + i2]);
                        const float *wt = wc + (k0 * a1.K + k1) * a2.K + k2;
#pragma unroll
                        for (int c = 0; c < kCo; ++c)
                            if (co0 + c < p.Cog) acc[c] += xv * wt[c * p.ktot];
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < kCo; ++c) {
            const int co = co0 + c;
            if (co < p.Cog) {
                float v = acc[c];
                if (p.has_bias) v += to_f32(bias[g * p.Cog + co]);
                if constexpr (ACT) v = activate<sizeof(T) == 2>(p.act, v);
                yb[(int64_t)co * p.y_plane] = from_f32<T>(v);
            }
        }
    }
}

// instances with an activation are separate (none of its code otherwise)
template <typename T, bool XS>
static void launch_direct_x(const DevParams &p, int64_t blocks, size_t lds, const void *x,
                            const void *w, const void *bias, void *y, hipStream_t stream) {
    if (p.act != CONVT_ACT_NONE)
        hipLaunchKernelGGL((direct_kernel<T, true, XS>), dim3((unsigned)blocks), dim3(256), lds, stream,
                           p, (const T *)x, (const T *)w, (const T *)bias, (T *)y);
    else
        hipLaunchKernelGGL((direct_kernel<T, false, XS>), dim3((unsigned)blocks), dim3(256), lds,
                           stream, p, (const T *)x, (const T *)w, (const T *)bias, (T *)y);
}

template <typename T>
static void launch_direct_t(const DevParams &p, int64_t blocks, size_t lds, bool xs, const void *x,
                            const void *w, const void *bias, void *y, hipStream_t stream) {
    if (xs)
        launch_direct_x<T, true>(p, blocks, lds, x, w, bias, y, stream);
    else
        launch_direct_x<T, false>(p, blocks, lds, x, w, bias, y, stream);
}

hipError_t launch_direct(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                         hipStream_t stream) {
    const DevParams &p = pl.dp;
    const int64_t ntile = (p.y_plane + kDirPos - 1) / kDirPos;
    const int64_t blocks = ntile * p.G * p.B;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    size_t lds = (size_t)p.Cig * p.Cog * p.ktot * sizeof(float);
    // the group's input planes in LDS too, when they fit beside the slab
    const int64_t x_bytes = (int64_t)p.Cig * p.x_plane * (int64_t)sizeof(float);
    const bool xs = x_bytes <= tiles::kDirXStageBytes;
    if (xs) lds += (size_t)x_bytes;
    if (pl.elem_bytes == 2 && p.f16)
        launch_direct_t<_Float16>(p, blocks, lds, xs, x, w, bias, y, stream);
    else if (pl.elem_bytes == 2)
        launch_direct_t<uint16_t>(p, blocks, lds, xs, x, w, bias, y, stream);
    else
        launch_direct_t<float>(p, blocks, lds, xs, x, w, bias, y, stream);
    return hipGetLastError();
}

}  // namespace convt

namespace convt {

// ---------------------------------------------------------------------------
// Backward data, naive gather: one thread per dx element. dx[b, ci, i]
// collects dy[b, oc, o] * W[ci, oc - g*Cog, kk] over the taps kk whose output
// o = i*s - p + kk*d lies inside y and the Cog output channels of ci's group;
// float32 accumulation, one rounding. Serves any problem.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void naive_bwd_kernel(DevParams p, const T *__restrict__ dy,
                                                         const T *__restrict__ w,
                                                         T *__restrict__ dx, int64_t total) {
    const DevAxis &a0 = p.ax[0], &a1 = p.ax[1], &a2 = p.ax[2];
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t plane = idx / p.x_plane;
        const int i = (int)(idx % p.x_plane);
        const int ci = (int)(plane % p.Ci);
        const int64_t b = plane / p.Ci;
        const int i2 = i % a2.I, i1 = (i / a2.I) % a1.I, i0 = i / (a2.I * a1.I);
        const int g = ci / p.Cig;
        const T *yb = dy + ((int64_t)b * p.Co + (int64_t)g * p.Cog) * p.y_plane;
        float acc = 0.0f;
        for (int k0 = 0; k0 < a0.K; ++k0) {
            const int o0 = i0 * a0.S - a0.P + k0 * a0.D;
            if (o0 < 0 || o0 >= a0.O) continue;
            for (int k1 = 0; k1 < a1.K; ++k1) {
                const int o1 = i1 * a1.S - a1.P + k1 * a1.D;
                if (o1 < 0 || o1 >= a1.O) continue;
                for (int k2 = 0; k2 < a2.K; ++k2) {
                    const int o2 = i2 * a2.S - a2.P + k2 * a2.D;
                    if (o2 < 0 || o2 >= a2.O) continue;
                    const int64_t opos = ((int64_t)o0 * a1.O + o1) * a2.O + o2;
                    const int kk = (k0 * a1.K + k1) * a2.K + k2;
                    for (int ocl = 0; ocl < p.Cog; ++ocl)
                        acc += to_f32(yb[(int64_t)ocl * p.y_plane + opos]) *
                               to_f32(w[w_offset(p, ci, ocl, kk)]);
                }
            }
        }
        dx[idx] = from_f32<T>(acc);
    }
}

hipError_t launch_naive_bwd(const Plan &pl, const void *dy, const void *w, void *dx,
                            hipStream_t stream) {
    const DevParams &p = pl.dp;  // the forward problem's axes and channels
    const int64_t total = (int64_t)p.B * p.Ci * p.x_plane;
    if (total <= 0) return hipSuccess;
    if (pl.elem_bytes == 2 && p.f16)
        hipLaunchKernelGGL(naive_bwd_kernel<_Float16>, dim3(grid_for(total)), dim3(256), 0, stream,
                           p, (const _Float16 *)dy, (const _Float16 *)w, (_Float16 *)dx, total);
    else if (pl.elem_bytes == 2)
        hipLaunchKernelGGL(naive_bwd_kernel<uint16_t>, dim3(grid_for(total)), dim3(256), 0, stream,
                           p, (const uint16_t *)dy, (const uint16_t *)w, (uint16_t *)dx, total);
    else
        hipLaunchKernelGGL(naive_bwd_kernel<float>, dim3(grid_for(total)), dim3(256), 0, stream, p,
                           (const float *)dy, (const float *)w, (float *)dx, total);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward data for few channels (the direct kernel turned around):
//     dx[b][g*Cig + ci][i] = sum over ocl < Cog and taps kk of
//                            dy[b][g*Cog + ocl][i*s - p + kk*d] * W[g*Cig + ci][ocl][kk]
// (p: the forward problem). Where Cig or Cog is small, the backward GEMM's
// tiles (64 dx channels x 16-channel chunks of dy) are mostly padding. A
// block owns 256 consecutive dx positions of one (batch, group); the group's
// weights sit in LDS as float32 [kk][ocl, padded to 8][ci, padded to CI], so
// that one 16-byte read gives four input channels (the same address for
// every lane: a broadcast), and a table holds each tap's dy offset and
// per-axis shifts. Each lane owns one dx position and CI input channels at a
// time; per tap it checks the window once, then takes the output channels 8
// at a time with buffer loads whose offsets are out of range (reading 0)
// where the tap falls outside dy or the channel is padding, so the loads
// carry no branches and issue together.
// ---------------------------------------------------------------------------
template <typename T, int CI, int PX>
__global__ __launch_bounds__(256) void direct_bwd_kernel(DevParams p, const T *__restrict__ dy,
                                                          const T *__restrict__ w,
                                                          T *__restrict__ dx) {
    extern __shared__ __attribute__((aligned(16))) float dslab[];
    const DevAxis &a0 = p.ax[0], &a1 = p.ax[1], &a2 = p.ax[2];
    constexpr int BP = kDirPos * PX;  // dx positions per block
    const int ntile = (p.x_plane + BP - 1) / BP;
    int bid = blockIdx.x;
    const int tile = bid % ntile;
    bid /= ntile;
    const int g = bid % p.G;
    const int b = bid / p.G;
    const int ktot = p.ktot, Cog = p.Cog, Cig = p.Cig;
    const int cog8 = (Cog + 7) / 8 * 8, cip = (Cig + CI - 1) / CI * CI;
    // Two-byte types (HP): 32-bit words holding the weights of one input
    // channel for two neighbouring output channels (raw 16-bit values), so
    // that a two-element dot instruction takes a pair of dy channels at once:
    // half the LDS reads and half the VALU work of float32 products.
    constexpr bool HP = sizeof(T) == 2;
    const int slab_n = HP ? ktot * (cog8 / 2) * cip : ktot * cog8 * cip;  // 32-bit words
    if constexpr (HP) {
        uint32_t *ws32 = (uint32_t *)dslab;
        for (int e = threadIdx.x; e < slab_n; e += 256) {
            const int cil = e % cip, r = e / cip, pr = r % (cog8 / 2), kk = r / (cog8 / 2);
            uint32_t lo = 0, hi = 0;
            if (cil < Cig) {
                if (2 * pr < Cog) lo = __builtin_bit_cast(uint16_t, w[w_offset(p, g * Cig + cil, 2 * pr, kk)]);
                if (2 * pr + 1 < Cog)
                    hi = __builtin_bit_cast(uint16_t, w[w_offset(p, g * Cig + cil, 2 * pr + 1, kk)]);
            }
            ws32[e] = lo | hi << 16;
        }
    } else {
        for (int e = threadIdx.x; e < slab_n; e += 256) {
            const int cil = e % cip, r = e / cip, ocl = r % cog8, kk = r / cog8;
            dslab[e] = (ocl < Cog && cil < Cig) ? to_f32(w[w_offset(p, g * Cig + cil, ocl, kk)]) : 0.0f;
        }
    }
    // per tap: dy offset from the tap-0 position, then the per-axis shifts
    int4 *tk = (int4 *)(dslab + slab_n);
    for (int kk = threadIdx.x; kk < ktot; kk += 256) {
        const int k2 = kk % a2.K, k1 = (kk / a2.K) % a1.K, k0 = kk / (a2.K * a1.K);
        tk[kk] = make_int4(((k0 * a0.D) * a1.O + k1 * a1.D) * a2.O + k2 * a2.D, k0 * a0.D, k1 * a1.D,
                           k2 * a2.D);
    }
    __syncthreads();
    // this lane's PX dx positions, 256 apart; dy coordinates of tap 0 (a
    // position past the plane gets coordinates no tap can bring inside)
    const int i_lane = tile * BP + threadIdx.x;
    if (i_lane >= p.x_plane) return;
    int e0[PX], e1[PX], e2[PX], base[PX];
#pragma unroll
    for (int q = 0; q < PX; ++q) {
        const int i = i_lane + q * kDirPos;
        const int i2 = i % a2.I, i1 = (i / a2.I) % a1.I, i0 = i / (a2.I * a1.I);
        const bool in = i < p.x_plane;
        e0[q] = in ? i0 * a0.S - a0.P : -(1 << 29);
        e1[q] = i1 * a1.S - a1.P;
        e2[q] = i2 * a2.S - a2.P;
        base[q] = in ? (e0[q] * a1.O + e1[q]) * a2.O + e2[q] : 0;
    }
    constexpr uint32_t ES = sizeof(T);
    const uint32_t ypl_bytes = (uint32_t)p.y_plane * ES;
    const __amdgpu_buffer_rsrc_t ys =
        make_rsrc(dy + ((int64_t)b * p.Co + (int64_t)g * Cog) * p.y_plane, (uint32_t)Cog * ypl_bytes);
    T *dxb = dx + ((int64_t)b * p.Ci + (int64_t)g * Cig) * p.x_plane + i_lane;
    for (int ci0 = 0; ci0 < Cig; ci0 += CI) {
        float acc[PX][CI];
#pragma unroll
        for (int q = 0; q < PX; ++q)
#pragma unroll
            for (int c = 0; c < CI; ++c) acc[q][c] = 0.0f;
        for (int kk = 0; kk < ktot; ++kk) {
            const int4 t = tk[kk];
            bool ok[PX];
            uint32_t off[PX];
#pragma unroll
            for (int q = 0; q < PX; ++q) {
                const int o0 = e0[q] + t.y, o1 = e1[q] + t.z, o2 = e2[q] + t.w;
                ok[q] = o0 >= 0 && o0 < a0.O && o1 >= 0 && o1 < a1.O && o2 >= 0 && o2 < a2.O;
                off[q] = (uint32_t)(base[q] + t.x) * ES;
            }
            const float *wk = dslab + (kk * cog8) * cip + ci0;
            for (int oc0 = 0; oc0 < Cog; oc0 += 8) {
                if constexpr (HP) {
                    // dy channel pairs (oc0 + 2pp, oc0 + 2pp + 1) as raw 16-bit pairs
                    uint32_t yp[PX][4];
#pragma unroll
                    for (int q = 0; q < PX; ++q)
#pragma unroll
                        for (int pp = 0; pp < 4; ++pp) {
                            uint32_t h[2];
#pragma unroll
                            for (int e = 0; e < 2; ++e) {
                                const int u = 2 * pp + e;
                                const uint32_t o = (ok[q] && oc0 + u < Cog)
                                                       ? off[q] + (uint32_t)(oc0 + u) * ypl_bytes
                                                       : kOutOfRange;
                                h[e] = __builtin_amdgcn_raw_buffer_load_b16(ys, o, 0, 0);
                            }
                            yp[q][pp] = h[0] | h[1] << 16;
                        }
                    const uint32_t *wp = (const uint32_t *)dslab + (kk * (cog8 / 2) + oc0 / 2) * cip + ci0;
#pragma unroll
                    for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
                        for (int c4 = 0; c4 < CI; c4 += 4) {
                            const u32x4 wv = *(const u32x4 *)(wp + pp * cip + c4);
#pragma unroll
                            for (int q = 0; q < PX; ++q)
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    acc[q][c4 + e] = dot2_acc<T>(yp[q][pp], wv[e], acc[q][c4 + e]);
                        }
                    }
                    continue;
                }
                float yv[PX][8];
#pragma unroll
                for (int q = 0; q < PX; ++q)
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const uint32_t o =
                            (ok[q] && oc0 + u < Cog) ? off[q] + (uint32_t)(oc0 + u) * ypl_bytes : kOutOfRange;
                        yv[q][u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ys, o, 0, 0));
                    }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float *wr = wk + (oc0 + u) * cip;
#pragma unroll
                    for (int c4 = 0; c4 < CI; c4 += 4) {
                        const float4 wv = *(const float4 *)(wr + c4);
#pragma unroll
                        for (int q = 0; q < PX; ++q) {
                            acc[q][c4] += yv[q][u] * wv.x;
                            acc[q][c4 + 1] += yv[q][u] * wv.y;
                            acc[q][c4 + 2] += yv[q][u] * wv.z;
                            acc[q][c4 + 3] += yv[q][u] * wv.w;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int q = 0; q < PX; ++q)
            if (i_lane + q * kDirPos < p.x_plane)
#pragma unroll
                for (int c = 0; c < CI; ++c)
                    if (ci0 + c < Cig)
                        dxb[(int64_t)(ci0 + c) * p.x_plane + q * kDirPos] = from_f32<T>(acc[q][c]);
    }
}

// One dx position per lane: the kernel is bound by the latency of its dy
// loads, which more lanes cover; two or four positions per lane (each LDS
// weight read serving all of them) measured slower on the grouped workload
// (90 against 80 us) and on small planes, where blocks become few.
constexpr int kDirBwdPx = 1;
template <typename T>
static void launch_direct_bwd_t(const DevParams &p, int64_t lds, const void *dy, const void *w,
                                void *dx, hipStream_t stream) {
    const int ci = tiles::dir_bwd_ci(p.Cig);
    const int px = kDirBwdPx;
    const int64_t ntile = (p.x_plane + (int64_t)kDirPos * px - 1) / ((int64_t)kDirPos * px);
    const dim3 grid((unsigned)(ntile * p.G * p.B));
    switch (ci) {
        case 4:
            hipLaunchKernelGGL((direct_bwd_kernel<T, 4, kDirBwdPx>), grid, dim3(256), lds, stream, p,
                               (const T *)dy, (const T *)w, (T *)dx);
            break;
        case 8:
            hipLaunchKernelGGL((direct_bwd_kernel<T, 8, kDirBwdPx>), grid, dim3(256), lds, stream, p,
                               (const T *)dy, (const T *)w, (T *)dx);
            break;
        default:
            hipLaunchKernelGGL((direct_bwd_kernel<T, 16, kDirBwdPx>), grid, dim3(256), lds, stream, p,
                               (const T *)dy, (const T *)w, (T *)dx);
            break;
    }
}

hipError_t launch_direct_bwd(const Plan &pl, const void *dy, const void *w, void *dx,
                             hipStream_t stream) {
    const DevParams &p = pl.dp;  // the forward problem's axes and channels
    const int64_t ntile = (p.x_plane + kDirPos - 1) / kDirPos;  // (at most; fewer with PX > 1)
    const int64_t blocks = ntile * p.G * p.B;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int64_t lds = tiles::dir_bwd_lds_bytes(p.Cig, p.Cog, p.ktot);
    // the group's dy planes must fit one buffer resource
    if (lds > tiles::kDirBwdLdsBytes || (int64_t)p.Cog * p.y_plane * pl.elem_bytes >= ((int64_t)1 << 31))
        return hipErrorInvalidConfiguration;
    if (pl.elem_bytes == 2 && p.f16)
        launch_direct_bwd_t<_Float16>(p, lds, dy, w, dx, stream);
    else if (pl.elem_bytes == 2)
        launch_direct_bwd_t<uint16_t>(p, lds, dy, w, dx, stream);
    else
        launch_direct_bwd_t<float>(p, lds, dy, w, dx, stream);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight reorder for the backward-data GEMM (p: the backward problem, whose
// rows m are the Cig input channels of a group and whose K channels are its
// Cog output channels):
//     W[g*Cig + m][oc][kk] -> Wb[g][tap][chunk][m][32 bytes of oc]
// tap: kk's index in the plan's tap order (phase by phase, each padded with
// zero taps to whole groups of gemm_gs); chunk = oc / BK (16 bfloat16 or 8
// float32 channels); the two 16-byte halves of a row swap where bit 3 of m
// is set (the operand reads' XOR swizzle). Rows past Cig, channels past Cog
// and padding taps are zero.
//
// A block owns 8 rows m, OCB channels oc (whole chunks) and KT taps kk: it
// reads the runs W[m][oc0 .. oc0 + OCB)[kk0 .. kk0 + KT) into LDS with
// consecutive lanes on consecutive elements, then writes, per (tap, chunk),
// the 8 rows' 256 contiguous bytes, consecutive lanes on consecutive 16-byte
// halves. Block P also writes phase P's part of the halo shift table (blocks
// take every gridDim-th phase when the grid is smaller): entry tapbase(P) + t
// holds, for tap t = (j0, j1, j2) of phase P with input offsets off_a =
// off0_a + j_a * ostep_a, the row of its window in the phase's halo box
// (which starts at the phase's largest offset u_a = off0_a + (n_a - 1) *
// ostep_a), ((u0 - off0) * E1 + (u1 - off1)) * E2 + (u2 - off2), E1 and E2
// the box extents (the dx tile plus span_max); padding taps get 0.
// ---------------------------------------------------------------------------
// (block `blk` of `nblk`; lds_raw: 8 * OCB * KT elements + 4 * KT bytes)
template <typename T>
__device__ __forceinline__ void reorder_bwd_block(const DevParams &p, const T *__restrict__ w,
                                                  T *__restrict__ wr, int32_t *__restrict__ tab,
                                                  int OCB, int KT, int vec_runs, int blk, int nblk,
                                                  unsigned char *lds_raw) {
    constexpr int VEC = 16 / sizeof(T), BK = 2 * VEC, MB = 8;
    const int Cm = p.Cog, Coc = p.Cig, ktot = p.ktot;
    const int nchunks = p.cig_pad / BK;
    const int nob = (p.cig_pad + OCB - 1) / OCB;
    const int nmb = p.cog_pad / MB;
    const int nkt = (ktot + KT - 1) / KT;
    int bid = blk;
    const int kb = bid % nkt;
    bid /= nkt;
    const int ob = bid % nob;
    bid /= nob;
    const int mb = bid % nmb;
    const int g = bid / nmb;
    const int m0 = mb * MB, oc0 = ob * OCB, kk0 = kb * KT;
    const int nk = ktot - kk0 < KT ? ktot - kk0 : KT;
    const int noc = p.cig_pad - oc0 < OCB ? p.cig_pad - oc0 : OCB;  // whole chunks
    T *brick = (T *)lds_raw;  // [MB][OCB][KT]
    int *dst_tap = (int *)(lds_raw + (size_t)MB * OCB * KT * sizeof(T));
    const int K1 = p.ax[1].K, K2 = p.ax[2].K;
    auto tap_lookup = [&]() __attribute__((always_inline)) {
        for (int k = threadIdx.x; k < nk; k += 256) {
            const int kk = kk0 + k;
            dst_tap[k] = tap_in_table(p, kk / (K1 * K2), (kk / K2) % K1, kk % K2);
        }
    };
    // With vec_runs (KT == ktot, every chunk of the block inside or wholly
    // outside Cog, 16-byte aligned runs), each row's run [oc0, oc0 + OCB) x
    // [0, ktot) moves as 16-byte vectors, 4 per lane in flight; the tap
    // lookups (chains of dependent parameter reads) run while a lane's first
    // loads are in flight.
    const int n_in = vec_runs ? 0 : MB * noc * nk;
    if (!vec_runs) tap_lookup();
    if (vec_runs) {
        const int nvr = noc * ktot * (int)sizeof(T) / 16;  // vectors of one row's run
        const int nv = MB * nvr;
        auto load = [&](int v0, u32x4 *v) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int vi = v0 + 256 * u;
                const int i = vi / nvr, r = vi - i * nvr;
                v[u] = u32x4{0u, 0u, 0u, 0u};
                if (vi < nv && m0 + i < Cm && oc0 < Coc)
                    v[u] = ((const u32x4 *)(w + (((int64_t)g * Cm + m0 + i) * Coc + oc0) * ktot))[r];
            }
        };
        u32x4 v[4];
        load(threadIdx.x, v);
        tap_lookup();
        for (int v0 = threadIdx.x; v0 < nv; v0 += 256 * 4) {
            if (v0 != (int)threadIdx.x) load(v0, v);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int vi = v0 + 256 * u;
                if (vi < nv) {
                    const int i = vi / nvr, r = vi - i * nvr;
                    ((u32x4 *)(brick + (size_t)i * OCB * KT))[r] = v[u];
                }
            }
        }
    }
    for (int e0 = threadIdx.x; e0 < n_in; e0 += 256 * 8) {
        T v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + 256 * u;
            const int i = e / (noc * nk), r = e - i * (noc * nk);
            const int col = r / nk, k = r - col * nk;
            const int m = m0 + i, oc = oc0 + col;
            const bool ok = e < n_in && m < Cm && oc < Coc;
            // p is the backward problem: the forward's Ci = p.Co, Co = p.Ci,
            // Cig = Cm, Cog = Coc
            v[u] = w[ok ? w_offset(p.w_layout, p.w_flip, p.Co, p.Ci, Cm, Coc, p.ax[0].K, p.ax[1].K,
                                   p.ax[2].K, g * Cm + m, oc, kk0 + k)
                        : 0];
            if (!ok) v[u] = from_f32<T>(0.0f);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + 256 * u;
            if (e < n_in) {
                const int i = e / (noc * nk), r = e - i * (noc * nk);
                brick[(i * OCB + r / nk) * KT + r % nk] = v[u];
            }
        }
    }
    __syncthreads();
    const int64_t chunk_elems = (int64_t)p.cog_pad * BK;
    T *wg = wr + (int64_t)g * p.ktot_pad * nchunks * chunk_elems;
    const int ncc = noc / BK;
    const int n_out = nk * ncc * MB * 2;
    for (int n = threadIdx.x; n < n_out; n += 256) {
        const int half = n & 1, i = (n >> 1) & (MB - 1), rest = n >> 4;
        const int cc = rest % ncc, k = rest / ncc;
        const int m = m0 + i;
        const T *src = brick + (i * OCB + cc * BK + half * VEC) * KT + k;
        u32x4 out;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = (uint32_t)src[(2 * e) * KT] | ((uint32_t)src[(2 * e + 1) * KT] << 16);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = __float_as_uint((float)src[e * KT]);
        }
        const int phys = half ^ ((m >> 3) & 1);
        *(u32x4 *)&wg[((int64_t)dst_tap[k] * nchunks + oc0 / BK + cc) * chunk_elems + (int64_t)m * BK +
                      phys * VEC] = out;
    }
    // padding taps of this (rows, chunks) tile (none when every phase's tap
    // count is a whole number of groups)
    if (kb == 0 && p.ktot_pad != p.ktot) {
        const int gs = p.gemm_gs;
        for (int P = 0; P < p.nphase; ++P) {
            const int nt = p.ph[P].ntaps;
            const int npad = (nt + gs - 1) / gs * gs - nt;
            for (int n = threadIdx.x; n < npad * ncc * MB * 2; n += 256) {
                const int half = n & 1, i = (n >> 1) & (MB - 1), rest = n >> 4;
                const int cc = rest % ncc, t = nt + rest / ncc;
                *(u32x4 *)&wg[((int64_t)(p.ph[P].tapbase + t) * nchunks + oc0 / BK + cc) * chunk_elems +
                              (int64_t)(m0 + i) * BK + half * VEC] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    // the halo shift table: block P writes phase P's entries
    {
        const int gs = p.gemm_gs;
        const DevAxis &a0 = p.ax[0], &a1 = p.ax[1], &a2 = p.ax[2];
        const int E1 = p.th + a1.span_max, E2 = p.tw + a2.span_max;
        for (int P = blk; P < p.nphase; P += nblk) {
            const PhaseDesc ph = phase_desc(p, P);
            const int padded = (ph.ntaps + gs - 1) / gs * gs;
            const int n1 = ph.n[1], n2 = ph.n[2];
            for (int t = threadIdx.x; t < padded; t += 256) {
                int v = 0;
                if (t < ph.ntaps) {
                    const int j2 = t % n2, j1 = (t / n2) % n1, j0 = t / (n1 * n2);
                    const int f0 = ph.off0[0] + j0 * a0.ostep, f1 = ph.off0[1] + j1 * a1.ostep,
                              f2 = ph.off0[2] + j2 * a2.ostep;
                    const int u0 = ph.off0[0] + (ph.n[0] - 1) * a0.ostep,
                              u1 = ph.off0[1] + (n1 - 1) * a1.ostep, u2 = ph.off0[2] + (n2 - 1) * a2.ostep;
                    v = ((u0 - f0) * E1 + (u1 - f1)) * E2 + (u2 - f2);
                }
                tab[ph.tapbase + t] = v;
            }
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void reorder_bwd_kernel(DevParams p, const T *__restrict__ w,
                                                          T *__restrict__ wr,
                                                          int32_t *__restrict__ tab, int OCB,
                                                          int KT, int vec_runs) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    reorder_bwd_block<T>(p, w, wr, tab, OCB, KT, vec_runs, blockIdx.x, gridDim.x, lds_raw);
}

static hipError_t reorder_bwd_grid(const Plan &pl, const void *w, ReorderGrid *r) {
    const DevParams &p = pl.bdp;
    const int es = pl.elem_bytes, bk = 32 / es;
    if (p.cig_pad % bk || p.cog_pad % 8) return hipErrorInvalidValue;
    // 8 rows x OCB channels (whole chunks) x KT taps per block, the brick
    // within 32 KiB, OCB halved while the grid has fewer than 1024 blocks
    int KT = p.ktot < 128 ? p.ktot : 128;
    int OCB = 32768 / (8 * KT * es) / bk * bk;
    if (OCB < bk) OCB = bk;
    if (OCB > p.cig_pad) OCB = p.cig_pad;
    const int64_t nkt = (p.ktot + KT - 1) / KT;
    const int64_t base = (int64_t)p.G * (p.cog_pad / 8) * nkt;
    while (OCB > bk && base * ((p.cig_pad + OCB - 1) / OCB) < 1024) OCB = (OCB / 2 + bk - 1) / bk * bk;
    r->a = OCB;
    r->KT = KT;
    r->blocks = base * ((p.cig_pad + OCB - 1) / OCB);
    r->vec_runs = p.w_layout == CONVT_FILTER_CI_CO_K && !p.w_flip && KT == p.ktot &&
                  p.Cig % OCB == 0 && p.cig_pad % OCB == 0 &&
                  ((int64_t)p.Cig * p.ktot * es) % 16 == 0 &&
                  ((int64_t)OCB * p.ktot * es) % 16 == 0 && (uintptr_t)w % 16 == 0;
    r->lds = (size_t)8 * OCB * KT * es + (size_t)4 * KT;
    if (r->blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    return hipSuccess;
}

hipError_t launch_reorder_bwd(const Plan &pl, const void *w, void *wr, hipStream_t stream) {
    const DevParams &p = pl.bdp;
    ReorderGrid r;
    const hipError_t e = reorder_bwd_grid(pl, w, &r);
    if (e != hipSuccess) return e;
    if (r.blocks <= 0) return hipSuccess;
    int32_t *tab = (int32_t *)((char *)wr + pl.bwd_tab_offset);
    if (pl.elem_bytes == 2)
        hipLaunchKernelGGL(reorder_bwd_kernel<uint16_t>, dim3((unsigned)r.blocks), dim3(256), r.lds,
                           stream, p, (const uint16_t *)w, (uint16_t *)wr, tab, r.a, r.KT, r.vec_runs);
    else
        hipLaunchKernelGGL(reorder_bwd_kernel<float>, dim3((unsigned)r.blocks), dim3(256), r.lds,
                           stream, p, (const float *)w, (float *)wr, tab, r.a, r.KT, r.vec_runs);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The two preparations of the two-byte phase GEMM in one launch: the weight
// reorder (forward or backward layout) and the channel-chunked copy of the
// input are independent, so blocks [0, nrb) reorder and the rest copy, and
// the reorder's latency (its blocks move little data) hides behind the
// copy's traffic instead of adding a launch of its own.
// ---------------------------------------------------------------------------
template <bool BWD, bool X8>
__global__ __launch_bounds__(256) void prep_kernel(DevParams p, const uint16_t *__restrict__ w,
                                                   uint16_t *__restrict__ wr, int32_t *__restrict__ tab,
                                                   int a, int KT, int vec_runs, int nrb,
                                                   const uint16_t *__restrict__ x,
                                                   uint16_t *__restrict__ xp, int ptiles) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    const int blk = blockIdx.x;
    if (blk < nrb) {
        if constexpr (BWD)
            reorder_bwd_block<uint16_t>(p, w, wr, tab, a, KT, vec_runs, blk, nrb, lds_raw);
        else
            reorder_chunked_block<uint16_t>(p, w, wr, tab, a, KT, vec_runs, blk, nrb, lds_raw);
    } else if constexpr (X8) {
        pack_x8_block(p, x, xp, ptiles, blk - nrb, (uint16_t *)lds_raw);
    } else {
        pack_x_block(p, x, xp, ptiles, blk - nrb);
    }
}

template <bool BWD>
static hipError_t launch_prep_t(const Plan &pl, const DevParams &p, const ReorderGrid &r,
                                const void *w, void *wr, int32_t *tab, const void *x, void *xp,
                                hipStream_t stream) {
    PackGrid g;
    const hipError_t e = pack_grid(p, x, &g);
    if (e != hipSuccess) return e;
    const int64_t rb = r.blocks > 0 ? r.blocks : 0, pb = g.blocks > 0 ? g.blocks : 0;
    if (rb + pb <= 0) return hipSuccess;
    if (rb + pb > 0x7fffffff) return hipErrorInvalidConfiguration;
    size_t lds = rb > 0 ? r.lds : 0;
    if (pb > 0 && g.x8 && lds < (size_t)kPackLdsBytes) lds = kPackLdsBytes;
    if (g.x8)
        hipLaunchKernelGGL((prep_kernel<BWD, true>), dim3((unsigned)(rb + pb)), dim3(256), lds, stream, p,
                           (const uint16_t *)w, (uint16_t *)wr, tab, r.a, r.KT, r.vec_runs, (int)rb,
                           (const uint16_t *)x, (uint16_t *)xp, g.ptiles);
    else
        hipLaunchKernelGGL((prep_kernel<BWD, false>), dim3((unsigned)(rb + pb)), dim3(256), lds, stream, p,
                           (const uint16_t *)w, (uint16_t *)wr, tab, r.a, r.KT, r.vec_runs, (int)rb,
                           (const uint16_t *)x, (uint16_t *)xp, g.ptiles);
    return hipGetLastError();
}

hipError_t launch_prep(const Plan &pl, const void *w, void *wr, const void *x, void *xp,
                       hipStream_t stream) {
    if (pl.elem_bytes != 2 || !pl.dp.wr_chunked || pl.xp_bytes == 0) return hipErrorInvalidValue;
    ReorderGrid r;
    const hipError_t e = reorder_chunked_grid(pl, w, &r);
    if (e != hipSuccess) return e;
    return launch_prep_t<false>(pl, pl.dp, r, w, wr, (int32_t *)((char *)wr + pl.tab_offset), x, xp,
                                stream);
}

hipError_t launch_prep_bwd(const Plan &pl, const void *w, void *wr, const void *dy, void *xp,
                           hipStream_t stream) {
    if (pl.elem_bytes != 2 || pl.bwd_xp_bytes == 0) return hipErrorInvalidValue;
    ReorderGrid r;
    const hipError_t e = reorder_bwd_grid(pl, w, &r);
    if (e != hipSuccess) return e;
    return launch_prep_t<true>(pl, pl.bdp, r, w, wr, (int32_t *)((char *)wr + pl.bwd_tab_offset), dy,
                               xp, stream);
}

}  // namespace convt
