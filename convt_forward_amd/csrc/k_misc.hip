// Weight reorder, bias fill, the one-thread-per-output gather kernel and the
// small-channel direct kernel.
#include "kcommon.h"
#include "launch.h"

namespace convt {

// ---------------------------------------------------------------------------
// Weight reorder + tap flip.
//
// W[g*Cig + ci][co][k0][k1][k2] (forward orientation, the layout the SKaiNET
// convTranspose2d page states) -> Wr[g][tap][co][ci] (grouped route) or
// Wr[g][tap][chunk][co][32 bytes of ci] (phase GEMM, the two 16-byte halves of
// a row swapped where bit 3 of co is set), where `tap` enumerates
// the taps phase by phase (phases in lexicographic residue order) and, within
// a phase, in ascending input offset (descending kk per axis: the
// tap-reversed order). ci is contiguous so that MFMA operands are 16-byte
// reads; co and ci are zero-padded to cog_pad and cig_pad so that the GEMM
// loads need no masks.
//
// A block owns one 16-byte vector of input channels (VEC = 8 bfloat16 or 4
// float32 channels) and a block of `ocb` output channels, over all taps. For
// each of its channels the [ocb][ktot] slab is contiguous in W, so the block
// reads it with consecutive lanes on consecutive elements into LDS; each lane
// then assembles whole destination vectors (VEC channels of one (tap, co))
// and writes them with one 16-byte store.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void reorder_kernel(DevParams p, const T *__restrict__ w,
                                                       T *__restrict__ wr, int ocb) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    T *brick = (T *)lds_raw;
    constexpr int VEC = 16 / sizeof(T);
    const int ktot = p.ktot;
    const int nci = p.cig_pad / VEC;
    const int nco = (p.cog_pad + ocb - 1) / ocb;
    int bid = blockIdx.x;
    const int co_b = bid % nco;
    bid /= nco;
    const int ci_b = bid % nci;
    const int g = bid / nci;
    const int n = ocb * ktot;
    const int co0 = co_b * ocb;
    // loads are unconditional (a masked element reads the slab's first
    // element and is then zeroed) and issued in batches of 8 before their
    // LDS stores, so that a batch is in flight together
    const T *wg = w + (int64_t)g * p.Cig * p.Cog * ktot;
    const int lim = (p.Cog - co0) * ktot;  // elements of a channel row inside W
    const int total = VEC * n;
    for (int e0 = threadIdx.x; e0 < total; e0 += 256 * 8) {
        T v[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + 256 * u;
            const int cil = e / n, r = e - cil * n;
            const int ci = ci_b * VEC + cil;
            ok[u] = e < total && ci < p.Cig && r < lim;
            v[u] = wg[ok[u] ? ((int64_t)ci * p.Cog + co0) * ktot + r : 0];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + 256 * u;
            if (e < total) brick[e] = ok[u] ? v[u] : from_f32<T>(0.0f);
        }
    }
    __syncthreads();
    const int K1 = p.ax[1].K, K2 = p.ax[2].K;
    const int nchunks = p.cig_pad / (2 * VEC);
    // destination of the vector (tap t, channel co) of this block's input channels
    auto dst_of = [&](int t, int co) -> int64_t {
        if (p.wr_chunked) {
            // [g][tap][chunk][co][2 vectors]; the two vectors of a row swap
            // places where bit 3 of co is set
            const int half = (ci_b & 1) ^ ((co >> 3) & 1);
            return ((((int64_t)g * p.ktot_pad + t) * nchunks + (ci_b >> 1)) * p.cog_pad + co) *
                       (2 * VEC) +
                   half * VEC;
        }
        return (((int64_t)g * ktot + t) * p.cog_pad + co) * p.cig_pad + ci_b * VEC;
    };
    for (int v = threadIdx.x; v < n; v += 256) {
        const int col = v / ktot, kk = v - col * ktot;
        const int co = co0 + col;
        if (co >= p.cog_pad) continue;
        const int k2 = kk % K2, k1 = (kk / K2) % K1, k0 = kk / (K1 * K2);
        const int tg = p.wr_chunked ? tap_in_table(p, k0, k1, k2) : tap_global(p, k0, k1, k2);
        u32x4 out;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = (uint32_t)brick[(2 * e) * n + v] | ((uint32_t)brick[(2 * e + 1) * n + v] << 16);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = __float_as_uint((float)brick[e * n + v]);
        }
        *(u32x4 *)&wr[dst_of(tg, co)] = out;
    }
    if (p.wr_chunked) {
        // the zero taps that pad each phase to whole tap groups
        const int gs = p.gemm_gs;
        for (int P = 0; P < p.nphase; ++P) {
            const int nt = p.ph[P].ntaps;
            const int npad = (nt + gs - 1) / gs * gs - nt;
            for (int v = threadIdx.x; v < npad * ocb; v += 256) {
                const int co = co0 + v % ocb;
                if (co < p.cog_pad)
                    *(u32x4 *)&wr[dst_of(p.ph[P].tapbase + nt + v / ocb, co)] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
}

// Output channels per reorder block: the LDS brick (16 bytes per output
// channel and tap) stays within 32 KiB.
static int reorder_ocb(const DevParams &p) {
    int ocb = 32768 / (16 * p.ktot);
    if (ocb < 1) ocb = 1;
    if (ocb > p.cog_pad) ocb = p.cog_pad;
    return ocb;
}

hipError_t launch_reorder(const Plan &pl, const void *w, void *wr, hipStream_t stream) {
    const DevParams &p = pl.dp;
    const int vec = 16 / pl.elem_bytes;
    if (p.cig_pad % (p.wr_chunked ? 2 * vec : vec)) return hipErrorInvalidValue;
    const int ocb = reorder_ocb(p);
    const int64_t nco = (p.cog_pad + ocb - 1) / ocb;
    const int64_t blocks = (int64_t)p.G * (p.cig_pad / vec) * nco;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)16 * ocb * p.ktot;
    if (lds > 65536) return hipErrorInvalidConfiguration;
    if (pl.elem_bytes == 2)
        hipLaunchKernelGGL(reorder_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), lds, stream,
                           p, (const uint16_t *)w, (uint16_t *)wr, ocb);
    else
        hipLaunchKernelGGL(reorder_kernel<float>, dim3((unsigned)blocks), dim3(256), lds, stream, p,
                           (const float *)w, (float *)wr, ocb);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Input re-layout for the bfloat16 phase GEMM:
//     x[b][g*Cig + ci][pos] -> xp[b][g][chunk][pos][16 channels]
// (32 bytes per position and chunk, channels past Cig zero), so that the GEMM
// copies a halo row of one chunk as two 16-byte pieces. One thread per
// (b, g, chunk, position): 16 two-byte loads, coalesced over the positions
// of a wave, and two 16-byte stores.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_x_kernel(DevParams p, const uint16_t *__restrict__ x,
                                                      uint16_t *__restrict__ xp, int ptiles) {
    const int nchunks = p.cig_pad / 16;
    const int64_t plane = p.x_plane;
    int bid = blockIdx.x;
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

hipError_t launch_pack_x(const Plan &pl, const void *x, void *xp, hipStream_t stream) {
    const DevParams &p = pl.dp;
    if (pl.xp_bytes == 0) return hipSuccess;
    const int64_t ptiles = ((int64_t)p.x_plane + 255) / 256;
    const int64_t blocks = (int64_t)p.B * p.G * (p.cig_pad / 16) * ptiles;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(pack_x_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p,
                       (const uint16_t *)x, (uint16_t *)xp, (int)ptiles);
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
        y[i] = p.has_bias ? bias[oc] : from_f32<T>(0.0f);
    }
}

static unsigned grid_for(int64_t total) {
    int64_t b = (total + 255) / 256;
    return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

hipError_t launch_fill(const Plan &pl, const void *bias, void *y, hipStream_t stream) {
    const DevParams &p = pl.dp;
    const int64_t total = (int64_t)p.B * p.Co * p.y_plane;
    if (total <= 0) return hipSuccess;
    if (pl.elem_bytes == 2)
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
            const T *wp = w + ((int64_t)(g * p.Cig + ci) * p.Cog + ocl) * p.ktot;
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
                               to_f32(wp[(k0 * a1.K + k1) * a2.K + k2]);
                    }
                }
            }
        }
        if (p.has_bias) acc += to_f32(bias[oc]);
        y[idx] = from_f32<T>(acc);
    }
}

hipError_t launch_naive(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                        hipStream_t stream) {
    const DevParams &p = pl.dp;
    const int64_t total = (int64_t)p.B * p.Co * p.y_plane;
    if (total <= 0) return hipSuccess;
    if (pl.elem_bytes == 2)
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
// no atomics are needed.
// ---------------------------------------------------------------------------
constexpr int kDirPos = 256;

template <typename T>
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
    for (int e = threadIdx.x; e < slab_n; e += 256) slab[e] = to_f32(wg[e]);
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
    const T *xb = x + ((int64_t)b * p.Ci + (int64_t)g * p.Cig) * p.x_plane;
    T *yb = y + ((int64_t)b * p.Co + (int64_t)g * p.Cog) * p.y_plane + o;
    for (int co0 = 0; co0 < p.Cog; co0 += kCo) {
        float acc[kCo];
#pragma unroll
        for (int c = 0; c < kCo; ++c) acc[c] = 0.0f;
        for (int ci = 0; ci < p.Cig; ++ci) {
            const T *xp = xb + (int64_t)ci * p.x_plane;
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
                        const float xv = to_f32(xp[((int64_t)i0 * a1.I + i1) * a2.I + i2]);
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
                yb[(int64_t)co * p.y_plane] = from_f32<T>(v);
            }
        }
    }
}

hipError_t launch_direct(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                         hipStream_t stream) {
    const DevParams &p = pl.dp;
    const int64_t ntile = (p.y_plane + kDirPos - 1) / kDirPos;
    const int64_t blocks = ntile * p.G * p.B;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)p.Cig * p.Cog * p.ktot * sizeof(float);
    if (pl.elem_bytes == 2)
        hipLaunchKernelGGL(direct_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), lds, stream,
                           p, (const uint16_t *)x, (const uint16_t *)w, (const uint16_t *)bias,
                           (uint16_t *)y);
    else
        hipLaunchKernelGGL(direct_kernel<float>, dim3((unsigned)blocks), dim3(256), lds, stream, p,
                           (const float *)x, (const float *)w, (const float *)bias, (float *)y);
    return hipGetLastError();
}

}  // namespace convt
