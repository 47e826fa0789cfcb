// Input gradient of a 2-D grouped transposed convolution with few channels
// per group (bfloat16 or half, MFMA 16x16x32).
//
// The adjoint of the forward scatter-add gathers, per input position i and
// input channel ci of group g,
//   dx[ci][i] = sum over (co < C_out/g, tap k) of W[ci][co][k] * dy[co][s*i - p + d*k]
// (the input adjoint that the SKaiNET convTranspose2d pull request's Summary
// lists beside the forward; its index map is the forward's scatter index read
// backwards). That is a strided correlation of dy,
// a dense contraction over K = (tap, output channel) for each dx position,
// so it runs on MFMA: rows = 16 dx positions along the width, columns = the
// group's input channels (at most 16), K = (tap, 8-channel slice of dy)
// slots, four per MFMA step, up to four steps.
//
// A tile is one (batch, group) and R dx rows over the full dx width; blocks
// are persistent (one per resident slot) and take tiles in turn, each tile's
// loads issued during the previous tile's MFMAs and stores:
//  1. the group's part of W, as W stores it, goes to LDS by LDS-destination
//     buffer loads (no registers, no arithmetic per element); after the first
//     barrier the block gathers the MFMA weight fragments from that layout
//     (its channel strides) into a slab whose rows the 16 lanes of a fragment
//     read without bank conflicts (gathered per wave straight from the stored
//     layout, 16 input channels whose rows lie 2 * C_out/g * taps bytes
//     apart conflicted up to 16-way);
//  2. dy's halo for the R rows (every tap's rows, the full dy width) goes to
//     LDS as 16-byte cells of 8 dy channels, [halo row][slice][column]: a
//     lane loads 8 positions of each of 8 channels (eight 16-byte loads) and
//     transposes the 8 x 8 block in registers; columns outside dy hold
//     zeros. With width stride 2 a (halo row, slice) holds its even columns
//     first, then its odd ones, so that neighbouring dx positions read
//     neighbouring cells (in column order they lie 2 cells apart, and the
//     lanes of a read shared banks);
//  3. each wave takes items (dx row, 16-position segment): one A fragment
//     read per K step (lane = dx position), the MFMAs, one rounding, and
//     8-byte stores of 4
//     consecutive dx values per lane (2-byte stores at ragged or unaligned
//     rows).
#include <cstddef>
#include <algorithm>
#include <cstring>

#include "kcommon.h"
#include "launch.h"

namespace convt {

constexpr uint32_t kGbPermLo = 0x05040100u;  // {second.lo, first.lo}
constexpr uint32_t kGbPermHi = 0x07060302u;  // {second.hi, first.hi}

template <typename E> struct GbElem;
template <> struct GbElem<__bf16> {
    static __device__ __forceinline__ f32x4 mfma(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};
template <> struct GbElem<_Float16> {
    static __device__ __forceinline__ f32x4 mfma(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      c, 0, 0, 0);
    }
};

// KS: MFMA K steps (slots / 4, rounded up); ST8: dx rows are whole 8-byte
// pieces from an 8-byte aligned dx (4 values per lane in one store).
template <typename E, int KS, bool ST8>
__global__ __launch_bounds__(256) void grouped_bwd_kernel(GrpBwdArgs a, const uint16_t *__restrict__ dy,
                                                          const uint16_t *__restrict__ w,
                                                          uint16_t *__restrict__ dx) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Cig = a.Cig, Cog = a.Cog, noct = a.noct, HWP = a.hwp;
    // halo column c -> its cell within a (halo row, slice): with width stride
    // 2 the even columns come first, then the odd ones (sp = 2), else in order
    const int sp1 = a.sp - 1, hp = a.hp;
    auto cell = [&](int c) __attribute__((always_inline)) { return (c & sp1) * hp + (c >> sp1); };
    const unsigned char *kseg = (const unsigned char *)__builtin_amdgcn_kernarg_segment_ptr();
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)&lds[0];
    const int ntiles = a.G * a.B * a.nt_h;
    // tile t: row tile fastest, then batch, then group
    auto coords = [&](int t, int &b, int &g, int &i1_0) __attribute__((always_inline)) {
        const int r = t / a.nt_h, th = t - r * a.nt_h;
        g = r / a.B;
        b = r - g * a.B;
        i1_0 = th * a.R;
    };

    // the group's W, as stored, -> LDS at w_off (1 KiB pieces per wave
    // instruction; the area is whole pieces); asynchronous, no registers
    const int nw = (Cig * Cog * a.ktot) >> 3;  // 16-byte pieces
    const u32x4 wrw = rsrc_words(w, (uint32_t)a.Ci * (uint32_t)Cog * (uint32_t)a.ktot * 2u);
    auto w_copy = [&](int g) __attribute__((always_inline)) {
        const int tpc = a.w_tap_pieces;
        for (int j = wave; j * 64 < nw; j += 4) {  // uniform
            const int pc = j * 64 + lane;
            uint32_t off;
            if (tpc == 0) {  // uniform: one run of the group's elements
                off = (uint32_t)(g * nw + pc) * 16u;
            } else {  // tap by tap: each tap's run of the group
                const int st = div_small(pc, tpc);
                off = ((uint32_t)(st * a.G + g) * (uint32_t)tpc + (uint32_t)(pc - st * tpc)) * 16u;
            }
            copy_to_lds<16>(lds_base + (uint32_t)a.w_off + (uint32_t)j * 1024, pc < nw ? off : kOutOfRange, wrw);
        }
    };

    // dy's halo: halo row hr is dy row S1 * i1_0 - P1 + hr, cell column hc
    // is dy column hc - P2. This thread's load unit (at most one: the
    // planner keeps the units within 256) = (halo row, slice, chunk k of 8
    // dy positions 8k .. 8k+7), cells P2 + 8k .. +7 of the row; rows outside
    // dy read zero. Chunks are fastest, so 8 neighbouring lanes read a row's
    // 128 contiguous bytes of one channel per load.
    const uint32_t ypl_bytes = (uint32_t)a.y_plane * 2u;
    const int nrs = a.hr * noct;  // (halo row, slice) pairs
    const int nk = a.O2 >> 3;
    const bool has_unit = tid < nrs * nk;
    const int u_rs = div_small(tid, nk), u_k = tid - u_rs * nk;
    const int u_hr = div_small(u_rs, noct), u_oct = u_rs - u_hr * noct;
    unsigned char *u_dst = lds + u_rs * HWP * 16;
    const int u_c0 = a.P2 + 8 * u_k;  // halo column of the unit's first position
    auto halo_load = [&](int b, int g, int i1_0, u32x4 (&v)[8]) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t ys = make_rsrc_uniform(
            dy + ((int64_t)b * a.Co + (int64_t)g * Cog) * a.y_plane, (uint32_t)Cog * ypl_bytes);
        const int oh = a.S1 * i1_0 - a.P1 + u_hr;
        const uint32_t off = (oh >= 0 && oh < a.O1)
                                 ? (uint32_t)(u_oct * 8) * ypl_bytes + (uint32_t)(oh * a.O2 + 8 * u_k) * 2u
                                 : kOutOfRange;
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = __builtin_amdgcn_raw_buffer_load_b128(ys, off + c * ypl_bytes, 0, 0);
    };
    // v[c]: positions 8k .. 8k+7 of channel 8 oct + c -> 8 cells (position
    // 8k + e, channels 2i, 2i+1 in word i)
    auto halo_store = [&](const u32x4 (&v)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            u32x4 cv;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                cv[i] = __builtin_amdgcn_perm(v[2 * i + 1][e >> 1], v[2 * i][e >> 1], (e & 1) ? kGbPermHi : kGbPermLo);
            *(u32x4 *)(u_dst + cell(u_c0 + e) * 16) = cv;
        }
    };

    // zero cells (columns left of dy, P2 of them, and right of it): the same
    // for every tile, written once
    {
        const int zn = a.hwr - a.O2, zunits = nrs * zn;
        for (int u = tid; u < zunits; u += 256) {
            const int rs = div_small(u, zn), z = u - rs * zn;
            const int col = z < a.P2 ? z : z + a.O2;
            *(u32x4 *)(lds + (rs * HWP + cell(col)) * 16) = u32x4{0u, 0u, 0u, 0u};
        }
    }

    // per lane, tile-independent: slot = 4 kb + kg4, its halo byte offset for
    // dx row 0, position 0; its slab row (input channel l16; channels past
    // Cig take the last one, their columns are never stored)
    const int l16 = lane & 15, kg4 = lane >> 4;
    const int32_t *slot_w = (const int32_t *)(kseg + offsetof(GrpBwdArgs, slot_w));
    const int32_t *slot_h = (const int32_t *)(kseg + offsetof(GrpBwdArgs, slot_h));
    uint32_t aoff[KS];
#pragma unroll
    for (int kb = 0; kb < KS; ++kb) {
        const int slot = 4 * kb + kg4;
        aoff[kb] = (uint32_t)slot_h[slot < a.nslots ? slot : 0];
    }
    const unsigned char *slab = lds + a.slab_off + min(l16, Cig - 1) * kGbSlabPitch;
    const int nseg = (a.I2 + 15) >> 4;
    const uint32_t xpl_bytes = (uint32_t)a.x_plane * 2u;
    const uint32_t lane_x = l16 < Cig ? (uint32_t)l16 * xpl_bytes : kOutOfRange;
    const uint32_t row_lds = (uint32_t)(a.S1 * noct * HWP * 16);  // halo bytes per dx row

    // Persistent blocks: tiles blockIdx.x, + gridDim.x, ... Each tile's halo
    // loads (registers) and weight copy (LDS) are issued before the previous
    // tile's MFMAs and stores, so they overlap them.
    int t = blockIdx.x;
    if (t >= ntiles) return;  // uniform (the host launches at most ntiles blocks)
    int b, g, i1_0;
    coords(t, b, g, i1_0);
    u32x4 v[8];
    if (has_unit) halo_load(b, g, i1_0, v);
    w_copy(g);
    for (;;) {  // uniform
        if (has_unit) halo_store(v);
        // this tile's halo cells are written and its weight copy has landed
        // (all of the wave's vector memory operations: loads and stores are
        // not ordered against each other, so the previous tile's stores are
        // waited for too)
        stage_barrier<0>();
        // the fragment slab: thread t builds (input channel t / 16, slot
        // t % 16), the slot's 8 dy channels of that input channel read from
        // W as stored (channel strides w_sci, w_sco), written as one 16-byte
        // row at [channel][slot] (pitch 17 slots: the 16 lanes of a fragment
        // read fall on distinct banks). Slots past nslots are zero.
        {
            const int ci = tid >> 4, slot = tid & 15;
            if (ci < Cig) {
                u32x4 wv = {0u, 0u, 0u, 0u};
                if (slot < a.nslots) {
                    const unsigned char *wp = lds + a.w_off + ci * a.w_sci + slot_w[slot];
                    const int wsco = a.w_sco;
                    if (wsco == 2) {  // uniform: the 8 dy channels are adjacent
                        wv = *(const u32x4 *)wp;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            wv[i] = (uint32_t)*(const uint16_t *)(wp + 2 * i * wsco) |
                                    (uint32_t)*(const uint16_t *)(wp + (2 * i + 1) * wsco) << 16;
                    }
                }
                *(u32x4 *)(lds + a.slab_off + ci * kGbSlabPitch + slot * 16) = wv;
            }
        }
        __syncthreads();  // the slab is built; W's area is free for the next copy
        const int tn = t + gridDim.x;
        const bool more = tn < ntiles;  // uniform
        int bn = 0, gn = 0, i1n = 0;
        if (more) {
            coords(tn, bn, gn, i1n);
            if (has_unit) halo_load(bn, gn, i1n, v);
            w_copy(gn);
        }
        u32x4 bw[KS];
#pragma unroll
        for (int kb = 0; kb < KS; ++kb) bw[kb] = *(const u32x4 *)(slab + (4 * kb + kg4) * 16);

        // items (dx row r, segment sg) of this tile dealt to the waves in turn
        const int rows = min(a.R, a.I1 - i1_0);
        const __amdgpu_buffer_rsrc_t xs = make_rsrc_uniform(
            dx + ((int64_t)b * a.Ci + (int64_t)g * Cig) * a.x_plane, (uint32_t)Cig * xpl_bytes);
        int r = 0, sg = wave;
        while (sg >= nseg) {  // uniform
            sg -= nseg;
            ++r;
        }
        for (; r < rows;) {  // uniform
            // this lane's dx position (clamped into the row for the read)
            const int i2 = sg * 16 + l16;
            const uint32_t abase = (uint32_t)r * row_lds + (uint32_t)((a.S2 >> sp1) * min(i2, a.I2 - 1) * 16);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KS; ++kb) {
                const u32x4 av = *(const u32x4 *)(lds + abase + aoff[kb]);
                acc = GbElem<E>::mfma(av, bw[kb], acc);
            }
            // lane: input channel l16, dx positions sg*16 + 4 kg4 + j
            const int p0 = sg * 16 + 4 * kg4;
            const uint32_t rowoff = (uint32_t)((i1_0 + r) * a.I2 + p0) * 2u;
            const uint32_t w0 = pack_half2<E>(acc[0], acc[1]), w1 = pack_half2<E>(acc[2], acc[3]);
            if constexpr (ST8) {
                if (p0 < a.I2) __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, xs, lane_x + rowoff, 0, 0);
            } else {
                const uint32_t wv2[2] = {w0, w1};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (p0 + j < a.I2)
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(wv2[j >> 1] >> (16 * (j & 1))), xs,
                                                              lane_x + rowoff + 2u * j, 0, 0);
            }
            sg += 4;
            while (sg >= nseg) {  // uniform
                sg -= nseg;
                ++r;
            }
        }
        if (!more) break;
        // every wave is done reading the halo and the slab before the next
        // tile's cells and slab overwrite them
        __syncthreads();
        t = tn;
        b = bn;
        g = gn;
        i1_0 = i1n;
    }
}

// one block per resident slot (blocks per CU by occupancy x CUs), at most
// one per tile
template <typename K>
static int gb_grid(K kernel, int lds_bytes, int ntiles) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, (size_t)lds_bytes) != hipSuccess ||
        cus <= 0 || per_cu <= 0)
        return ntiles;
    return (int)std::min<int64_t>((int64_t)cus * per_cu, ntiles);
}

template <typename E, int KS>
static void launch_gb_e(const Plan &pl, const void *dy, const void *w, void *dx, bool st8, hipStream_t stream) {
    const GrpBwdArgs &a = pl.gb;
    const int ntiles = a.G * a.B * a.nt_h;
    const uint16_t *d = (const uint16_t *)dy, *ww = (const uint16_t *)w;
    uint16_t *o = (uint16_t *)dx;
    if (st8) {
        auto k = grouped_bwd_kernel<E, KS, true>;
        hipLaunchKernelGGL(k, dim3(gb_grid(k, a.lds_bytes, ntiles)), dim3(256), (size_t)a.lds_bytes, stream, a, d,
                           ww, o);
    } else {
        auto k = grouped_bwd_kernel<E, KS, false>;
        hipLaunchKernelGGL(k, dim3(gb_grid(k, a.lds_bytes, ntiles)), dim3(256), (size_t)a.lds_bytes, stream, a, d,
                           ww, o);
    }
}

template <typename E>
static hipError_t launch_gb_t(const Plan &pl, const void *dy, const void *w, void *dx, bool st8, hipStream_t stream) {
    switch (pl.gb.ks) {
        case 1: launch_gb_e<E, 1>(pl, dy, w, dx, st8, stream); break;
        case 2: launch_gb_e<E, 2>(pl, dy, w, dx, st8, stream); break;
        case 3: launch_gb_e<E, 3>(pl, dy, w, dx, st8, stream); break;
        case 4: launch_gb_e<E, 4>(pl, dy, w, dx, st8, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipSuccess;
}

hipError_t launch_grouped_bwd(const Plan &pl, const void *dy, const void *w, void *dx, hipStream_t stream) {
    const GrpBwdArgs &a = pl.gb;
    if (a.B == 0 || a.nt_h == 0 || a.G == 0) return hipSuccess;
    if ((int64_t)a.G * a.B * a.nt_h > 0x7fffffff) return hipErrorInvalidConfiguration;
    // 8-byte stores: dx rows of whole 8-byte pieces from an 8-byte aligned dx
    const bool st8 = a.I2 % 4 == 0 && (uintptr_t)dx % 8 == 0;
    const hipError_t e = pl.dp.f16 ? launch_gb_t<_Float16>(pl, dy, w, dx, st8, stream)
                                   : launch_gb_t<__bf16>(pl, dy, w, dx, st8, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace convt
