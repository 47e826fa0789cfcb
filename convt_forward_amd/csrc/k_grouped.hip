// Grouped / few-channel stride-phase kernel (bfloat16 or half, MFMA
// 16x16x32).
//
// For grouped problems with few channels per group (C_in/groups a multiple
// of 8 up to 64, C_out/groups up to 16) the phase GEMM's tiles would be
// mostly empty. Here one block owns one (batch, group) and a tile of q rows
// at one q-depth, over the full q width, for EVERY stride phase. This keeps
// the idea of the grouped stride-phase blocked variant that the huggingface
// ai.onnx.ConvTranspose page lists under Implementation variants: the work
// unit is a set of output pixels times all of its group's output channels,
// so each input value read serves every one of those channels, and the
// group's weights are brought on chip once per block.
//
// The work per output is tiny (a few K slots) and the output is 4x the
// input, so the kernel is written for a small instruction count per stored
// byte and for stores that write whole 128-byte rows:
//  1. the group's part of W, as stored, and a slot table (a record per
//     phase; per (tap, 8-channel slice) slot the LDS offset of the tap's
//     window and the byte offset of the tap's weights in that part of W),
//     built by the planner and passed with the kernel's arguments, are
//     copied to LDS; the block then gathers each MFMA weight fragment (8
//     input channels of one output channel for one slot) once into a slab
//     [output channel][slot] of 16-byte entries written over the stored
//     copy; the input halo (the q tile grown by the union of all
//     phases' input windows) goes to LDS as 16-byte cells of 8 channels,
//     [halo row][slice][column]. When x rows are whole 16-byte chunks, a lane
//     loads 8 positions of each of 8 channels (eight 16-byte loads),
//     transposes the 8 x 8 block in registers (v_perm) and writes 8 cells;
//     otherwise it falls back to 2-byte loads;
//  2. per (depth, height) residue pair, a wave reads the weight fragments of
//     every width residue from the slab into registers and takes chunks of 16-position
//     segments of the block's q rows in turn: per segment and width residue
//     up to four 16x16x32 MFMAs (rows = 16 positions, columns =
//     the group's output channels padded to 16, K = (tap, slice) slots, four
//     per MFMA), with the bias as the accumulator's initial value. A lane
//     then holds, for one channel, 4*S2 consecutive outputs of one row;
//  3. the outputs (after the activation, if any) are rounded to the element
//     type in pairs and leave as 16-byte
//     stores in which 8 consecutive lanes cover 128 contiguous bytes: with
//     width stride 2 and at most 8 channels, a segment pair's second half
//     moves into the padding lanes (DPP) and a lane permutation orders the
//     row pieces; otherwise chunks go through a per-wave LDS staging area.
//     Edge segments are stored straight from registers.
#include <cstddef>
#include <cstring>

#include "kcommon.h"
#include "launch.h"

namespace convt {

constexpr int kGrpRsrcWord3 = 0x00020000;
constexpr uint32_t kGrpOutOfRange = 0x80000000u;
// flag in the kernel's st_align argument: y takes 16-byte stores of row
// pieces (the low bits hold the widest aligned store of a lane's run)
constexpr int kStageOk = 32;

// v_perm_b32 selectors pairing the low (resp. high) 16-bit halves of two
// words: result = {second.lo, first.lo} (resp. {second.hi, first.hi}).
constexpr uint32_t kPermLo = 0x05040100u;
constexpr uint32_t kPermHi = 0x07060302u;

template <bool B> struct BoolTag {
    static constexpr bool value = B;
};
template <int V> struct IntTag {
    static constexpr int value = V;
};

// One 16x16x32 MFMA step on two-byte elements of type E (bfloat16 or half).
template <typename E> struct GrpElem;
template <> struct GrpElem<__bf16> {
    typedef bf16x8 v8;
    static __device__ __forceinline__ f32x4 mfma(const u32x4 &a, const v8 &b, const f32x4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), b, c, 0, 0, 0);
    }
};
template <> struct GrpElem<_Float16> {
    typedef f16x8 v8;
    static __device__ __forceinline__ f32x4 mfma(const u32x4 &a, const v8 &b, const f32x4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), b, c, 0, 0, 0);
    }
};

// a lane's run of 4*S2 outputs (2*S2 words) into the staging row
template <int S2>
__device__ __forceinline__ void stage_run_t(const uint32_t *pk, unsigned char *w) {
    if constexpr ((S2 & 1) == 0) {
#pragma unroll
        for (int k = 0; k < S2 / 2; ++k)
            *(u32x4 *)(w + 16 * k) = u32x4{pk[4 * k], pk[4 * k + 1], pk[4 * k + 2], pk[4 * k + 3]};
    } else {
#pragma unroll
        for (int k = 0; k < S2; ++k) *(u32x2 *)(w + 8 * k) = u32x2{pk[2 * k], pk[2 * k + 1]};
    }
}

// The kernel's arguments: the plan fields it reads, packed into a few cache
// lines (kernel arguments are fetched line by line on first use).
struct GrpAxis {
    int32_t I, O, S, umin;
};
struct GrpArgs {
    GrpAxis ax[3];
    int32_t G, Ci, Co, Cig, Cog, has_bias;
    int32_t x_plane, y_plane;
    int32_t th, tw, hd, hh, hw;
    int32_t grp_hwp, grp_hshift, grp_nk, grp_nsc;
    int32_t grp_w_off, grp_tab_off, grp_st_off, grp_st_pitch, grp_slab_off, grp_ns;
    int32_t ktot, nphase;
    int32_t tab_n;                      // int2 entries of tab
    int32_t w_sc, w_so, w_tap_pieces;   // the group's weights as stored (GrpTables)
    int32_t tab[2 * kGrpTabMax];        // the slot table (GrpTables)
};

// Eight waves per SIMD (8 blocks per CU) where the registers allow it: the
// scalar registers are capped too, since more of them than the cap admits
// keep blocks from being resident. Instances with more weight fragments in
// registers (S2 * KS > 2) trade occupancy for having no spills.
//
// PD: the host has checked that every item takes the segment-pair path
// (width stride 2, at most 8 channels, whole segments, every phase's slots
// filling its K steps, y aligned for 16-byte row pieces); the instance holds
// only that path, none of the other paths' set-up.
template <int S2, int KS, typename E, int ACT, bool PD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(S2 * KS <= 2 ? 8 : 4, 8))) void grouped_kernel(
    GrpArgs p, const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ y, int st_align, int x_vec) {
    static_assert(!PD || S2 == 2, "the segment-pair path needs width stride 2");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    // uniform per wave: lets the plan tables be read with scalar loads
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // grid: (group + G * batch, row tile, q depth)
    const int th_i = blockIdx.y, qd = blockIdx.z;
    const int b = blockIdx.x / p.G, g = blockIdx.x - b * p.G;

    const GrpAxis &a0 = p.ax[0], &a1 = p.ax[1], &a2 = p.ax[2];
    const int Cig = p.Cig, noct = Cig >> 3;
    const int R = p.th, Qw = p.tw;
    const int HH = p.hh, HW = p.hw, HWP = p.grp_hwp;
    const int q0h = th_i * R;
    const int h0 = qd + a0.umin, h1 = q0h + a1.umin, h2 = a2.umin;
    const int nrow = p.hd * HH;

    // 1a. the group's part of W, as stored, and the slot table (a record per
    // phase, then per (tap, slice) slot the LDS byte offset of the tap's
    // window origin in the halo and the byte offset of its weights in the
    // group's part of W) -> LDS by DMA, in 1 KiB and 256-byte pieces dealt
    // to the waves (their areas are whole pieces). The weights need no
    // reordering: the MFMA fragments are gathered from them as stored (per
    // fragment eight input channels of one output channel, w_sc bytes apart)
    // into the slab below. The copies take no registers and land while the
    // halo is staged.
    {
        const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)&lds[0];
        const int npc = (Cig * p.Cog) >> 3;       // 16-byte pieces per tap
        const int nw = npc * p.ktot;              // ... of the group's weights
        const int tpc = p.w_tap_pieces;           // 0: one run, else tap by tap
        const u32x4 wrw = rsrc_words(w, (uint32_t)p.Ci * (uint32_t)p.Cog * (uint32_t)p.ktot * 2u);
        const uint32_t w_lds = lds_base + (uint32_t)p.grp_w_off;
        for (int j = wave; j * 64 < nw; j += 4) {  // uniform
            const int pc = j * 64 + lane;
            uint32_t off;
            if (tpc == 0) {  // uniform
                off = (uint32_t)(g * nw + pc) * 16u;
            } else {
                const int st = div_small(pc, tpc);
                off = ((uint32_t)(st * p.G + g) * (uint32_t)tpc + (uint32_t)(pc - st * tpc)) * 16u;
            }
            copy_to_lds<16>(w_lds + (uint32_t)j * 1024, pc < nw ? off : kOutOfRange, wrw);
        }
        const unsigned char *kseg = (const unsigned char *)__builtin_amdgcn_kernarg_segment_ptr();
        const u32x4 trw = rsrc_words(kseg + offsetof(GrpArgs, tab), (uint32_t)p.tab_n * 8u);
        const uint32_t t_lds = lds_base + (uint32_t)p.grp_tab_off;
        for (int j = wave; j * 64 < 2 * p.tab_n; j += 4)  // uniform
            copy_to_lds<4>(t_lds + (uint32_t)j * 256, (uint32_t)(j * 64 + lane) * 4, trw);
    }
    // 1b. input halo -> LDS cells; positions outside the input read an
    // out-of-range offset (zero).
    const uint32_t xpl_bytes = (uint32_t)p.x_plane * 2;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x + ((int64_t)b * p.Ci + (int64_t)g * Cig) * p.x_plane), (short)0,
        (int)((uint32_t)Cig * xpl_bytes), kGrpRsrcWord3);
    const int nk = p.grp_nk, col0 = p.grp_hshift - a2.umin;
    if (x_vec) {  // uniform
        // zero cells: columns left of the row (col0 of them) and right of it
        const int zl = col0, zn = HWP - a2.I;
        const int zunits = nrow * noct * zn;
        for (int u = tid; u < zunits; u += 256) {
            const int ro = div_small(u, zn), z = u - ro * zn;
            const int col = z < zl ? z : z + a2.I;
            *(u32x4 *)(lds + (ro * HWP + col) * 16) = u32x4{0u, 0u, 0u, 0u};
        }
    }
    if (x_vec) {  // uniform
        // unit = (halo row, slice, chunk k of 8 input positions 8k .. 8k+7),
        // whose cells are columns col0 + 8k .. +7 of the row; rows outside the
        // input read zero. Neighbouring lanes take neighbouring rows, whose
        // cells the odd row pitch spreads over the LDS banks.
        const int units = nrow * noct * nk;
        // unit u's source offset (out of range for rows outside the input
        // and past the last unit) and its first cell
        auto unit_at = [&](int u, unsigned char *&dst) __attribute__((always_inline)) {
            const int t = div_small(u, nrow), row = u - t * nrow;
            const int k = div_small(t, noct), oct = t - k * noct;
            const int d = div_small(row, HH), h = row - d * HH;
            const int i0 = h0 + d, i1 = h1 + h;
            const bool ok = u < units && i0 >= 0 && i0 < a0.I && i1 >= 0 && i1 < a1.I;
            dst = lds + ((row * noct + oct) * HWP + col0 + 8 * k) * 16;
            return ok ? (uint32_t)(oct * 8) * xpl_bytes + (uint32_t)((i0 * a1.I + i1) * a2.I + 8 * k) * 2
                      : kGrpOutOfRange;
        };
        // v[c]: positions 8k .. 8k+7 of channel 8*oct + c
        auto unit_load = [&](uint32_t off, u32x4 (&v)[8]) __attribute__((always_inline)) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
                v[c] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off + c * xpl_bytes, 0, 0);
        };
        auto unit_store = [&](const u32x4 (&v)[8], unsigned char *dst) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u32x4 cell;  // position 8k + e, channels 2i, 2i+1 in word i
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    cell[i] = __builtin_amdgcn_perm(v[2 * i + 1][e >> 1], v[2 * i][e >> 1],
                                                    (e & 1) ? kPermHi : kPermLo);
                *(u32x4 *)(dst + e * 16) = cell;
            }
        };
        for (int u = tid; u < units; u += 256) {
            unsigned char *dst;
            u32x4 v[8];
            unit_load(unit_at(u, dst), v);
            unit_store(v, dst);
        }
    } else {
        // Element loads: a wave takes whole halo rows (one slice each) and its
        // lanes walk the row's positions. (slice, depth, row) triples are
        // dealt to the waves in turn; a wave issues the loads of four of its
        // rows before writing any of them.
        const int total = nrow * noct, hshift = p.grp_hshift;
        int pr = wave, oct = 0, c0 = 0, c1 = wave;
        auto norm = [&]() __attribute__((always_inline)) {
            while (c1 >= HH) {
                c1 -= HH;
                if (++c0 == p.hd) {
                    c0 = 0;
                    ++oct;
                }
            }
        };
        norm();
        for (int c2b = 0; c2b < HW; c2b += 64) {
            int spr = pr, soct = oct, sc0 = c0, sc1 = c1;
            const int c2 = c2b + lane;
            const int i2 = h2 + c2;
            const bool col_ok = c2 < HW && i2 >= 0 && i2 < a2.I;
            while (spr < total) {  // uniform
                u32x4 v[4];
                int dst[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    dst[u] = -1;
                    if (spr < total) {  // uniform
                        const int i0 = h0 + sc0, i1 = h1 + sc1;
                        const bool ok = col_ok && i0 >= 0 && i0 < a0.I && i1 >= 0 && i1 < a1.I;
                        const uint32_t off =
                            ok ? (uint32_t)(soct * 8) * xpl_bytes +
                                     (uint32_t)((i0 * a1.I + i1) * a2.I + i2) * 2
                               : kGrpOutOfRange;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
                                xrs, off + (2 * e) * xpl_bytes, 0, 0);
                            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
                                xrs, off + (2 * e + 1) * xpl_bytes, 0, 0);
                            v[u][e] = lo | (hi << 16);
                        }
                        dst[u] = (((sc0 * HH + sc1) * noct + soct) * HWP + c2 + hshift) * 16;
                        spr += 4;
                        sc1 += 4;
                        while (sc1 >= HH) {
                            sc1 -= HH;
                            if (++sc0 == p.hd) {
                                sc0 = 0;
                                ++soct;
                            }
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (dst[u] >= 0 && c2 < HW) *(u32x4 *)(lds + dst[u]) = v[u];
            }
        }
    }
    const int4 *precs = (const int4 *)(lds + p.grp_tab_off);
    const int2 *tab = (const int2 *)(lds + p.grp_tab_off + 16 * p.nphase);
    // every wave's copies (weights, table; halo without DMA) have landed and
    // the cells are written
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // the weight-fragment slab, built in place of the weights: entry (output
    // channel co, slot s) holds the slot's 8 input channels of channel co,
    // gathered from W as stored (the slot's weight offset from the table,
    // channel strides w_so, w_sc); rows of ns | 1 slots, so the 16 lanes of
    // a fragment read fall on distinct banks (read per pair straight from the
    // stored layout, they conflicted). Each thread gathers its entries (at
    // most 4: the group's weights are at most 16 KiB) into registers before
    // any is written.
    const int ns = p.grp_ns, slab_pitch = (ns | 1) * 16;
    {
        const int wsc = p.w_sc, nent = p.Cog * ns;
        u32x4 ent[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i;
            if (e < nent) {
                const int co = div_small(e, ns), sl = e - co * ns;
                const unsigned char *wp = lds + p.grp_w_off + co * p.w_so + tab[sl].y;
                if (wsc == 2) {  // uniform: the eight channels are adjacent
                    ent[i] = *(const u32x4 *)wp;
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        ent[i][k] = (uint32_t)*(const uint16_t *)(wp + 2 * k * wsc) |
                                    (uint32_t)*(const uint16_t *)(wp + (2 * k + 1) * wsc) << 16;
                }
            }
        }
        __syncthreads();  // every gather has read the weights
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i;
            if (e < nent) {
                const int co = div_small(e, ns), sl = e - co * ns;
                *(u32x4 *)(lds + p.grp_slab_off + co * slab_pitch + sl * 16) = ent[i];
            }
        }
    }
    __syncthreads();

    // 2. Per (depth residue, height residue) pair, each wave takes chunks of
    // nsc 16-position segments of the block's q rows in turn. For a segment
    // it runs the MFMA chain of every width residue r2 < S2, so lane l
    // (channel l%16, positions 4*(l/16) + i of the segment) holds the
    // outputs ow = S2*q + r2 for four consecutive q and every r2: a run of
    // 4*S2 outputs of one output row.
    // 3. Whole chunks go through the wave's LDS staging area,
    // [channel][chunk of the output row], and leave as 16-byte pieces of
    // whole rows (1 KiB per store instruction at the workloads' shapes);
    // other segments are stored from registers.
    const int l16 = lane & 15, kg4 = lane >> 4;
    const int Cog = p.Cog;
    const int O2 = a2.O;
    // this lane's row of the fragment slab (the padding channels take the
    // last one: their columns are never stored)
    const unsigned char *slab_lane = lds + p.grp_slab_off + min(l16, Cog - 1) * slab_pitch;
    const int nseg = (Qw + 15) >> 4;
    // nsc == 0: width stride 2, at most 8 channels, an even segment count:
    // chunks are segment pairs that leave through DPP (no staging)
    const bool pair_dpp = p.grp_nsc == 0;
    const int nsc = pair_dpp ? 2 : p.grp_nsc, nchunk = (nseg + nsc - 1) / nsc;
    const float bvf = (p.has_bias && l16 < Cog) ? half_to_f32<E>(bias[g * Cog + l16]) : 0.0f;
    // the outputs' activation, then one rounding to E, two per word
    auto pack2 = [](float a, float b) __attribute__((always_inline)) {
        if constexpr (ACT != CONVT_ACT_NONE) {
            a = activate<true>(ACT, a);
            b = activate<true>(ACT, b);
        }
        return pack_half2<E>(a, b);
    };
    const f32x4 binit = {bvf, bvf, bvf, bvf};
    // output planes of the group; a lane's channel plane, or out of range
    // (dropped) for the padding channels
    const uint32_t ypl_bytes = (uint32_t)p.y_plane * 2;
    // (built from lane 0's words: kept in scalar registers, no per-store
    // loop over the lanes' resources)
    const __amdgpu_buffer_rsrc_t ys = make_rsrc_uniform(
        y + ((int64_t)b * p.Co + (int64_t)g * Cog) * p.y_plane, Cog * ypl_bytes, kGrpRsrcWord3);
    const uint32_t lane_st =
        (l16 < Cog ? (uint32_t)l16 * ypl_bytes : kGrpOutOfRange) + (uint32_t)(S2 * 4 * kg4) * 2;
    // staging: this lane's run in segment s of a chunk at st_w + s * 32 * S2
    // (the padding channels' lanes all write one spare row); read back in
    // passes of 1 KiB, flat byte f = 1024 * pass + 16 * lane of the chunk's
    // [channel][cb] bytes
    const int st_pitch = p.grp_st_pitch;
    const uint32_t cb = (uint32_t)(nsc * S2 * 32);
    unsigned char *stg = lds + p.grp_st_off + wave * (Cog + 1) * st_pitch;
    const uint32_t st_w = (uint32_t)(min(l16, Cog) * st_pitch + kg4 * S2 * 8);
    const int st_tot = Cog * (int)cb, npass = (st_tot + 1023) >> 10;
    // DPP pairs: after the merge, lane 16k + 8h + c holds 16-byte piece
    // 4h + k of channel c's 128-byte row; a lane permutation then gives lane
    // 8c + j piece j of channel c, so that 8 consecutive lanes store a row
    const int bp_src = 4 * (16 * (lane & 3) + 8 * ((lane >> 2) & 1) + (lane >> 3));
    const uint32_t dpp_st =
        ((lane >> 3) < Cog ? (uint32_t)(lane >> 3) * ypl_bytes : kGrpOutOfRange) + (uint32_t)((lane & 7) * 16);
    uint32_t st_r[2], st_y[2];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
        const int f = 1024 * ps + 16 * lane;
        const int c = f / (int)cb, o = f - c * (int)cb;
        st_r[ps] = f < st_tot ? (uint32_t)(c * st_pitch + o) : 0u;
        st_y[ps] = f < st_tot ? (uint32_t)c * ypl_bytes + (uint32_t)o : kGrpOutOfRange;
    }
    const uint32_t row_lds = (uint32_t)(noct * HWP * 16);  // halo bytes per q row
    // this wave's chunks are items wave, wave + 4, ... of (row, chunk): per
    // step the chunk advances by dc and the row by dq (plus a carry)
    const int dq = 4 / nchunk, dc = 4 - dq * nchunk;
    const int ql0 = wave / nchunk, ch0 = wave - ql0 * nchunk;
    const uint32_t yrow_bytes = (uint32_t)(a1.S * O2 * 2);  // y bytes per q row
    const uint32_t seg_lds = 256, seg_y = (uint32_t)(S2 * 32);  // per segment
    // offsets advance by dq rows and dc chunks per step, plus one row minus a
    // row's chunks on a carry
    const uint32_t ub_step = (uint32_t)dq * row_lds + (uint32_t)(dc * nsc) * seg_lds;
    const uint32_t so_step = (uint32_t)dq * yrow_bytes + (uint32_t)(dc * nsc) * seg_y;
    const uint32_t ub_wrap = row_lds - (uint32_t)(nchunk * nsc) * seg_lds;
    const uint32_t so_wrap = yrow_bytes - (uint32_t)(nchunk * nsc) * seg_y;
    constexpr int MS = S2;  // width residues kept in registers
    auto stage_run = [](const uint32_t *pk, unsigned char *w) __attribute__((always_inline)) {
        stage_run_t<S2>(pk, w);
    };
    // the tile's q rows [rlo, rhi), every phase
    auto compute_rows = [&](int rlo, int rhi) __attribute__((always_inline)) {
    const int qb0 = rlo + ql0;  // this wave's first row
    for (int r0 = 0; r0 < a0.S; ++r0) {
        for (int r1 = 0; r1 < a1.S; ++r1) {
            // phases (r0, r1, r2 < S2): their records and this lane's K slots
            int qn0 = 0, qn1 = 0, qn2min = 1 << 30, qn2[MS];
            uint32_t rd[MS][KS];  // LDS byte offset of the lane's A cell, segment origin excluded
            typename GrpElem<E>::v8 bw[MS][KS];
            bool sl_ok[MS][KS];
            bool regular = true;  // every phase fills all KS steps with real slots (uniform)
#pragma unroll
            for (int r2 = 0; r2 < MS; ++r2) {
                // record: q counts per axis, then slot base | slot count << 16
                const int4 rec = precs[(r0 * a1.S + r1) * S2 + r2];
                qn0 = __builtin_amdgcn_readfirstlane(rec.x);
                qn1 = __builtin_amdgcn_readfirstlane(rec.y);
                qn2[r2] = __builtin_amdgcn_readfirstlane(rec.z);
                qn2min = min(qn2min, qn2[r2]);
                const int sw = __builtin_amdgcn_readfirstlane(rec.w);
                const int sbase = sw & 0xffff, nslots = sw >> 16;
                regular = regular && nslots == 4 * KS;
#pragma unroll
                for (int kb = 0; kb < KS; ++kb) {
                    const int slot = kb * 4 + kg4;
                    sl_ok[r2][kb] = PD || slot < nslots;
                    int2 e = make_int2(0, 0);
                    u32x4 wv = {0u, 0u, 0u, 0u};
                    if (sl_ok[r2][kb]) {
                        e = tab[sbase + slot];
                        wv = *(const u32x4 *)(slab_lane + (sbase + slot) * 16);
                    }
                    rd[r2][kb] = (uint32_t)e.x + (uint32_t)l16 * 16;
                    bw[r2][kb] = __builtin_bit_cast(typename GrpElem<E>::v8, wv);
                }
            }
            const int rows = min(rhi, qn1 - q0h) - rlo;  // q rows of the range with outputs here
            if (qd >= qn0 || rows <= 0) continue;  // uniform
            const int nitems = rows * nchunk;
            // segments whose 16 positions are inside every residue's q range;
            // chunks of only such segments are staged when y takes 16-byte
            // stores of row pieces
            const int nfull = min(nseg, qn2min >> 4);
            const int nstaged = (!pair_dpp && (st_align & kStageOk)) ? nfull / nsc : 0;  // no staging area with DPP pairs
            const bool seg_b128 = (MS & 1) == 0 && (st_align & 31) >= 16;
            const uint32_t so0 = (uint32_t)(((int64_t)(a0.S * qd + r0) * a1.O + a1.S * q0h + r1) * O2 * 2);
            // the chunk loop, instantiated without (regular) and with masks
            // for the padding slots (A cells of padding slots read as zero)
            auto run_items = [&](auto pad_tag) __attribute__((always_inline)) {
                constexpr bool PAD = decltype(pad_tag)::value;
                int it = wave, ch = ch0;
                // LDS offset and y offset of the chunk (uniform), advanced with it
                uint32_t ub = (uint32_t)qb0 * row_lds + (uint32_t)(ch0 * nsc) * seg_lds;
                uint32_t so = so0 + (uint32_t)qb0 * yrow_bytes + (uint32_t)(ch0 * nsc) * seg_y;
                while (it < nitems) {  // uniform
                    const bool staged = ch < nstaged;
                    for (int s = 0; s < nsc; ++s) {  // uniform
                        const int seg = ch * nsc + s;
                        if (seg >= nseg) break;
                        const uint32_t ubs = ub + (uint32_t)s * seg_lds, sos = so + (uint32_t)s * seg_y;
                        f32x4 acc[MS];
#pragma unroll
                        for (int r2 = 0; r2 < MS; ++r2) {
                            acc[r2] = binit;
#pragma unroll
                            for (int kb = 0; kb < KS; ++kb) {
                                u32x4 av = *(const u32x4 *)(lds + rd[r2][kb] + ubs);
                                if constexpr (PAD) {
                                    if (!sl_ok[r2][kb]) av = u32x4{0u, 0u, 0u, 0u};
                                }
                                acc[r2] = GrpElem<E>::mfma(av, bw[r2][kb], acc[r2]);
                            }
                        }
                        // the run's 4*S2 outputs as 2*S2 words (word e2:
                        // outputs 2*e2, 2*e2 + 1; output index S2*i + r2)
                        uint32_t pk[2 * MS];
#pragma unroll
                        for (int e2 = 0; e2 < 2 * MS; ++e2) {
                            const int ea = 2 * e2, eb = 2 * e2 + 1;
                            pk[e2] = pack2(acc[ea % S2][ea / S2], acc[eb % S2][eb / S2]);
                        }
                        if (staged) {  // uniform
                            stage_run(pk, stg + st_w + (uint32_t)s * seg_y);
                            continue;
                        }
                        const int q0 = seg * 16;
                        if (seg_b128 && seg < nfull) {  // uniform: 16-byte runs, all inside
                            if constexpr ((MS & 1) == 0) {
#pragma unroll
                                for (int k = 0; k < MS / 2; ++k)
                                    __builtin_amdgcn_raw_buffer_store_b128(
                                        u32x4{pk[4 * k], pk[4 * k + 1], pk[4 * k + 2], pk[4 * k + 3]},
                                        ys, lane_st + k * 16, sos, 0);
                            }
                            continue;
                        }
                        const int qb = q0 + 4 * kg4;
                        bool full = true;  // every output of the lane's run inside the row
#pragma unroll
                        for (int r2 = 0; r2 < MS; ++r2) full = full && (qb + 3 < qn2[r2]);
                        const int al = st_align & 31;
                        if (full && al >= 8) {
#pragma unroll
                            for (int k = 0; k < MS; ++k)
                                __builtin_amdgcn_raw_buffer_store_b64(u32x2{pk[2 * k], pk[2 * k + 1]}, ys,
                                                                      lane_st + k * 8, sos, 0);
                        } else if (full && al >= 4) {
#pragma unroll
                            for (int e2 = 0; e2 < 2 * MS; ++e2)
                                __builtin_amdgcn_raw_buffer_store_b32(pk[e2], ys, lane_st + e2 * 4, sos, 0);
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
#pragma unroll
                                for (int r2 = 0; r2 < MS; ++r2) {
                                    const int e = S2 * i + r2;
                                    if (qb + i < qn2[r2])
                                        __builtin_amdgcn_raw_buffer_store_b16(
                                            (uint16_t)(pk[e >> 1] >> (16 * (e & 1))), ys,
                                            lane_st + e * 2, sos, 0);
                                }
                        }
                    }
                    if (staged) {  // uniform
                        // the wave's LDS accesses complete in order: the
                        // staged runs are read back after their writes, and
                        // the next chunk's writes follow these reads
                        asm volatile("" ::: "memory");
                        for (int ps = 0; ps < npass; ++ps) {  // uniform
                            const u32x4 v = *(const u32x4 *)(stg + st_r[ps]);
                            __builtin_amdgcn_raw_buffer_store_b128(v, ys, st_y[ps], so, 0);
                        }
                        asm volatile("" ::: "memory");
                    }
                    it += 4;
                    ch += dc;
                    ub += ub_step;
                    so += so_step;
                    if (ch >= nchunk) {
                        ch -= nchunk;
                        ub += ub_wrap;
                        so += so_wrap;
                    }
                }
            };
            // the common case (every chunk staged, no padding slots): the
            // chunk loop unrolled over its segments, with immediate offsets
            auto run_fast = [&](auto nsc_tag) __attribute__((always_inline)) {
                constexpr int NSC = decltype(nsc_tag)::value;
                int it = wave, ch = ch0;
                uint32_t ub = (uint32_t)qb0 * row_lds + (uint32_t)(ch0 * NSC) * seg_lds;
                uint32_t so = so0 + (uint32_t)qb0 * yrow_bytes + (uint32_t)(ch0 * NSC) * seg_y;
                unsigned char *sw = stg + st_w;
                while (it < nitems) {  // uniform
#pragma unroll
                    for (int s = 0; s < NSC; ++s) {
                        f32x4 acc[MS];
#pragma unroll
                        for (int r2 = 0; r2 < MS; ++r2) {
                            acc[r2] = binit;
#pragma unroll
                            for (int kb = 0; kb < KS; ++kb) {
                                const u32x4 av = *(const u32x4 *)(lds + rd[r2][kb] + ub + s * 256);
                                acc[r2] = GrpElem<E>::mfma(av, bw[r2][kb], acc[r2]);
                            }
                        }
                        uint32_t pk[2 * MS];
#pragma unroll
                        for (int e2 = 0; e2 < 2 * MS; ++e2) {
                            const int ea = 2 * e2, eb = 2 * e2 + 1;
                            pk[e2] = pack2(acc[ea % S2][ea / S2], acc[eb % S2][eb / S2]);
                        }
                        stage_run(pk, sw + s * 32 * S2);
                    }
                    // the wave's LDS accesses complete in order: the staged
                    // runs are read back after their writes, and the next
                    // chunk's writes follow these reads
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4 *)(stg + st_r[0]), ys, st_y[0], so, 0);
                    if (npass > 1)
                        __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4 *)(stg + st_r[1]), ys, st_y[1],
                                                               so, 0);
                    asm volatile("" ::: "memory");
                    it += 4;
                    ch += dc;
                    ub += ub_step;
                    so += so_step;
                    if (ch >= nchunk) {
                        ch -= nchunk;
                        ub += ub_wrap;
                        so += so_wrap;
                    }
                }
            };
            // segment pairs through DPP (width stride 2, at most 8 channels;
            // generic, so that only the instances that call it compile it)
            auto run_dpp = [&](auto) __attribute__((always_inline)) {
                // segment pairs: the second segment's runs move into lanes
                // 8..15 of each 16-lane row (the padding channels), then the
                // lanes are permuted so that one 16-byte store writes 8
                // channels x one whole 128-byte row, 8 lanes per row
                int it = wave, ch = ch0;
                uint32_t ub = (uint32_t)qb0 * row_lds + (uint32_t)(ch0 * 2) * seg_lds;
                uint32_t so = so0 + (uint32_t)qb0 * yrow_bytes + (uint32_t)(ch0 * 2) * seg_y;
                while (it < nitems) {  // uniform
                    u32x4 pr[2];
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        f32x4 acc[MS];
#pragma unroll
                        for (int r2 = 0; r2 < MS; ++r2) {
                            acc[r2] = binit;
#pragma unroll
                            for (int kb = 0; kb < KS; ++kb) {
                                const u32x4 av = *(const u32x4 *)(lds + rd[r2][kb] + ub + s * 256);
                                acc[r2] = GrpElem<E>::mfma(av, bw[r2][kb], acc[r2]);
                            }
                        }
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2)
                            pr[s][e2] = pack2(acc[(2 * e2) % 2][(2 * e2) / 2],
                                                    acc[(2 * e2 + 1) % 2][(2 * e2 + 1) / 2]);
                    }
                    // row_ror:8 (lane i of a row takes lane i - 8), written
                    // to lanes 8..15 of each row only (bank mask 0b1100)
                    u32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = __builtin_amdgcn_update_dpp((int)pr[0][e], (int)pr[1][e], 0x128, 0xf,
                                                                  0xc, false);
                        v[e] = (uint32_t)__builtin_amdgcn_ds_bpermute(bp_src, m);
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(v, ys, dpp_st, so, 0);
                    it += 4;
                    ch += dc;
                    ub += ub_step;
                    so += so_step;
                    if (ch >= nchunk) {
                        ch -= nchunk;
                        ub += ub_wrap;
                        so += so_wrap;
                    }
                }
            };
            if constexpr (PD) {
                run_dpp(0);
                continue;
            } else {
            if constexpr (MS == 2 && KS >= 1) {
                if (pair_dpp && regular && (st_align & kStageOk) && nfull == nseg) {  // uniform
                    run_dpp(0);
                    continue;
                }
            }
            if (regular && nstaged == nchunk && nsc == 1)
                run_fast(IntTag<1>{});
            else if (regular && nstaged == nchunk && nsc == 2)
                run_fast(IntTag<2>{});
            else if (regular && nstaged == nchunk && nsc == 4)
                run_fast(IntTag<4>{});
            else if (regular)
                run_items(BoolTag<false>{});
            else
                run_items(BoolTag<true>{});
            }
        }
    }
    };
    compute_rows(0, R);
}

static GrpArgs grp_args(const Plan &pl) {
    const DevParams &p = pl.dp;
    GrpArgs a;
    for (int i = 0; i < 3; ++i) a.ax[i] = GrpAxis{p.ax[i].I, p.ax[i].O, p.ax[i].S, p.ax[i].umin};
    a.G = p.G; a.Ci = p.Ci; a.Co = p.Co; a.Cig = p.Cig; a.Cog = p.Cog; a.has_bias = p.has_bias;
    a.x_plane = p.x_plane; a.y_plane = p.y_plane;
    a.th = p.th; a.tw = p.tw; a.hd = p.hd; a.hh = p.hh; a.hw = p.hw;
    a.grp_hwp = p.grp_hwp; a.grp_hshift = p.grp_hshift; a.grp_nk = p.grp_nk; a.grp_nsc = p.grp_nsc;
    a.grp_w_off = p.grp_w_off; a.grp_tab_off = p.grp_tab_off; a.grp_st_off = p.grp_st_off;
    a.grp_st_pitch = p.grp_st_pitch;
    a.grp_slab_off = p.grp_slab_off;
    a.grp_ns = p.grp_ns;
    a.ktot = p.ktot; a.nphase = p.nphase;
    a.tab_n = pl.gt.tab_n;
    a.w_sc = pl.gt.w_sc;
    a.w_so = pl.gt.w_so;
    a.w_tap_pieces = pl.gt.w_tap_pieces;
    memcpy(a.tab, pl.gt.tab, sizeof(a.tab));
    return a;
}

template <int S2, int KS, typename E>
static void launch_grouped_e(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                             int st_align, int x_vec, bool pd, hipStream_t stream) {
    const DevParams &p = pl.dp;
    const dim3 grid(p.G * p.B, p.nt_h, p.nt_d);
    const size_t lds = (size_t)p.grp_lds_bytes;
    const GrpArgs a = grp_args(pl);
    const uint16_t *xs = (const uint16_t *)x, *ws = (const uint16_t *)w,
                   *bs = (const uint16_t *)bias;
    uint16_t *ys = (uint16_t *)y;
    // one instance per activation: the activation folds into the unrolled
    // store loop (a run-time switch there splits it into branches the
    // compiler cannot schedule across, which cost even ReLU 70%)
#define CONVT_GRP_LAUNCH(A)                                                                           \
    do {                                                                                              \
        if constexpr (S2 == 2) {                                                                      \
            if (pd) {                                                                                 \
                hipLaunchKernelGGL((grouped_kernel<S2, KS, E, A, true>), grid, dim3(256), lds, stream, a, \
                                   xs, ws, bs, ys, st_align, x_vec);                                  \
                break;                                                                                \
            }                                                                                         \
        }                                                                                             \
        hipLaunchKernelGGL((grouped_kernel<S2, KS, E, A, false>), grid, dim3(256), lds, stream, a, xs, \
                           ws, bs, ys, st_align, x_vec);                                              \
    } while (0)
    switch (p.act) {
        case CONVT_ACT_RELU: CONVT_GRP_LAUNCH(CONVT_ACT_RELU); break;
        case CONVT_ACT_SIGMOID: CONVT_GRP_LAUNCH(CONVT_ACT_SIGMOID); break;
        case CONVT_ACT_TANH: CONVT_GRP_LAUNCH(CONVT_ACT_TANH); break;
        case CONVT_ACT_SILU: CONVT_GRP_LAUNCH(CONVT_ACT_SILU); break;
        case CONVT_ACT_GELU: CONVT_GRP_LAUNCH(CONVT_ACT_GELU); break;
        default: CONVT_GRP_LAUNCH(CONVT_ACT_NONE); break;
    }
#undef CONVT_GRP_LAUNCH
}

template <int S2, int KS>
static void launch_grouped_t(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                             int st_align, int x_vec, bool pd, hipStream_t stream) {
    if (pl.dp.f16)
        launch_grouped_e<S2, KS, _Float16>(pl, x, w, bias, y, st_align, x_vec, pd, stream);
    else
        launch_grouped_e<S2, KS, __bf16>(pl, x, w, bias, y, st_align, x_vec, pd, stream);
}

template <int S2>
static hipError_t launch_grouped_s(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                                   int st_align, int x_vec, bool pd, hipStream_t stream) {
    switch (pl.dp.grp_ksteps) {
        case 1: launch_grouped_t<S2, 1>(pl, x, w, bias, y, st_align, x_vec, pd, stream); break;
        case 2: launch_grouped_t<S2, 2>(pl, x, w, bias, y, st_align, x_vec, pd, stream); break;
        case 4: launch_grouped_t<S2, 4>(pl, x, w, bias, y, st_align, x_vec, pd, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipSuccess;
}

hipError_t launch_grouped(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                          hipStream_t stream) {
    const DevParams &p = pl.dp;
    if (p.n_blocks <= 0) return hipSuccess;
    // Widest store (bytes) that every output run starts aligned to: a run of
    // 4*S2 outputs starts at 8*S2*(q/4) bytes into a row; rows and channel
    // planes start at multiples of 2*O_w bytes from y.
    const int S2 = p.ax[2].S;
    int st_align = 2;
    for (int a = 16; a >= 4; a /= 2) {
        if ((uintptr_t)y % a == 0 && (2 * (int64_t)p.ax[2].O) % a == 0 && (8 * S2) % a == 0) {
            st_align = a;
            break;
        }
    }
    // staged chunks leave as 16-byte pieces of rows
    if ((uintptr_t)y % 16 == 0 && (2 * (int64_t)p.ax[2].O) % 16 == 0) st_align |= kStageOk;
    // chunked halo gather: x rows are whole 16-byte chunks (the plan then
    // gives the halo rows whole chunks of columns)
    const int x_vec = (uintptr_t)x % 16 == 0 && p.grp_nk > 0;
    if ((int64_t)p.G * p.B > 0x7fffffff || p.nt_h > 65535 || p.nt_d > 65535)
        return hipErrorInvalidConfiguration;
    // every item takes the segment-pair path (each phase's slots fill its K
    // steps and its q width covers every segment): the instance without the
    // other paths
    bool pd = S2 == 2 && p.grp_nsc == 0 && (st_align & kStageOk);
    const int nseg = (p.tw + 15) >> 4;
    for (int P = 0; pd && P < p.nphase; ++P)
        pd = (pl.gt.tab[4 * P + 3] >> 16) == 4 * p.grp_ksteps && (pl.gt.tab[4 * P + 2] >> 4) >= nseg;
    hipError_t e;
    switch (S2) {
        case 1: e = launch_grouped_s<1>(pl, x, w, bias, y, st_align, x_vec, pd, stream); break;
        case 2: e = launch_grouped_s<2>(pl, x, w, bias, y, st_align, x_vec, pd, stream); break;
        case 3: e = launch_grouped_s<3>(pl, x, w, bias, y, st_align, x_vec, pd, stream); break;
        case 4: e = launch_grouped_s<4>(pl, x, w, bias, y, st_align, x_vec, pd, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace convt
