// Grouped / few-channel stride-phase kernel (bfloat16, MFMA 16x16x32).
//
// For grouped problems with few channels per group (C_in/groups a multiple
// of 8 up to 64, C_out/groups up to 16) the phase GEMM's tiles would be
// mostly empty. Here one block owns one (batch, group) and a tile of q rows
// at one q-depth, over the full q width, for EVERY stride phase, so that the
// block's output rows are complete and leave as dense 16-byte stores: the
// huggingface ai.onnx.ConvTranspose page's grouped stride-phase blocked
// variant (an invocation owns output pixels and a block of its group's output
// channels; every gathered input sample feeds the whole channel block; the
// group's weight slab is staged once per workgroup), laid out for gfx950.
//
// Per block:
//  1. the input halo (the q tile grown by the union of all phases' input
//     windows) for the group's Cig channels goes to LDS with channels
//     contiguous, and the group's reordered weights [tap][16 co][Cig] too;
//  2. per phase, each wave keeps the phase's weight fragments in registers
//     and runs, for each of its 16-position segments of a q row, up to four
//     v_mfma_f32_16x16x32_bf16: rows = 16 positions, columns = the group's
//     output channels (padded to 16), K = (tap, 8-channel slice) slots, four
//     per MFMA. A lane reads its 8 channels of one tap as one 16-byte LDS row;
//  3. results + bias are rounded to bfloat16 into an LDS output tile
//     [co][depth residue][rows][O_w], interleaving the phases;
//  4. the tile is written to y row by row with 16-byte stores.
// The kernel's loops carry no per-lane integer division: positions advance
// by 16-wide segments of a row and the K-slot decode is done once per phase.
#include "kcommon.h"
#include "launch.h"

namespace convt {

constexpr int kGrpRsrcWord3 = 0x00020000;

constexpr uint32_t kGrpOutOfRange = 0x80000000u;

template <int S2, int KS>
__global__ __launch_bounds__(256) void grouped_kernel(DevParams p, const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ wr,
                                                      const uint16_t *__restrict__ bias,
                                                      uint16_t *__restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    uint16_t *xs = (uint16_t *)lds;
    uint16_t *wsl = (uint16_t *)(lds + p.grp_w_off);

    const int tid = threadIdx.x, lane = tid & 63;
    // uniform per wave: lets the plan tables be read with scalar loads
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bid = remap_block(blockIdx.x, p.n_blocks, p.xcd_remap);
    const int th_i = bid % p.nt_h;
    bid /= p.nt_h;
    const int qd = bid % p.nt_d;
    bid /= p.nt_d;
    const int g = bid % p.G;
    const int b = bid / p.G;

    const DevAxis &a0 = p.ax[0], &a1 = p.ax[1], &a2 = p.ax[2];
    const int Cig = p.Cig, noct = Cig >> 3;
    const int R = p.th, Qw = p.tw;
    const int HH = p.hh, HW = p.hw;
    const int q0h = th_i * R;
    const int h0 = qd + a0.umin, h1 = q0h + a1.umin, h2 = a2.umin;

    // 1a. input halo -> LDS [row][Cig]; positions outside the input read
    // an out-of-range offset (zero). A wave takes whole halo rows (one
    // 8-channel slice each); its lanes walk the row's positions.
    const uint32_t xpl_bytes = (uint32_t)p.x_plane * 2;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x + ((int64_t)b * p.Ci + (int64_t)g * Cig) * p.x_plane), (short)0,
        (int)((uint32_t)Cig * xpl_bytes), kGrpRsrcWord3);
    {
        // (slice, depth, row) triples are dealt to the waves in turn; a wave
        // issues the loads of four of its rows before writing any of them
        const int nrow = p.hd * HH, total = nrow * noct;
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
                        dst[u] = ((sc0 * HH + sc1) * HW + c2) * Cig + soct * 8;
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
                    if (dst[u] >= 0 && c2 < HW) *(u32x4 *)&xs[dst[u]] = v[u];
            }
        }
    }
    // 1b. the group's weights [tap][16][Cig] -> LDS
    {
        const int nvec = p.ktot * tiles::kGrpCog * noct;
        const u32x4 *src = (const u32x4 *)(wr + (int64_t)g * p.ktot * tiles::kGrpCog * Cig);
        for (int v = tid; v < nvec; v += 256) ((u32x4 *)wsl)[v] = src[v];
    }
    // 1c. K-slot table: for slot (tap, 8-channel slice) of every phase, the
    // halo element offset of the tap's window origin and the weight offset
    int2 *tab = (int2 *)(lds + p.grp_tab_off);
    for (int P = 0; P < p.nphase; ++P) {  // uniform
        const PhaseDesc ph = phase_desc(p, P);
        const int nslots = ph.ntaps * noct;
        const int n1 = ph.n[1], n2 = ph.n[2];
        for (int sl = tid; sl < nslots; sl += 256) {
            const int tap = sl / noct, oct = sl - tap * noct;
            const int j2 = tap % n2, j1 = (tap / n2) % n1, j0 = tap / (n2 * n1);
            const int dl = (((ph.off0[0] - a0.umin + j0 * a0.ostep) * HH +
                             (ph.off0[1] - a1.umin + j1 * a1.ostep)) * HW +
                            (ph.off0[2] - a2.umin + j2 * a2.ostep)) * Cig + oct * 8;
            tab[ph.tapbase * noct + sl] = make_int2(dl, (ph.tapbase + tap) * tiles::kGrpCog * Cig + oct * 8);
        }
    }
    __syncthreads();

    // 2. Per (depth residue, height residue) pair, each wave takes 16-position
    // segments of the block's q rows. For a segment it runs the MFMA chain of
    // every width residue r2 < S2 (kept in registers), so lane l (channel
    // l%16, positions 4*(l/16) + i of the segment) holds the outputs
    // ow = S2*q + r2 for four consecutive q and every r2: a contiguous run of
    // 4*S2 outputs, stored straight from registers.
    const int l16 = lane & 15, kg4 = lane >> 4;
    const int Cog = p.Cog;
    const int co = l16;
    const int O2 = a2.O;
    const int nseg = (Qw + 15) >> 4;
    const float bvf = (p.has_bias && co < Cog) ? bf16_to_f32(bias[g * Cog + co]) : 0.0f;
    // output plane of this lane's channel; rows past the group's channels are
    // outside the resource and dropped
    const uint32_t ypl_bytes = (uint32_t)p.y_plane * 2;
    const __amdgpu_buffer_rsrc_t ys = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(y + ((int64_t)b * p.Co + (int64_t)g * Cog) * p.y_plane), (short)0,
        (int)((uint32_t)Cog * ypl_bytes), kGrpRsrcWord3);
    const uint32_t co_bytes = co < Cog ? (uint32_t)co * ypl_bytes : kGrpOutOfRange;
    const bool row_pairs = (O2 & 1) == 0;  // outputs of a row start 4-byte aligned
    constexpr int MS = S2;  // width residues kept in registers
    for (int r0 = 0; r0 < a0.S; ++r0) {
        for (int r1 = 0; r1 < a1.S; ++r1) {
            // phases (r0, r1, r2 < S2): their records and this lane's K slots
            int qn0 = 0, qn1 = 0, qn2[MS], nkb[MS], dl[MS][KS];
            bf16x8 bw[MS][KS];
            bool sl_ok[MS][KS];
#pragma unroll
            for (int r2 = 0; r2 < MS; ++r2) {
                {
                    const PhaseDesc ph = phase_desc(p, (r0 * a1.S + r1) * S2 + r2);
                    qn0 = ph.qn[0];
                    qn1 = ph.qn[1];
                    qn2[r2] = ph.qn[2];
                    const int nslots = ph.ntaps * noct;
                    nkb[r2] = (nslots + 3) >> 2;
#pragma unroll
                    for (int kb = 0; kb < KS; ++kb) {
                        const int slot = kb * 4 + kg4;
                        sl_ok[r2][kb] = kb < nkb[r2] && slot < nslots;
                        int2 e = make_int2(0, 0);
                        u32x4 wv = {0u, 0u, 0u, 0u};
                        if (sl_ok[r2][kb]) {
                            e = tab[ph.tapbase * noct + slot];
                            wv = *(const u32x4 *)&wsl[e.y + l16 * Cig];
                        }
                        dl[r2][kb] = e.x;
                        bw[r2][kb] = __builtin_bit_cast(bf16x8, wv);
                    }
                }
            }
            if (qd >= qn0) continue;  // uniform: these phases have no output here
            const int od = a0.S * qd + r0;
            int mb = 0;
            for (int ql = 0; ql < R; ++ql) {
                const int qh = q0h + ql;
                if (qh >= qn1) break;  // uniform: rows past this residue's q range
                const uint32_t row_bytes = (uint32_t)(((int64_t)od * a1.O + a1.S * qh + r1) * O2 * 2);
                for (int seg = 0; seg < nseg; ++seg, ++mb) {
                    if ((mb & 3) != wave) continue;  // uniform
                    const int qw = seg * 16 + l16;
                    const int arow = (ql * HW + qw) * Cig;
                    f32x4 acc[MS];
#pragma unroll
                    for (int r2 = 0; r2 < MS; ++r2) {
                        acc[r2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                        {
#pragma unroll
                            for (int kb = 0; kb < KS; ++kb) {
                                if (kb < nkb[r2]) {
                                    u32x4 av = {0u, 0u, 0u, 0u};
                                    if (sl_ok[r2][kb] && qw < Qw)
                                        av = *(const u32x4 *)&xs[arow + dl[r2][kb]];
                                    acc[r2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                        __builtin_bit_cast(bf16x8, av), bw[r2][kb], acc[r2], 0, 0, 0);
                                }
                            }
                        }
                    }
                    // lane: positions q = qb + i (i < 4), outputs ow = S2*q + r2
                    const int qb = seg * 16 + 4 * kg4;
                    const uint32_t base = co_bytes + row_bytes + (uint32_t)(S2 * qb) * 2;
                    bool full = true;  // every output of the run inside the row
#pragma unroll
                    for (int r2 = 0; r2 < MS; ++r2)
                        full = full && (qb + 3 < qn2[r2]);
                    if (full && row_pairs) {
                        // 4*S2 consecutive outputs as 2*S2 dwords
#pragma unroll
                        for (int e2 = 0; e2 < 2 * MS; ++e2) {
                            {
                                const int ea = 2 * e2, eb = 2 * e2 + 1;  // output indices S2*i + r2
                                const float va = acc[ea % S2][ea / S2] + bvf;
                                const float vb = acc[eb % S2][eb / S2] + bvf;
                                const uint32_t pk = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)va) |
                                                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)vb) << 16);
                                __builtin_amdgcn_raw_buffer_store_b32(pk, ys, base + e2 * 4, 0, 0);
                            }
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int r2 = 0; r2 < MS; ++r2)
                                if (qb + i < qn2[r2])
                                    __builtin_amdgcn_raw_buffer_store_b16(
                                        __builtin_bit_cast(uint16_t, (__bf16)(acc[r2][i] + bvf)), ys,
                                        base + (S2 * i + r2) * 2, 0, 0);
                    }
                }
            }
        }
    }
}

template <int S2, int KS>
static void launch_grouped_t(const DevParams &p, const void *x, const void *wr, const void *bias,
                             void *y, hipStream_t stream) {
    hipLaunchKernelGGL((grouped_kernel<S2, KS>), dim3(p.n_blocks), dim3(256), (size_t)p.grp_lds_bytes,
                       stream, p, (const uint16_t *)x, (const uint16_t *)wr, (const uint16_t *)bias,
                       (uint16_t *)y);
}

template <int S2>
static hipError_t launch_grouped_s(const DevParams &p, const void *x, const void *wr,
                                   const void *bias, void *y, hipStream_t stream) {
    switch (p.grp_ksteps) {
        case 1: launch_grouped_t<S2, 1>(p, x, wr, bias, y, stream); break;
        case 2: launch_grouped_t<S2, 2>(p, x, wr, bias, y, stream); break;
        case 4: launch_grouped_t<S2, 4>(p, x, wr, bias, y, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipSuccess;
}

hipError_t launch_grouped(const Plan &pl, const void *x, const void *wr, const void *bias, void *y,
                          hipStream_t stream) {
    const DevParams &p = pl.dp;
    if (p.n_blocks <= 0) return hipSuccess;
    hipError_t e;
    switch (p.ax[2].S) {
        case 1: e = launch_grouped_s<1>(p, x, wr, bias, y, stream); break;
        case 2: e = launch_grouped_s<2>(p, x, wr, bias, y, stream); break;
        case 3: e = launch_grouped_s<3>(p, x, wr, bias, y, stream); break;
        case 4: e = launch_grouped_s<4>(p, x, wr, bias, y, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace convt
