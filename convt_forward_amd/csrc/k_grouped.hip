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

__global__ __launch_bounds__(256) void grouped_kernel(DevParams p, const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ wr,
                                                      const uint16_t *__restrict__ bias,
                                                      uint16_t *__restrict__ y, int vec_store) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    uint16_t *xs = (uint16_t *)lds;
    uint16_t *wsl = (uint16_t *)(lds + p.grp_w_off);
    uint16_t *os = (uint16_t *)(lds + p.grp_out_off);

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
    // an out-of-range offset (zero)
    const int hrows = p.hd * HH * HW;
    const uint32_t xpl_bytes = (uint32_t)p.x_plane * 2;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x + ((int64_t)b * p.Ci + (int64_t)g * Cig) * p.x_plane), (short)0,
        (int)((uint32_t)Cig * xpl_bytes), kGrpRsrcWord3);
    for (int it = tid; it < hrows * noct; it += 256) {
        const int oct = it / hrows, row = it - oct * hrows;
        const int c2 = row % HW, c1 = (row / HW) % HH, c0 = row / (HW * HH);
        const int i0 = h0 + c0, i1 = h1 + c1, i2 = h2 + c2;
        const bool ok = i0 >= 0 && i0 < a0.I && i1 >= 0 && i1 < a1.I && i2 >= 0 && i2 < a2.I;
        const uint32_t off = ok ? (uint32_t)(oct * 8) * xpl_bytes +
                                      (uint32_t)((i0 * a1.I + i1) * a2.I + i2) * 2
                                : kGrpOutOfRange;
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(xrs, off + (2 * e) * xpl_bytes, 0, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(xrs, off + (2 * e + 1) * xpl_bytes, 0, 0);
            v[e] = lo | (hi << 16);
        }
        *(u32x4 *)&xs[row * Cig + oct * 8] = v;
    }
    // 1b. the group's weights [tap][16][Cig] -> LDS
    {
        const int nvec = p.ktot * tiles::kGrpCog * noct;
        const u32x4 *src = (const u32x4 *)(wr + (int64_t)g * p.ktot * tiles::kGrpCog * Cig);
        for (int v = tid; v < nvec; v += 256) ((u32x4 *)wsl)[v] = src[v];
    }
    __syncthreads();

    // 2-3. MFMA per (phase, 16-position row segment); results into the tile
    const int l16 = lane & 15, kg4 = lane >> 4;
    const int Cog = p.Cog;
    const int co = l16;
    const int orows = p.out_rows;
    const int O2 = a2.O;
    const int cstride = p.grp_out_cstride;
    const int nseg = (Qw + 15) >> 4;
    const int nmb = R * nseg;
    const float bvf = (p.has_bias && co < Cog) ? bf16_to_f32(bias[g * Cog + co]) : 0.0f;
    uint16_t *os_co = os + co * cstride;
    for (int P = 0; P < p.nphase; ++P) {
        const PhaseDesc ph = phase_desc(p, P);
        const int qn0 = a0.qn[ph.r[0]], qn1 = a1.qn[ph.r[1]], qn2 = a2.qn[ph.r[2]];
        if (qd >= qn0) continue;  // uniform: no output of this phase in this block
        const int nslots = ph.ntaps * noct;
        const int nkb = (nslots + 3) >> 2;  // <= kGrpMaxKSteps (planner)
        const int n1 = ph.n[1], n2 = ph.n[2];
        // this lane's K slot per MFMA step: halo row delta and channel slice,
        // plus the weight fragment (constant over the phase)
        int dl[tiles::kGrpMaxKSteps];
        bool sl_ok[tiles::kGrpMaxKSteps];
        bf16x8 bw[tiles::kGrpMaxKSteps];
#pragma unroll
        for (int kb = 0; kb < tiles::kGrpMaxKSteps; ++kb) {
            const int slot = kb * 4 + kg4;
            sl_ok[kb] = kb < nkb && slot < nslots;
            const int sl = sl_ok[kb] ? slot : 0;
            const int tap = sl / noct, oct = sl - tap * noct;
            const int j2 = tap % n2, j1 = (tap / n2) % n1, j0 = tap / (n2 * n1);
            dl[kb] = (((a0.off0[ph.r[0]] - a0.umin + j0 * a0.ostep) * HH +
                       (a1.off0[ph.r[1]] - a1.umin + j1 * a1.ostep)) * HW +
                      (a2.off0[ph.r[2]] - a2.umin + j2 * a2.ostep)) * Cig + oct * 8;
            const u32x4 wv = *(const u32x4 *)&wsl[((ph.tapbase + tap) * tiles::kGrpCog + l16) * Cig + oct * 8];
            bw[kb] = __builtin_bit_cast(bf16x8, sl_ok[kb] ? wv : u32x4{0u, 0u, 0u, 0u});
        }
        uint16_t *os_ph = os_co + ph.r[0] * orows * O2 + ph.r[1] * O2 + ph.r[2];
        for (int mb = wave; mb < nmb; mb += 4) {
            const int ql = mb / nseg, seg = mb - ql * nseg;  // uniform
            if (q0h + ql >= qn1) continue;                   // uniform
            const int qw = seg * 16 + l16;
            const int arow = (ql * HW + qw) * Cig;
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < tiles::kGrpMaxKSteps; ++kb) {
                if (kb < nkb) {
                    u32x4 av = {0u, 0u, 0u, 0u};
                    if (sl_ok[kb] && qw < Qw) av = *(const u32x4 *)&xs[arow + dl[kb]];
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                                  bw[kb], acc, 0, 0, 0);
                }
            }
            // D[m = 4*kg4 + i][n = l16]: positions qw0 + i of row ql, channel co
            if (co < Cog) {
                const int qw0 = seg * 16 + 4 * kg4;
                uint16_t *dst = os_ph + a1.S * ql * O2 + a2.S * qw0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (qw0 + i < qn2) dst[a2.S * i] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i] + bvf));
            }
        }
    }
    __syncthreads();

    // 4. dense rows out
    const int rows_co = a0.S * orows;
    const int nrows = Cog * rows_co;
    uint16_t *yb = y + ((int64_t)b * p.Co + (int64_t)g * Cog) * p.y_plane;
    if (vec_store) {
        const int vpr = O2 >> 3;
        for (int v = tid; v < nrows * vpr; v += 256) {
            const int row = v / vpr, c = v - row * vpr;
            const int cc = row / rows_co, rr = row - cc * rows_co;
            const int r0 = rr / orows, oh_l = rr - r0 * orows;
            const int od = a0.S * qd + r0, oh = a1.S * q0h + oh_l;
            if (od < a0.O && oh < a1.O)
                *(u32x4 *)&yb[(int64_t)cc * p.y_plane + ((int64_t)od * a1.O + oh) * O2 + c * 8] =
                    *(const u32x4 *)&os[cc * cstride + rr * O2 + c * 8];
        }
    } else {
        for (int e = tid; e < nrows * O2; e += 256) {
            const int row = e / O2, c = e - row * O2;
            const int cc = row / rows_co, rr = row - cc * rows_co;
            const int r0 = rr / orows, oh_l = rr - r0 * orows;
            const int od = a0.S * qd + r0, oh = a1.S * q0h + oh_l;
            if (od < a0.O && oh < a1.O)
                yb[(int64_t)cc * p.y_plane + ((int64_t)od * a1.O + oh) * O2 + c] =
                    os[cc * cstride + rr * O2 + c];
        }
    }
}

hipError_t launch_grouped(const Plan &pl, const void *x, const void *wr, const void *bias, void *y,
                          hipStream_t stream) {
    const DevParams &p = pl.dp;
    if (p.n_blocks <= 0) return hipSuccess;
    const int vec = (p.ax[2].O % 8 == 0 && ((uintptr_t)y % 16) == 0) ? 1 : 0;
    hipLaunchKernelGGL(grouped_kernel, dim3(p.n_blocks), dim3(256), (size_t)p.grp_lds_bytes, stream,
                       p, (const uint16_t *)x, (const uint16_t *)wr, (const uint16_t *)bias,
                       (uint16_t *)y, vec);
    return hipGetLastError();
}

}  // namespace convt
