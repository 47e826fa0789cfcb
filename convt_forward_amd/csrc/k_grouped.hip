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
//  2. for each (phase, 16 positions) pair a wave runs ceil(taps*Cig/32)
//     v_mfma_f32_16x16x32_bf16: rows = 16 positions, columns = the group's
//     output channels (padded to 16), K = (tap, 8-channel slice) slots, four
//     per MFMA. A lane reads its 8 channels of one tap as one 16-byte LDS row;
//  3. results + bias are rounded to bfloat16 into an LDS output tile
//     [co][depth residue][rows][O_w], interleaving the phases;
//  4. the tile is written to y row by row with 16-byte stores.
#include "kcommon.h"
#include "launch.h"

namespace convt {

__global__ __launch_bounds__(256) void grouped_kernel(DevParams p, const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ wr,
                                                      const uint16_t *__restrict__ bias,
                                                      uint16_t *__restrict__ y, int vec_store) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    uint16_t *xs = (uint16_t *)lds;
    uint16_t *wsl = (uint16_t *)(lds + p.grp_w_off);
    uint16_t *os = (uint16_t *)(lds + p.grp_out_off);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

    // 1a. input halo -> LDS [row][Cig]
    const int hrows = p.hd * HH * HW;
    const uint16_t *xg = x + ((int64_t)b * p.Ci + (int64_t)g * Cig) * p.x_plane;
    const int64_t xpl = p.x_plane;
    for (int it = tid; it < hrows * noct; it += 256) {
        const int oct = it / hrows, row = it - oct * hrows;
        const int c2 = row % HW, c1 = (row / HW) % HH, c0 = row / (HW * HH);
        const int i0 = h0 + c0, i1 = h1 + c1, i2 = h2 + c2;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (i0 >= 0 && i0 < a0.I && i1 >= 0 && i1 < a1.I && i2 >= 0 && i2 < a2.I) {
            const uint16_t *src = xg + (int64_t)(oct * 8) * xpl + ((i0 * a1.I + i1) * a2.I + i2);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = (uint32_t)src[(2 * e) * xpl] | ((uint32_t)src[(2 * e + 1) * xpl] << 16);
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

    // 2-3. MFMA per (phase, 16 positions); results into the output tile
    const int npos = R * Qw;
    const int nmb = (npos + 15) >> 4;
    const int npairs = p.nphase * nmb;
    const int l16 = lane & 15, kg4 = lane >> 4;
    const int Cog = p.Cog;
    const int orows = p.out_rows;
    const int O2 = a2.O;
    for (int pair = wave; pair < npairs; pair += 4) {
        const int P = pair / nmb, mb = pair - P * nmb;
        const PhaseDesc ph = phase_desc(p, P);
        const int m = mb * 16 + l16;
        const int qh_l = m / Qw, qw = m - qh_l * Qw;
        const int base = ((a0.off0[ph.r[0]] - a0.umin) * HH + (qh_l + a1.off0[ph.r[1]] - a1.umin)) * HW +
                         (qw + a2.off0[ph.r[2]] - a2.umin);
        const int nslots = ph.ntaps * noct;
        const int n1 = ph.n[1], n2 = ph.n[2];
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int kb = 0; kb < nslots; kb += 4) {
            const int slot = kb + kg4;
            u32x4 av = {0u, 0u, 0u, 0u}, bv = {0u, 0u, 0u, 0u};
            if (slot < nslots) {
                const int tap = slot / noct, oct = slot - tap * noct;
                const int j2 = tap % n2, j1 = (tap / n2) % n1, j0 = tap / (n2 * n1);
                if (m < npos) {
                    const int row = base + ((j0 * a0.ostep) * HH + j1 * a1.ostep) * HW + j2 * a2.ostep;
                    av = *(const u32x4 *)&xs[row * Cig + oct * 8];
                }
                bv = *(const u32x4 *)&wsl[((ph.tapbase + tap) * tiles::kGrpCog + l16) * Cig + oct * 8];
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
        }
        // D[m = 4*kg4 + i][n = l16]: position rows, channel columns
        const int co = l16;
        if (co < Cog && qd < a0.qn[ph.r[0]]) {
            const float bvf = p.has_bias ? bf16_to_f32(bias[g * Cog + co]) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mm = mb * 16 + 4 * kg4 + i;
                if (mm < npos) {
                    const int ql = mm / Qw, qw2 = mm - ql * Qw;
                    if (q0h + ql < a1.qn[ph.r[1]] && qw2 < a2.qn[ph.r[2]]) {
                        const int oh_l = a1.S * ql + ph.r[1], ow = a2.S * qw2 + ph.r[2];
                        os[((co * a0.S + ph.r[0]) * orows + oh_l) * O2 + ow] = f32_to_bf16(acc[i] + bvf);
                    }
                }
            }
        }
    }
    __syncthreads();

    // 4. dense rows out
    const int nrows = Cog * a0.S * orows;
    uint16_t *yb = y + ((int64_t)b * p.Co + (int64_t)g * Cog) * p.y_plane;
    if (vec_store) {
        const int vpr = O2 >> 3;
        for (int v = tid; v < nrows * vpr; v += 256) {
            const int row = v / vpr, c = v - row * vpr;
            const int oh_l = row % orows, r0 = (row / orows) % a0.S, co = row / (orows * a0.S);
            const int od = a0.S * qd + r0, oh = a1.S * q0h + oh_l;
            if (od < a0.O && oh < a1.O)
                *(u32x4 *)&yb[(int64_t)co * p.y_plane + ((int64_t)od * a1.O + oh) * O2 + c * 8] =
                    *(const u32x4 *)&os[row * O2 + c * 8];
        }
    } else {
        for (int e = tid; e < nrows * O2; e += 256) {
            const int row = e / O2, c = e - row * O2;
            const int oh_l = row % orows, r0 = (row / orows) % a0.S, co = row / (orows * a0.S);
            const int od = a0.S * qd + r0, oh = a1.S * q0h + oh_l;
            if (od < a0.O && oh < a1.O)
                yb[(int64_t)co * p.y_plane + ((int64_t)od * a1.O + oh) * O2 + c] = os[row * O2 + c];
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
