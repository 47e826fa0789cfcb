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
// Block: 256 threads (4 waves as WGM x 4/WGM, one per SIMD), BM output
// channels x BN positions of one phase; its LDS stays within 160 KiB / occ
// (the configuration's blocks per CU; 80 KiB for two), so two
// blocks share each CU and one block's barrier and LDS waits overlap the
// other's MFMAs. The BN positions form a
// (td, th, tw) box in q space. K runs over chunks of 32 bytes of input
// channels (16 bfloat16 / 8 float32) and, within a chunk, over groups of up
// to four taps; one (chunk, tap group) pair is a pipeline stage.
//
// All operands move global -> LDS by buffer loads with an LDS destination
// (lane l of a wave instruction writes its element at the destination base +
// l * element slot), so no registers stage them and the only waits are the
// explicit vector-memory counts before each barrier.
//
// Halo: for each chunk the block stages the box's input halo (the box grown
// by the phase's tap span) in LDS, one row per channel of 4-byte slots over
// the box positions (a bfloat16 load fills the low half of its slot), and
// reuses it for every tap (tap t reads the positions shifted by its offset).
// A wave instruction copies 64 consecutive box positions of one channel, each
// lane gathering its own position of the channel-planar input. The halo of a
// chunk is requested one or two chunks ahead through a ring of two or three
// buffers (a tile configuration's choice: two leave room for larger halos).
//
// Weights: the reordered weights hold, per (tap, chunk), the [co][32 bytes]
// tile contiguously, its two 16-byte halves swapped on rows with bit 3 of co
// set (an XOR swizzle that spreads a wave's A-operand reads over all LDS
// banks). Each stage's tiles are copied 1 KiB per wave instruction, two
// stages ahead, through a ring of three buffers.
//
// Loads go through raw buffer resources, whose range check returns zero for
// reads past the resource's size: each input channel is read through a
// resource covering its plane (empty for channels past the group's last, so
// a ragged channel chunk reads zeros), and positions outside the input use an
// offset of 2^31, always out of range. Every per-lane offset is a 32-bit
// byte offset.
//
// MFMA: two-byte inputs use v_mfma_f32_32x32x16_bf16 or _f16 (each lane
// supplies 8 consecutive channels of one row of each operand, one 16-byte
// LDS read each), float32 inputs use
// v_mfma_f32_32x32x2_f32 (each lane reads 4 consecutive channels of its
// weight row and feeds them to 4 MFMAs, with the input of the same channel;
// A and B pair the same channel in every lane, so the sum is the full
// reduction). Operand A is the weight tile (rows = co), operand B the
// gathered inputs (columns = positions). Within a stage, the operands of tap
// u+1 are read from LDS while the MFMAs of tap u run.
//
// Epilogue: acc + bias[co] in float32, the activation if the plan has one,
// one rounding to the output type (nearest even), stored to
// y[b][g*Cog+co][s*q + r]; outputs beyond the phase's q range or past Cog
// fall outside the store resource and are dropped.
//
// Backward data (BWD): dx[i] gathers dy[s*i - p + kk*d] * W[kk]; the taps of
// forward output residue r read the dy phase plane dy_r[j] = dy[s*j + r] at
// j = i - off(kk), so dx is the sum over phases of stride-1 correlations.
// The same kernel runs it with the roles swapped (rows = input channels, K =
// output channels x taps, columns = dx positions): a block owns a box of dx
// positions and runs every phase's taps in one K loop, in units of (channel
// chunk, phase) whose halo is the box in that phase plane (gathered at
// stride s from dy, or from its channel-chunked copy), stored densely.
#include <type_traits>

#include "kcommon.h"
#include "launch.h"

namespace convt {

template <typename T, int CFG, int GS, bool BWD, bool ACT>
__global__ __launch_bounds__(tiles::kGemmCfg[CFG].nw * 64) __attribute__((amdgpu_waves_per_eu(
    tiles::kGemmCfg[CFG].occ * tiles::kGemmCfg[CFG].nw / 4, tiles::kGemmCfg[CFG].occ * tiles::kGemmCfg[CFG].nw / 4))) void phase_gemm_kernel(DevParams p, const T *__restrict__ x,
                                                         const T *__restrict__ wr,
                                                         const int32_t *__restrict__ tab,
                                                         const T *__restrict__ bias,
                                                         T *__restrict__ y) {
    constexpr tiles::GemmTile CT = tiles::kGemmCfg[CFG];
    static_assert((CT.bf16 != 0) == (sizeof(T) == 2), "tile config does not match the element type");
    static_assert(GS >= 1 && GS <= tiles::kGemmTapGroup, "taps per stage");
    constexpr int BM = CT.bm, BN = CT.bn, WGM = CT.wgm, SC = CT.sc;
    constexpr int ES = (int)sizeof(T);
    constexpr int BK = tiles::gemm_chunk_ch(CT);          // channels per chunk (32 bytes)
    constexpr int BKS = SC * BK;                          // channels per stage (chunk group)
    constexpr int HALO = tiles::gemm_halo_cap(CT, GS);    // halo positions per chunk buffer
    constexpr int XROW = tiles::gemm_xrow_bytes(CT, GS);  // float32 halo: one channel row, bytes
    constexpr int XSUB = tiles::gemm_xsub_bytes(CT, GS);  // one chunk's halo buffer
    constexpr int XBUF = SC * XSUB;                       // one ring slot: a chunk group's halos
    constexpr int XB = CT.xb;  // halo ring slots
    constexpr int WROW = tiles::kGemmWRowBytes;           // weight row bytes
    constexpr int NW = CT.nw, WGN = NW / WGM;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int MT = WM / 32, NT = WN / 32;
    constexpr int WSLOT = BM * WROW;                      // bytes of one (chunk, tap) weight tile
    constexpr int NV = SC * GS;                           // (chunk, tap) pairs of a stage
    constexpr int WBUF = NV * WSLOT;                      // bytes of one stage's weight tiles
    constexpr int NPIECE = WBUF / 1024;                   // 1 KiB weight copies per stage
    constexpr int NDMA = (NPIECE + NW - 1) / NW;          // per wave, at most
    // halo copies per wave and chunk, at most: bfloat16 in 1 KiB pieces of 32
    // rows dealt over the waves; float32 XCH channels per wave, each in
    // pieces of 64 positions
    constexpr int XCH = ES == 2 ? 1 : BK / NW;
    constexpr int XJ = ES == 2 ? (HALO / 32 + NW - 1) / NW : HALO / 64;
    static_assert(tiles::gemm_cfg_valid(CT, GS), "configuration invalid for this tap count");
    static_assert(MT >= 1 && NT >= 1 && WM * WGM == BM && WN * WGN == BN, "wave tiling");
    static_assert(NPIECE * 1024 == WBUF && WSLOT % 1024 == 0, "weight tiles are whole KiB");
    static_assert(BK * ES == WROW && (ES == 2 || XCH * NW == BK), "chunk split");
    static_assert(ES == 2 ? HALO % 32 == 0 && XSUB == HALO / 32 * 1024
                          : HALO % 64 == 0 && XJ * 256 <= XROW,
                  "halo buffers hold whole pieces");
    static_assert(tiles::kGemmWRing * WBUF + XB * XBUF <= tiles::gemm_lds_budget(CT), "LDS budget");

    __shared__ __attribute__((aligned(1024))) unsigned char ws[tiles::kGemmWRing][WBUF];
    __shared__ __attribute__((aligned(256))) unsigned char xs[XB][XBUF];

    // LDS byte addresses of the buffers, for the copy instructions
    const uint32_t ws_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)&ws[0][0];
    const uint32_t xs_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)&xs[0][0];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int wm = wave / WGN, wn = wave % WGN;

    int bid = remap_block(blockIdx.x, p.n_blocks, p.xcd_remap);
    const int co_t = bid % p.n_co_tiles;
    bid /= p.n_co_tiles;
    // backward data: every block runs all phases (no phase in the grid)
    int P = 0;
    if constexpr (!BWD) {
        P = bid % p.nphase;
        bid /= p.nphase;
    }
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
    // phase's smallest input offset. Backward data: dx position i reads the
    // phase plane at i - off for the phase's offsets off, so phase P's box
    // starts at q - (its largest offset); every phase's box gets the extents
    // of the widest tap span (span_max), so one layout serves all phases.
    const int E0 = BWD ? T0 + a0.span_max : T0 + (ph.n[0] > 0 ? (ph.n[0] - 1) * a0.ostep : 0);
    const int E1 = BWD ? T1 + a1.span_max : T1 + (ph.n[1] > 0 ? (ph.n[1] - 1) * a1.ostep : 0);
    const int E2 = BWD ? T2 + a2.span_max : T2 + (ph.n[2] > 0 ? (ph.n[2] - 1) * a2.ostep : 0);
    const int hsz = E0 * E1 * E2;
    const int h00 = q00 + ph.off0[0];  // forward only; the backward box is set per phase
    const int h01 = q01 + ph.off0[1];
    const int h02 = q02 + ph.off0[2];

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.0f;

    const int ntaps = BWD ? p.bwd_nstages : ph.ntaps;
    const int nchunks = p.cig_pad / BKS;  // chunk groups (one per stage and tap group)
    const int Cig = p.Cig;
    const uint32_t xpl_bytes = (uint32_t)p.x_plane * ES;

    if (ntaps > 0) {
        // ---- halo copies ----
        // bfloat16: x here is the channel-chunked copy [b][g][chunk][pos][32 B];
        // a chunk's halo is hsz rows of 32 bytes, copied in 1 KiB pieces of 32
        // rows, piece q by wave q % 8; lane l takes row q*32 + l/2, 16-byte
        // half l&1, which holds the row's logical half (l&1) ^ (bit 3 of the
        // row) (the rows' XOR swizzle, undone by the operand reads).
        // float32: wave w copies channel w of the chunk from x itself, in
        // pieces of 64 consecutive box positions, lane l taking position
        // 64j + l.
        // xsp[j]: this lane's byte offset for its piece j, out of range
        // outside the input. Forward: the box starts at input position (b0,
        // b1, b2). Backward data: the box is in the phase plane
        // dy_r[j] = dy[s*j + r] of the phase with residues r (set before each
        // halo copy), read from dy itself (its channel-chunked copy for
        // bfloat16) at stride s.
        const int xpieces = ES == 2 ? (hsz + 31) / 32 : (hsz + 63) / 64;
        const int nxw = ES == 2 ? (xpieces - wave + NW - 1) / NW : xpieces;  // pieces of this wave
        uint32_t xsp[XJ];
        auto halo_offsets = [&](int b0, int b1, int b2) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < XJ; ++j) {
                const int row = ES == 2 ? (j * NW + wave) * 32 + (lane >> 1) : j * 64 + lane;
                const int c2 = row % E2, c1 = (row / E2) % E1, c0 = row / (E2 * E1);
                const int i0 = b0 + c0, i1 = b1 + c1, i2 = b2 + c2;
                const uint32_t pos = (uint32_t)((i0 * a1.I + i1) * a2.I + i2);
                const uint32_t off = ES == 2 ? pos * 32 + (uint32_t)(((lane & 1) ^ ((row >> 3) & 1)) * 16)
                                             : pos * 4;
                xsp[j] = (row < hsz && i0 >= 0 && i0 < a0.I && i1 >= 0 && i1 < a1.I && i2 >= 0 &&
                          i2 < a2.I)
                             ? off
                             : kOutOfRange;
            }
        };
        if constexpr (!BWD) halo_offsets(h00, h01, h02);
        // Backward data: the box coordinates of this lane's rows, packed as
        // c2 | c1 << 11 | c0 << 22 (all-ones past the box), and their byte
        // offsets relative to the box origin at stride s, computed once; a
        // phase then needs per-axis bounds on c and one add (halo_phase).
        uint32_t hcode[BWD ? XJ : 1], hrel[BWD ? XJ : 1];
        if constexpr (BWD) {
#pragma unroll
            for (int j = 0; j < XJ; ++j) {
                const int row = ES == 2 ? (j * NW + wave) * 32 + (lane >> 1) : j * 64 + lane;
                const int c2 = row % E2, c1 = (row / E2) % E1, c0 = row / (E2 * E1);
                hcode[j] = row < hsz ? (uint32_t)c2 | (uint32_t)c1 << 11 | (uint32_t)c0 << 22 : ~0u;
                const uint32_t rel = (uint32_t)((c0 * a0.S * a1.I + c1 * a1.S) * a2.I + c2 * a2.S);
                hrel[j] = ES == 2 ? rel * 32 + (uint32_t)(((lane & 1) ^ ((row >> 3) & 1)) * 16) : rel * 4;
            }
        }
        // box starting at phase-plane position b of the phase with residues
        // r and q counts qn: phase-plane position b + c holds dy[(b + c)*s + r]
        // for 0 <= b + c < qn, i.e. c in [max(0, -b), qn - 1 - b] per axis
        auto halo_phase = [&](int b0, int b1, int b2, int r0, int r1, int r2, int n0, int n1,
                              int n2) __attribute__((always_inline)) {
            const int e0 = b0 * a0.S + r0, e1 = b1 * a1.S + r1, e2 = b2 * a2.S + r2;
            const int lo0 = b0 < 0 ? -b0 : 0, lo1 = b1 < 0 ? -b1 : 0, lo2 = b2 < 0 ? -b2 : 0;
            const int hi0 = n0 - 1 - b0, hi1 = n1 - 1 - b1, hi2 = n2 - 1 - b2;
            const int kb = ((e0 * a1.I + e1) * a2.I + e2) * (ES == 2 ? 32 : 4);
#pragma unroll
            for (int j = 0; j < XJ; ++j) {
                const int c2 = (int)(hcode[j] & 0x7ffu), c1 = (int)((hcode[j] >> 11) & 0x7ffu),
                          c0 = (int)(hcode[j] >> 22);
                const bool ok = c0 >= lo0 && c0 <= hi0 && c1 >= lo1 && c1 <= hi1 && c2 >= lo2 &&
                                c2 <= hi2;
                xsp[j] = ok ? hrel[j] + (uint32_t)kb : kOutOfRange;
            }
        };
        // halos of the chunks of group cg into ring slot xbi
        auto load_x = [&](int xbi, int cg) __attribute__((always_inline)) {
#pragma unroll
            for (int sc = 0; sc < SC; ++sc) {
                const int c = cg * SC + sc;  // chunk
                const uint32_t sub = xs_lds + (uint32_t)(xbi * XBUF + sc * XSUB);
                if constexpr (ES == 2) {
                    const T *src =
                        x + (((int64_t)b * p.G + g) * (p.cig_pad / 16) + c) * p.x_plane * 16;
                    const u32x4 rs = rsrc_words(src, xpl_bytes * 16);
#pragma unroll
                    for (int j = 0; j < XJ; ++j)
                        if (j < nxw) copy_to_lds<16>(sub + (uint32_t)((j * NW + wave) * 1024), xsp[j], rs);
                } else {
#pragma unroll
                    for (int h = 0; h < XCH; ++h) {
                        const int ch = wave * XCH + h;  // channel within the chunk
                        const int ci = c * BK + ch;     // channel within the group
                        const T *src = x + ((int64_t)b * p.Ci + (int64_t)g * Cig + ci) * p.x_plane;
                        const u32x4 rs = rsrc_words(src, ci < Cig ? xpl_bytes : 0u);
                        const uint32_t dst = sub + (uint32_t)(ch * XROW);
#pragma unroll
                        for (int j = 0; j < XJ; ++j)
                            if (j < nxw) copy_to_lds<4>(dst + j * 256, xsp[j], rs);
                    }
                }
            }
        };

        // ---- weight tiles: per stage NV = SC * GS slots of [BM][32 bytes],
        // slot sc * GS + u holding chunk sc of the group and tap u; wave w
        // copies the 1 KiB pieces j*4 + w (piece q: slot q / (BM/32), rows
        // (q % (BM/32))*32 ... +32), lane l taking 16 bytes at 16*l ----
        const uint32_t tap_bytes = (uint32_t)p.cog_pad * p.cig_pad * ES;
        const uint32_t chunk_bytes = (uint32_t)p.cog_pad * WROW;
        const int ngrp = (ntaps + GS - 1) / GS;  // tap groups; the phase is padded with zero taps
        // backward data: the resource spans the group's taps of every phase
        const u32x4 wrs =
            BWD ? rsrc_words(wr + (int64_t)g * p.ktot_pad * p.cog_pad * p.cig_pad,
                             (uint32_t)p.ktot_pad * tap_bytes)
                : rsrc_words(wr + (int64_t)(g * p.ktot_pad + ph.tapbase) * p.cog_pad * p.cig_pad,
                             (uint32_t)(ngrp * GS) * tap_bytes);
        const int ndma = (NPIECE - wave + NW - 1) / NW;  // pieces of this wave (uniform)
        uint32_t wv[NDMA];
#pragma unroll
        for (int j = 0; j < NDMA; ++j) {
            const int q = j * NW + wave, slot = q / (BM / 32), rb = q % (BM / 32);
            const int sc = slot / GS, u = slot % GS;
            wv[j] = (uint32_t)u * tap_bytes + (uint32_t)sc * chunk_bytes +
                    (uint32_t)(co_t * BM + rb * 32) * WROW + (uint32_t)lane * 16;
        }
        // weight tiles of tap group gi of chunk group cg into buffer wbi (tb:
        // the phase's first tap, backward data only)
        auto load_w = [&](int wbi, int gi, int cg, int tb) __attribute__((always_inline)) {
            const uint32_t base =
                (uint32_t)(tb + gi * GS) * tap_bytes + (uint32_t)(cg * SC) * chunk_bytes;
#pragma unroll
            for (int j = 0; j < NDMA; ++j)
                if (j < ndma)
                    copy_to_lds<16>(ws_lds + (uint32_t)(wbi * WBUF + (j * NW + wave) * 1024), wv[j] + base, wrs);
        };

        // ---- operand addresses of this lane ----
        // A: row m of the slot, 16-byte half kv = lane/32, stored at half
        // kv ^ (bit 3 of m); 8 (bf16) or 4 (f32) channels
        const int am = wm * WM + (lane & 31);
        const int aoff = am * WROW + (((lane >> 5) ^ ((am >> 3) & 1)) * 16);
        // B: the lane's halo row (position) for each 32-position tile
        int brow[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n = wn * WN + nt * 32 + (lane & 31);
            const int c2 = n % T2, c1 = (n / T2) % T1, c0 = n / (T2 * T1);
            brow[nt] = (c0 * E1 + c1) * E2 + c2;
        }
        const int kvl = lane >> 5;
        // halo shifts of the phase's taps (the zero taps that pad it to whole
        // groups shift by 0)
        const int32_t *ptab = tab + (BWD ? 0 : ph.tapbase);

        using Frag = typename std::conditional<
            ES == 2, typename std::conditional<std::is_same<T, _Float16>::value, f16x8, bf16x8>::type,
            f32x4>::type;
        // operands of one tap: weight slot wsl, halo rows shifted by drow
        auto read_frags = [&](Frag (&fa)[MT], Frag (&fb)[NT], const unsigned char *wsl,
                              const unsigned char *xsl, int drow) __attribute__((always_inline)) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                fa[mt] = __builtin_bit_cast(Frag, *(const u32x4 *)(wsl + aoff + mt * 32 * WROW));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int r = brow[nt] + drow;
                if constexpr (ES == 2) {
                    // 8 channels kv*8..: 16-byte half kv of row r, swizzled
                    fb[nt] = __builtin_bit_cast(
                        Frag, *(const u32x4 *)(xsl + r * 32 + ((kvl ^ ((r >> 3) & 1)) << 4)));
                } else {
                    // channels kv*4 + e, one row per channel
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        fb[nt][e] = *(const float *)(xsl + (kvl * 4 + e) * XROW + r * 4);
                }
            }
        };
        auto mfma = [&](const Frag (&fa)[MT], const Frag (&fb)[NT]) __attribute__((always_inline)) {
            if constexpr (std::is_same<T, _Float16>::value) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[mt], fb[nt],
                                                                             acc[mt][nt], 0, 0, 0);
            } else if constexpr (ES == 2) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mt], fb[nt],
                                                                              acc[mt][nt], 0, 0, 0);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[mt][i], fb[nt][i],
                                                                              acc[mt][nt], 0, 0, 0);
            }
        };

        // ---- pipeline ----
        // Stage s = chunk * ngrp + gi computes tap group gi of chunk group
        // `chunk` from weight buffer s % 3 and halo slot chunk % XB. At its
        // start it requests the halos of group chunk + XB - 1 (first tap
        // group only), then the weights of stage s + 2; at its end it waits
        // for what stage s + 1 reads and joins the barrier.
        // Backward data: the halo unit is (chunk group, phase), phases inner
        // and those without taps skipped, each unit with its phase's tap
        // groups as stages and a halo slot of its own (the phase plane's
        // box); halo copies run XB - 1 units ahead through a unit cursor.
        const int nstages = BWD ? p.bwd_nstages : nchunks * ngrp;
        const int nx = SC * XCH * nxw;  // halo copies of one chunk group by this wave
        // backward data: the phases with taps, in order (p.bwd_live), by index k
        auto live_after = [&](int k) __attribute__((always_inline)) {
            return k + 1 < p.bwd_nlive ? k + 1 : -1;
        };
        auto phase_of = [&](int k) __attribute__((always_inline)) {
            return BWD ? (int)p.bwd_live[k] : P;
        };
        auto groups_of = [&](int k) __attribute__((always_inline)) {
            return BWD ? (p.ph[phase_of(k)].ntaps + GS - 1) / GS : ngrp;
        };
        auto tapbase_of = [&](int k) __attribute__((always_inline)) {
            return BWD ? p.ph[phase_of(k)].tapbase : 0;
        };
        const int first = 0;
        auto next_unit = [&](int &c, int &q) __attribute__((always_inline)) {
            ++c;
            if constexpr (BWD) {
                q = live_after(q);
                if (q < 0)
                    q = first;
                else
                    --c;
            }
        };
        auto next_stage = [&](int &c, int &q, int &gi) __attribute__((always_inline)) {
            if (++gi == groups_of(q)) {
                gi = 0;
                next_unit(c, q);
            }
        };
        // backward data: halo copy of the unit at the cursor (cx, qx)
        int cx = 0, qx = first;
        auto issue_x = [&](int xbi) __attribute__((always_inline)) {
            // the box starts at q - (the phase's largest offset per axis: first
            // offset + (taps - 1) * ostep)
            const PhaseDesc d = phase_desc(p, phase_of(qx));
            halo_phase(q00 - d.off0[0] - (d.n[0] - 1) * a0.ostep,
                       q01 - d.off0[1] - (d.n[1] - 1) * a1.ostep,
                       q02 - d.off0[2] - (d.n[2] - 1) * a2.ostep, d.r[0], d.r[1], d.r[2], d.qn[0],
                       d.qn[1], d.qn[2]);
            load_x(xbi, cx);
            next_unit(cx, qx);
        };
        int chunk = 0, gi = 0, qc = first;  // of stage s
        int c2n = 0, gi2 = 0, q2 = first;   // of stage s + 2
        // Prologue: what stage 0 reads (the first halo, the first weights)
        // is requested before what later stages read, so that stage 0 waits
        // for its own copies only (loads complete in issue order).
        if constexpr (BWD)
            issue_x(0);
        else
            load_x(0, 0);
        load_w(0, 0, 0, tapbase_of(q2));
        next_stage(c2n, q2, gi2);
        bool x1 = false;
        if constexpr (BWD) {
            if (XB == 3 && cx < nchunks) {
                issue_x(1);
                x1 = true;
            }
        } else if (XB == 3 && nchunks > 1) {
            load_x(1, 1);
            x1 = true;
        }
        const bool w1 = nstages > 1;
        if (w1) load_w(1, gi2, c2n, tapbase_of(q2));
        next_stage(c2n, q2, gi2);
        // halo shifts of the first stage's taps
        int dl[GS];
#pragma unroll
        for (int u = 0; u < GS; ++u) dl[u] = ptab[tapbase_of(qc) + u];
        {
            const int fly0 = (x1 ? nx : 0) + (w1 ? ndma : 0);
            if (fly0 == 0)
                stage_barrier<0>();
            else
                stage_barrier_n<NDMA + SC * XCH * XJ>(fly0);
        }
        int wb = 0, xb = 0;  // buffers of stage s: s % 3, its unit % XB
        for (int s = 0; s < nstages; ++s) {
            const unsigned char *wsb = ws[wb];
            const unsigned char *xsb = xs[xb];
            // (chunk, tap) pair v = sc * GS + u: weight slot v, the halo of
            // chunk sc shifted by dl[u]. The operands of the first pair are
            // requested first; then this stage's copies; then, pair by pair,
            // the operands of v + 1 before the MFMAs of v. The scheduling
            // barriers keep the compiler from reordering these groups.
            Frag fa[2][MT], fb[2][NT];
            read_frags(fa[0], fb[0], wsb, xsb, dl[0]);
            __builtin_amdgcn_sched_barrier(0);
            const bool x_issue = gi == 0 && (BWD ? cx < nchunks : chunk + XB - 1 < nchunks);
            if (x_issue) {
                const int xbi = xb == 0 ? XB - 1 : xb - 1;
                if constexpr (BWD)
                    issue_x(xbi);
                else
                    load_x(xbi, chunk + XB - 1);
            }
            const bool w_issue = s + 2 < nstages;
            if (w_issue) load_w(wb == 0 ? 2 : wb - 1, gi2, c2n, tapbase_of(q2));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                if (v + 1 < NV)
                    read_frags(fa[(v + 1) & 1], fb[(v + 1) & 1], wsb + (v + 1) * WSLOT,
                               xsb + ((v + 1) / GS) * XSUB, dl[(v + 1) % GS]);
                __builtin_amdgcn_sched_barrier(0);
                mfma(fa[v & 1], fb[v & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // the next stage's halo shifts, fetched before the barrier
            {
                int cn = chunk, qn = qc, gin = gi;
                next_stage(cn, qn, gin);
#pragma unroll
                for (int u = 0; u < GS; ++u) dl[u] = ptab[tapbase_of(qn) + gin * GS + u];
            }
            if (s + 1 < nstages) {
                // the weights of stage s + 2 may still fly, and with three
                // halo slots the halos requested now; everything older (all
                // that stage s + 1 reads) must have landed. (With two slots
                // the halo requested now, before the weights, is awaited.)
                const int fly = (XB == 3 && x_issue ? nx : 0) + (w_issue ? ndma : 0);
                if (fly == 0)
                    stage_barrier<0>();
                else
                    stage_barrier_n<NDMA + SC * XCH * XJ>(fly);
            }
            wb = wb == 2 ? 0 : wb + 1;
            next_stage(chunk, qc, gi);
            if (gi == 0) xb = xb == XB - 1 ? 0 : xb + 1;
            if (w_issue) next_stage(c2n, q2, gi2);
        }
    }

    // ---- epilogue: bias, one rounding, strided stores ----
    // per position: byte offset in the output plane, out of range if masked
    uint32_t yoff[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = wn * WN + nt * 32 + (lane & 31);
        const int c2 = n % T2, c1 = (n / T2) % T1, c0 = n / (T2 * T1);
        const int qd = q00 + c0, qh = q01 + c1, qw = q02 + c2;
        yoff[nt] = kOutOfRange;
        if constexpr (BWD) {
            // dx positions: the box itself
            if (c0 < T0 && qd < a0.O && qh < a1.O && qw < a2.O)
                yoff[nt] = (uint32_t)((qd * a1.O + qh) * a2.O + qw) * ES;
        } else if (c0 < T0 && qd < ph.qn[0] && qh < ph.qn[1] && qw < ph.qn[2]) {
            const int o0 = a0.S * qd + ph.r[0], o1 = a1.S * qh + ph.r[1], o2 = a2.S * qw + ph.r[2];
            yoff[nt] = (uint32_t)((o0 * a1.O + o1) * a2.O + o2) * ES;
        }
    }
    const int co_w = co_t * BM + wm * WM;  // first output channel of this wave
    const int act = p.act;  // the activation after the bias (ACT instances only)
    // arithmetic type of two-byte elements
    using HT = typename std::conditional<std::is_same<T, _Float16>::value, _Float16, __bf16>::type;
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
        // the stores, instantiated per activation code A (the switch on the
        // activation runs once, outside the unrolled loops)
        auto store_all = [&](auto act_tag) __attribute__((always_inline)) {
            constexpr int A = decltype(act_tag)::value;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    // this lane's channel: mt*32 + 8*(j/4) + 4*(lane/32) + j%4
                    const uint32_t co_u = mt * 32 + 8 * (j >> 2) + (j & 3);
                    float bv;
                    if constexpr (ES == 2)
                        bv = half_to_f32<HT>(__builtin_amdgcn_raw_buffer_load_b16(bs, (co_u + lane_co) * 2, 0, 0));
                    else
                        bv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bs, (co_u + lane_co) * 4, 0, 0));
                    // rows past Cog (tile padding) store nothing: their channel
                    // offset could wrap the 32-bit range on large planes and
                    // land inside the slice; for real rows yoff + cbytes stays
                    // below 2^32 (the slice is below 2^31 bytes)
                    const bool row_ok = (int)(co_u + lane_co) < co_left;
                    const uint32_t cbytes = (co_u + lane_co) * ypl_bytes;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        float v = acc[mt][nt][j] + bv;
                        if constexpr (A != CONVT_ACT_NONE) v = activate<ES == 2>(A, v);
                        const uint32_t off = row_ok ? yoff[nt] + cbytes : kOutOfRange;
                        if constexpr (ES == 2)
                            __builtin_amdgcn_raw_buffer_store_b16(f32_to_half<HT>(v), ys, off, 0, 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ys, off, 0, 0);
                    }
                }
            }
        };
        if constexpr (ACT) {
            switch (act) {
                case CONVT_ACT_RELU: store_all(std::integral_constant<int, CONVT_ACT_RELU>{}); break;
                case CONVT_ACT_SIGMOID: store_all(std::integral_constant<int, CONVT_ACT_SIGMOID>{}); break;
                case CONVT_ACT_TANH: store_all(std::integral_constant<int, CONVT_ACT_TANH>{}); break;
                case CONVT_ACT_SILU: store_all(std::integral_constant<int, CONVT_ACT_SILU>{}); break;
                case CONVT_ACT_GELU: store_all(std::integral_constant<int, CONVT_ACT_GELU>{}); break;
                default: store_all(std::integral_constant<int, CONVT_ACT_NONE>{}); break;
            }
        } else {
            store_all(std::integral_constant<int, CONVT_ACT_NONE>{});
        }
    }
}

// Instances with an activation (ACT) are separate, so that kernels without
// one carry none of its code in their unrolled epilogue.
template <typename T, int CFG, int GS, bool BWD>
static void launch_cfg(const DevParams &p, int64_t tab_offset, const void *x, const void *ws,
                       const void *bias, void *y, hipStream_t stream) {
    if constexpr (tiles::gemm_cfg_valid(tiles::kGemmCfg[CFG], GS)) {
        const int32_t *tab = (const int32_t *)((const char *)ws + tab_offset);
        const dim3 grid(p.n_blocks), block(tiles::kGemmCfg[CFG].nw * 64);
        if constexpr (!BWD) {
            if (p.act != CONVT_ACT_NONE) {
                hipLaunchKernelGGL((phase_gemm_kernel<T, CFG, GS, false, true>), grid, block, 0,
                                   stream, p, (const T *)x, (const T *)ws, tab, (const T *)bias,
                                   (T *)y);
                return;
            }
        }
        hipLaunchKernelGGL((phase_gemm_kernel<T, CFG, GS, BWD, false>), grid, block, 0, stream, p,
                           (const T *)x, (const T *)ws, tab, (const T *)bias, (T *)y);
    }
}

template <typename T, int CFG, bool BWD>
static hipError_t launch_gs(const DevParams &p, int64_t tab_offset, const void *x, const void *ws,
                            const void *bias, void *y, hipStream_t stream) {
    const int gs = p.gemm_gs;
    if (gs < 1 || gs > tiles::kGemmTapGroup || !tiles::gemm_cfg_valid(tiles::kGemmCfg[CFG], gs))
        return hipErrorInvalidValue;
    switch (gs) {
        case 1: launch_cfg<T, CFG, 1, BWD>(p, tab_offset, x, ws, bias, y, stream); break;
        case 2: launch_cfg<T, CFG, 2, BWD>(p, tab_offset, x, ws, bias, y, stream); break;
        case 3: launch_cfg<T, CFG, 3, BWD>(p, tab_offset, x, ws, bias, y, stream); break;
        case 4: launch_cfg<T, CFG, 4, BWD>(p, tab_offset, x, ws, bias, y, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool BWD>
static hipError_t launch_any(const DevParams &p, int64_t tab_offset, const void *x, const void *wr,
                             const void *bias, void *y, hipStream_t stream) {
    if (p.n_blocks <= 0) return hipSuccess;
    if (!p.wr_chunked) return hipErrorInvalidValue;
    switch (p.gemm_cfg) {
        case 0: return p.f16 ? launch_gs<_Float16, 0, BWD>(p, tab_offset, x, wr, bias, y, stream)
                             : launch_gs<uint16_t, 0, BWD>(p, tab_offset, x, wr, bias, y, stream);
        case 1: return p.f16 ? launch_gs<_Float16, 1, BWD>(p, tab_offset, x, wr, bias, y, stream)
                             : launch_gs<uint16_t, 1, BWD>(p, tab_offset, x, wr, bias, y, stream);
        case 2: return p.f16 ? launch_gs<_Float16, 2, BWD>(p, tab_offset, x, wr, bias, y, stream)
                             : launch_gs<uint16_t, 2, BWD>(p, tab_offset, x, wr, bias, y, stream);
        case 3: return launch_gs<float, 3, BWD>(p, tab_offset, x, wr, bias, y, stream);
        case 4: return launch_gs<float, 4, BWD>(p, tab_offset, x, wr, bias, y, stream);
        case 5: return launch_gs<float, 5, BWD>(p, tab_offset, x, wr, bias, y, stream);
        case 6: return p.f16 ? launch_gs<_Float16, 6, BWD>(p, tab_offset, x, wr, bias, y, stream)
                             : launch_gs<uint16_t, 6, BWD>(p, tab_offset, x, wr, bias, y, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_phase_gemm(const Plan &pl, const void *x, const void *wr, const void *bias,
                             void *y, hipStream_t stream) {
    return launch_any<false>(pl.dp, pl.tab_offset, x, wr, bias, y, stream);
}

// Backward data: x is dy (channel-chunked copy for bfloat16), y is dx, no
// bias (the backward problem has has_bias = 0, so the bias resource is
// empty; dx stands in for its pointer).
hipError_t launch_phase_gemm_bwd(const Plan &pl, const void *dy, const void *wr, void *dx,
                                 hipStream_t stream) {
    return launch_any<true>(pl.bdp, pl.bwd_tab_offset, dy, wr, dx, dx, stream);
}

}  // namespace convt
