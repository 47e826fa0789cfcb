// Stride-phase implicit-gather GEMM for two-byte inputs, reading x in its
// NC[D]HW layout (gfx950, one 256-thread block per CU).
//
// The operation splits by output residue (the stride phases): output
// s*q + r of an axis gathers x[q + off(kk)] * w[kk] over the taps kk of
// residue r, so each phase P is, for batch b and group g, the GEMM
//     D[co][q] = sum over (tap, ci) of Wr[g][P][tap][ci][co] * x[b][g*Cig+ci][q + off(tap)]
// with inputs outside x read as zero (the implicit padding): no
// zero-inserted input, no column matrix, no scatter pass. The huggingface
// ai.onnx.ConvTranspose page (Implementation variants) describes this
// implicit GEMM for stride 1 over the in-channel-by-tap depth, with input
// windows read straight from the tensor; the phase split carries it to every
// stride.
//
// Tile: a block computes BM output channels x BN positions of one phase
// (the positions a (T0, T1, T2) box in q space), four waves each holding a
// 128 x 128 accumulator tile (4 x 4 fragments of v_mfma_f32_32x32x16). The
// K loop runs over chunks of 16 input channels; one pipeline stage is one
// chunk with every tap of the phase (GS taps, the phase padded with zero
// taps), so a stage loads the chunk's weight tiles and its input halo once
// and feeds GS taps of MFMAs from them.
//
// Operands in LDS, two buffers each:
//  * weights: GS tiles of [BM][32 bytes] (16 channels of one output channel
//    per row), copied unchanged from the reordered weights, whose row
//    halves are XOR-swizzled on bit 3 of the row;
//  * input halo: the q box grown by the phase's tap span, as rows of 32
//    bytes (16 channels of one position), halves swizzled the same way on
//    bit 3 of the row index. x itself is channel-planar, so each thread
//    loads 4-byte pairs of neighbouring positions from 8 channels and
//    transposes them with byte permutes into two 16-byte position rows.
//    The box's first column and its width are even, so every pair lies
//    within one row of x (the planner requires an even x row length).
//
// Pipeline: all global loads go into registers through buffer loads whose
// range check returns zero outside the (batch, group) slice, two stages
// ahead (two register sets, alternating): at the top of stage s the loads
// of stage s + 2 are issued; the MFMAs of stage s read LDS buffer s % 2; at
// the bottom the registers of stage s + 1 (issued one stage earlier) are
// written to LDS buffer (s + 1) % 2, and the block meets at a barrier.
// Within a stage the operands of tap u + 1 are read from LDS while the
// MFMAs of tap u run.
//
// Epilogue: acc + bias in float32, the activation if any, one rounding to
// the element type, stored to y[b][g*Cog+co][s*q + r]; positions past the
// phase's q range and rows past Cog fall outside the store resource.
#include <type_traits>

#include "kcommon.h"
#include "launch.h"

namespace convt {

namespace {

constexpr int kNThreads = 256;

}  // namespace

template <typename T, int WGM, int GS, int XU, int ACT, bool Y16>
__global__ __launch_bounds__(kNThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void phase_gemm_nchw_kernel(DevParams p, const T *__restrict__ x, const T *__restrict__ wr,
                            const T *__restrict__ bias, T *__restrict__ y) {
    constexpr int MT = 4, NT = 4;           // 32 x 32 fragments per wave
    constexpr int WGN = 4 / WGM;            // waves along the positions
    constexpr int BM = WGM * MT * 32;       // output channels per block
    constexpr int WROW = 32;                // bytes of a weight or halo row (16 channels)
    constexpr int WTILE = BM * WROW;        // one tap's weight tile
    constexpr int WBUF = GS * WTILE;        // one stage's weight tiles
    constexpr int WV = WBUF / 16 / kNThreads;  // 16-byte weight vectors per thread and stage
    static_assert(WV * 16 * kNThreads == WBUF, "weight tiles split evenly over the threads");
    using HT = typename std::conditional<std::is_same<T, _Float16>::value, _Float16, __bf16>::type;
    using Frag = typename std::conditional<std::is_same<T, _Float16>::value, f16x8, bf16x8>::type;

    constexpr int XBUF = XU * kNThreads * WROW;  // one halo buffer: 256 * XU rows
    // LDS: two stages of weight tiles, two halo buffers, the block's bias
    // and a 32-byte sink that halo units past the halo write to (a select,
    // not a branch, keeps each tap's instructions in one block for the
    // scheduler)
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * WBUF + 2 * XBUF + BM * 4 + 32];
    unsigned char *ws0 = lds, *ws1 = lds + WBUF;
    unsigned char *xs0 = lds + 2 * WBUF, *xs1 = xs0 + XBUF;
    float *bias_s = (float *)(xs1 + XBUF);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;

    // ---- block coordinates: co tile fastest, then phase, q tile, group, batch
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
    // the halo box of this phase: origin (relative to the q box) at the
    // phase's smallest input offset per axis, the last axis rounded down to
    // an even column; extents the box plus the tap span, the last rounded up
    // to even
    const int h0 = ph.off0[0], h1 = ph.off0[1], h2 = ph.off0[2] & ~1;
    const int E0 = T0 + (ph.n[0] - 1) * a0.ostep;
    const int E1 = T1 + (ph.n[1] - 1) * a1.ostep;
    const int E2 = (T2 + (ph.n[2] - 1) * a2.ostep + (ph.off0[2] - h2) + 1) & ~1;
    const int npairs = E0 * E1 * (E2 >> 1);  // position pairs of the halo
    const int nunits = 2 * npairs;            // (pair, 8-channel half) units
    const int co0 = co_t * BM;

    // ---- bias of the block's channels: requested now, written to LDS (in
    // float32) once the first stages' loads are on their way ----
    float bias_v = 0.0f;
    if (tid < BM && p.has_bias && co0 + tid < p.Cog)
        bias_v = half_to_f32<HT>(__builtin_bit_cast(uint16_t, bias[g * p.Cog + co0 + tid]));

    // ---- per-thread halo units: (pair, half) u = tid + 256 k, pairs fastest
    // so that a wave's loads of one channel cover consecutive positions ----
    const uint32_t plane2 = (uint32_t)p.x_plane * 2u;
    // xoff: byte offset of the unit's first channel and pair (out of range
    // for positions outside x and for units past the halo, which read zeros);
    // xdst: LDS byte offset of the unit's first row in a halo buffer (+ 32
    // for the second), or 0xffffffff for units past the halo
    uint32_t xoff[XU];
    uint32_t xdst[XU];
#pragma unroll
    for (int k = 0; k < XU; ++k) {
        const int u = tid + kNThreads * k;
        xoff[k] = kOutOfRange;
        xdst[k] = 0xffffffffu;
        if (u < nunits) {
            const int hh = u >= npairs ? 1 : 0;
            const int pr = u - hh * npairs;
            const int hp = E2 >> 1;
            const int prh = div_small(pr, hp), cp = pr - prh * hp;
            const int e0 = div_small(prh, E1), e1 = prh - e0 * E1;
            const int row = (e0 * E1 + e1) * E2 + 2 * cp;
            xdst[k] = (uint32_t)(row * WROW + ((hh ^ ((row >> 3) & 1)) << 4));
            const int i0 = q00 + h0 + e0, i1 = q01 + h1 + e1, i2 = q02 + h2 + 2 * cp;
            if (i0 >= 0 && i0 < a0.I && i1 >= 0 && i1 < a1.I && i2 >= 0 && i2 < a2.I)
                xoff[k] = (uint32_t)((i0 * a1.I + i1) * a2.I + i2) * 2u + (uint32_t)(hh * 8) * plane2;
        }
    }
    // the (batch, group) slice of x: channels past Cig read zero
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc_uniform(
        x + ((int64_t)b * p.Ci + (int64_t)g * p.Cig) * p.x_plane, (uint32_t)p.Cig * plane2);

    // ---- weight tiles: stage c (chunk c) holds, for the phase's taps
    // t < GS, the tile Wr[g][tapbase + t][c][co0 .. co0 + BM)[32 bytes];
    // thread tid copies 16-byte vectors v = tid + 256 j ----
    const int nchunks = p.cig_pad / 16;
    const uint32_t tile_stride = (uint32_t)nchunks * (uint32_t)p.cog_pad * WROW;  // between taps
    const uint32_t chunk_stride = (uint32_t)p.cog_pad * WROW;
    const u32x4 wrs = rsrc_words(wr + (int64_t)(g * p.ktot_pad + ph.tapbase) * nchunks * p.cog_pad * 16,
                                 (uint32_t)GS * tile_stride);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)&lds[0];
    uint32_t woff[WV];
#pragma unroll
    for (int j = 0; j < WV; ++j) {
        const int v = tid + kNThreads * j;
        const int t = v / (BM * 2), within = v % (BM * 2);
        woff[j] = (uint32_t)t * tile_stride + (uint32_t)co0 * WROW + (uint32_t)within * 16u;
    }

    // ---- weights go global -> LDS directly (16-byte LDS-destination
    // loads, one stage ahead: lane l of vector v = tid + 256 j lands at
    // wsb + v * 16, the tiles' linear layout); part t (of GS) copies the
    // vectors j with j = t (mod GS) of chunk c into buffer wsb
    auto copy_w_part = [&](unsigned char *wsb, int c, int t) __attribute__((always_inline)) {
        const uint32_t cw = (uint32_t)c * chunk_stride;
        const uint32_t base = lds_base + (uint32_t)(wsb - lds) + (uint32_t)wave * 1024u;
#pragma unroll
        for (int j = 0; j < WV; ++j) {
            if (j % GS != t) continue;
            copy_to_lds<16>(base + (uint32_t)(j * kNThreads * 16), woff[j] + cw, wrs);
        }
    };
    // ---- register stages (the input halo) ----
    struct Stage {
        uint32_t xv[XU][8];
    };
    // part t (of GS) of loading chunk c into a stage's registers: the halo
    // units k with k = t (mod GS) (offsets common to the wave go in the
    // scalar offset, which the range check includes like the vector one)
    auto load_part = [&](Stage &st, int c, int t) __attribute__((always_inline)) {
        const uint32_t cx = (uint32_t)(c * 16) * plane2;
#pragma unroll
        for (int k = 0; k < XU; ++k) {
            if (k % GS != t) continue;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                st.xv[k][e] = __builtin_amdgcn_raw_buffer_load_b32(xrs, xoff[k], cx + (uint32_t)e * plane2, 0);
        }
    };
    auto load_stage = [&](Stage &st, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < GS; ++t) load_part(st, c, t);
    };
    // part t (of GS) of writing a stage's registers to LDS: the halo units k
    // with k = t (mod GS); units past the halo write the sink
    auto store_part = [&](const Stage &st, unsigned char *xsb, int t) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < XU; ++k) {
            if (k % GS != t) continue;
            const uint32_t *d = st.xv[k];
            const u32x4 r0 = {lo_pair(d[0], d[1]), lo_pair(d[2], d[3]), lo_pair(d[4], d[5]), lo_pair(d[6], d[7])};
            const u32x4 r1 = {hi_pair(d[0], d[1]), hi_pair(d[2], d[3]), hi_pair(d[4], d[5]), hi_pair(d[6], d[7])};
            // the sink, as an offset from this halo buffer
            const uint32_t sink = (uint32_t)(lds + 2 * WBUF + 2 * XBUF + BM * 4 - xsb);
            const bool used = xdst[k] != 0xffffffffu;
            *(u32x4 *)(xsb + (used ? xdst[k] : sink)) = r0;
            *(u32x4 *)(xsb + (used ? xdst[k] + WROW : sink + 16)) = r1;
        }
    };
    auto store_stage = [&](const Stage &st, unsigned char *xsb) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < GS; ++t) store_part(st, xsb, t);
    };

    // ---- MFMA operands ----
    // A: weight row m (output channel) of the tap's tile, 16-byte half kv
    // (channels 8 kv ..), stored at half kv ^ (bit 3 of m)
    const int kv = lane >> 5;
    int aoff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = wm * MT * 32 + mt * 32 + (lane & 31);
        aoff[mt] = m * WROW + ((kv ^ ((m >> 3) & 1)) << 4);
    }
    // B: the halo row of each of this lane's positions for a zero tap shift
    // (the box extents are powers of two)
    const int lg2 = __builtin_ctz(T2), lg1 = __builtin_ctz(T1);
    int brow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = wn * NT * 32 + nt * 32 + (lane & 31);
        const int c2 = n & (T2 - 1), c1 = (n >> lg2) & (T1 - 1), c0 = n >> (lg2 + lg1);
        brow[nt] = (c0 * E1 + c1) * E2 + c2;
    }
    // halo row shift of each tap (taps in (j0, j1, j2) order, ascending
    // input offset; the padding taps, whose weights are zero, shift by 0)
    int drow[GS];
#pragma unroll
    for (int t = 0; t < GS; ++t) {
        int d = 0;
        if (t < ph.ntaps) {
            const int j2 = t % ph.n[2], j1 = (t / ph.n[2]) % ph.n[1], j0 = t / (ph.n[1] * ph.n[2]);
            d = ((ph.off0[0] + j0 * a0.ostep - h0) * E1 + (ph.off0[1] + j1 * a1.ostep - h1)) * E2 +
                (ph.off0[2] + j2 * a2.ostep - h2);
        }
        drow[t] = __builtin_amdgcn_readfirstlane(d);
    }

    f32x16 acc[MT][NT];

    auto read_frags = [&](Frag (&fa)[MT], Frag (&fb)[NT], const unsigned char *wsb,
                          const unsigned char *xsb, int t) __attribute__((always_inline)) {
        const unsigned char *wt = wsb + t * WTILE;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) fa[mt] = __builtin_bit_cast(Frag, *(const u32x4 *)(wt + aoff[mt]));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int r = brow[nt] + drow[t];
            fb[nt] = __builtin_bit_cast(Frag, *(const u32x4 *)(xsb + r * WROW + ((kv ^ ((r >> 3) & 1)) << 4)));
        }
    };
    auto mfma = [&](const Frag (&fa)[MT], const Frag (&fb)[NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if constexpr (std::is_same<T, _Float16>::value)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[mt], fb[nt], acc[mt][nt], 0, 0, 0);
                else
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mt], fb[nt], acc[mt][nt], 0, 0, 0);
            }
    };
    // the MFMAs of one stage from LDS buffers (wsb, xsb). Between the taps'
    // MFMA groups (issued as a whole, so the matrix pipe stays fed) the wave
    // copies part of chunk wc's weights into the next stage's buffer nwsb,
    // writes part of the next stage's halo registers (nst) to its buffer
    // nxsb (no wave reads those buffers during this stage), and issues part
    // of the halo loads of chunk lc into the registers lst: spread this way,
    // neither the loads nor the stores hold up the MFMA issue in one burst.
    auto compute = [&](const unsigned char *wsb, const unsigned char *xsb, const Stage &nst,
                       unsigned char *nwsb, unsigned char *nxsb, Stage &lst, int lc, int wc)
        __attribute__((always_inline)) {
        Frag fa[2][MT], fb[2][NT];
        read_frags(fa[0], fb[0], wsb, xsb, 0);
#pragma unroll
        for (int t = 0; t < GS; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            if (t + 1 < GS) read_frags(fa[(t + 1) & 1], fb[(t + 1) & 1], wsb, xsb, t + 1);
            mfma(fa[t & 1], fb[t & 1]);
            copy_w_part(nwsb, wc, t);
            store_part(nst, nxsb, t);
            load_part(lst, lc, t);
            // issue order within the tap: each MFMA followed by at most one
            // LDS read, one global load, one LDS write and a few VALU ops
#pragma unroll
            for (int i = 0; i < MT * NT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // the weight copies of the next stage (and every other load) landed,
    // this wave's LDS writes done, then the block's barrier
    auto barrier = [&]() __attribute__((always_inline)) { stage_barrier<0>(); };

    // ---- pipeline over the chunks (an even count: the planner pads the
    // channels to whole pairs of chunks with zero weights) ----
    const int last = nchunks - 1;
    Stage R0, R1;
#pragma unroll
    for (int t = 0; t < GS; ++t) copy_w_part(ws0, 0, t);
    load_stage(R0, 0);
    load_stage(R1, 1);
    if (tid < BM) bias_s[tid] = bias_v;
    store_stage(R0, xs0);
    barrier();
    // the accumulators start at the bias of their output channel (lane l of
    // fragment (mt, nt) holds rows mt*32 + 8*(j/4) + 4*(l/32) + j%4)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float bv = bias_s[wm * MT * 32 + mt * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3)];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt][j] = bv;
        }
    for (int c = 0; c < nchunks; c += 2) {
        // stage c from buffers 0, writing stage c + 1 (R1) to buffers 1 and
        // loading chunk c + 2 into R0; the loads past the last chunk repeat
        // it and are never used
        compute(ws0, xs0, R1, ws1, xs1, R0, min(c + 2, last), c + 1);
        barrier();
        // stage c + 1 from buffers 1, writing stage c + 2 (R0) to buffers 0
        compute(ws1, xs1, R0, ws0, xs0, R1, min(c + 3, last), min(c + 2, last));
        barrier();
    }

    // ---- epilogue: the activation if any, one rounding, 2-byte stores
    // (a phase's outputs are s apart along each axis) ----
    uint32_t yoff[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = wn * NT * 32 + nt * 32 + (lane & 31);
        const int c2 = n & (T2 - 1), c1 = (n >> lg2) & (T1 - 1), c0 = n >> (lg2 + lg1);
        const int qd = q00 + c0, qh = q01 + c1, qw = q02 + c2;
        yoff[nt] = kOutOfRange;
        if (qd < ph.qn[0] && qh < ph.qn[1] && qw < ph.qn[2]) {
            const int o0 = a0.S * qd + ph.r[0], o1 = a1.S * qh + ph.r[1], o2 = a2.S * qw + ph.r[2];
            yoff[nt] = (uint32_t)((o0 * a1.O + o1) * a2.O + o2) * 2u;
        }
    }
    const int co_w = co0 + wm * MT * 32;  // first output channel of this wave
    const int co_left = p.Cog - co_w;
    if (co_left <= 0) return;
    const uint32_t ypl_bytes = (uint32_t)p.y_plane * 2u;
    const __amdgpu_buffer_rsrc_t ys = make_rsrc_uniform(
        y + ((int64_t)b * p.Co + (int64_t)g * p.Cog + co_w) * p.y_plane, (uint32_t)co_left * ypl_bytes);
    const uint32_t lane_co = 4u * (uint32_t)(lane >> 5);
    // The lane's position (and its half's 4-row channel step) in the vector
    // offset, the fragment row in the scalar one: the range check covers
    // both, so rows past Cog (and masked positions) fall outside the
    // resource, which ends at Cog; the planner keeps every such sum below
    // 2^32.
    uint32_t vo[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) vo[nt] = yoff[nt] + lane_co * ypl_bytes;
    // channel j pairs (j, j + 1), j even, are rows 1 apart: one conversion
    // gives both, stored from the low and the high half
    auto store_all = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                const uint32_t so = (uint32_t)(mt * 32 + 8 * (j >> 2) + (j & 3)) * ypl_bytes;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    float v0 = acc[mt][nt][j], v1 = acc[mt][nt][j + 1];
                    if constexpr (ACT != CONVT_ACT_NONE) {
                        v0 = activate<true>(ACT, v0);
                        v1 = activate<true>(ACT, v1);
                    }
                    const uint32_t pk = pack_half2<HT>(v0, v1);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pk, ys, vo[nt], so, 0);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pk >> 16), ys, vo[nt], so + ypl_bytes, 0);
                }
            }
    };
    // Y16 (width stride 1, output rows of whole 16-byte pieces, y 16-byte
    // aligned; a compile-time choice, so that each instance holds one store
    // path): a wave stages 32 channels x its 128 positions at a time in
    // LDS (the stage buffers are free past the loop's last barrier) and
    // stores 16-byte row pieces, 8 positions each, instead of 2-byte stores
    auto store_staged = [&]() __attribute__((always_inline)) {
        constexpr int SP = 2 * NT * 32 + 16;  // staging bytes per channel
        unsigned char *stg = lds + wave * (32 * SP);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                const int r = 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);  // fragment rows r, r + 1
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    float v0 = acc[mt][nt][j], v1 = acc[mt][nt][j + 1];
                    if constexpr (ACT != CONVT_ACT_NONE) {
                        v0 = activate<true>(ACT, v0);
                        v1 = activate<true>(ACT, v1);
                    }
                    const uint32_t pk = pack_half2<HT>(v0, v1);
                    const int pos = nt * 32 + (lane & 31);
                    *(uint16_t *)(stg + r * SP + pos * 2) = (uint16_t)pk;
                    *(uint16_t *)(stg + (r + 1) * SP + pos * 2) = (uint16_t)(pk >> 16);
                }
            }
            // piece k = lane + 64 i: channel row k / 16, positions 8 (k % 16) ..
#pragma unroll
            for (int i = 0; i < NT * 32 * 32 / 8 / 64; ++i) {
                const int k = lane + 64 * i, r = k >> 4, pp = k & 15;
                const u32x4 v = *(const u32x4 *)(stg + r * SP + pp * 16);
                const int n = wn * NT * 32 + pp * 8;
                const int c2 = n & (T2 - 1), c1 = (n >> lg2) & (T1 - 1), c0 = n >> (lg2 + lg1);
                const int qd = q00 + c0, qh = q01 + c1, qw = q02 + c2;
                uint32_t off = kOutOfRange;
                if (qd < ph.qn[0] && qh < ph.qn[1] && qw < ph.qn[2]) {
                    const int o0 = a0.S * qd + ph.r[0], o1 = a1.S * qh + ph.r[1];
                    off = (uint32_t)((o0 * a1.O + o1) * a2.O + qw) * 2u;
                }
                __builtin_amdgcn_raw_buffer_store_b128(v, ys, off, (uint32_t)(mt * 32 + r) * ypl_bytes, 0);
            }
        }
    };
    // The activation kind is a template parameter (the launcher picks the
    // instance), so each instance holds one store path: an inlined copy per
    // kind behind a run-time switch left the staged instances with
    // kilobytes of scratch per lane in the epilogue.
    if constexpr (Y16)
        store_staged();
    else
        store_all();
}

template <typename T, int CFG, bool Y16>
static hipError_t launch_nchw_y(const Plan &pl, const void *x, const void *wr, const void *bias,
                                void *y, hipStream_t stream) {
    constexpr tiles::NchwCfg C = tiles::kNchwCfg[CFG];
    const DevParams &p = pl.dp;
    const dim3 grid(p.n_blocks), block(kNThreads);
    const size_t lds = 0;  // static
    auto go = [&](auto act_tag) {
        hipLaunchKernelGGL((phase_gemm_nchw_kernel<T, C.wgm, C.gs, C.xu, decltype(act_tag)::value, Y16>), grid,
                           block, lds, stream, p, (const T *)x, (const T *)wr, (const T *)bias, (T *)y);
    };
#ifndef NCHW_TUNE
    switch (p.act) {
        case CONVT_ACT_RELU: go(std::integral_constant<int, CONVT_ACT_RELU>{}); break;
        case CONVT_ACT_SIGMOID: go(std::integral_constant<int, CONVT_ACT_SIGMOID>{}); break;
        case CONVT_ACT_TANH: go(std::integral_constant<int, CONVT_ACT_TANH>{}); break;
        case CONVT_ACT_SILU: go(std::integral_constant<int, CONVT_ACT_SILU>{}); break;
        case CONVT_ACT_GELU: go(std::integral_constant<int, CONVT_ACT_GELU>{}); break;
        default: go(std::integral_constant<int, CONVT_ACT_NONE>{}); break;
    }
#else
    go(std::integral_constant<int, CONVT_ACT_NONE>{});
#endif
    return hipGetLastError();
}

template <typename T, int CFG>
static hipError_t launch_nchw_t(const Plan &pl, const void *x, const void *wr, const void *bias,
                                void *y, hipStream_t stream) {
    const DevParams &p = pl.dp;
    // 16-byte output pieces: width stride 1 (a phase's outputs contiguous
    // along the row), rows and the box's width whole 8-position pieces
    const bool y16 = p.ax[2].S == 1 && p.ax[2].O % 8 == 0 && p.tw % 8 == 0 && (uintptr_t)y % 16 == 0;
    return y16 ? launch_nchw_y<T, CFG, true>(pl, x, wr, bias, y, stream)
               : launch_nchw_y<T, CFG, false>(pl, x, wr, bias, y, stream);
}

template <typename T>
static hipError_t launch_nchw_cfg(const Plan &pl, const void *x, const void *wr, const void *bias,
                                  void *y, hipStream_t stream) {
    switch (pl.dp.nchw_cfg) {
        case 0: return launch_nchw_t<T, 0>(pl, x, wr, bias, y, stream);
#ifndef NCHW_TUNE
        case 1: return launch_nchw_t<T, 1>(pl, x, wr, bias, y, stream);
        case 2: return launch_nchw_t<T, 2>(pl, x, wr, bias, y, stream);
        case 3: return launch_nchw_t<T, 3>(pl, x, wr, bias, y, stream);
#endif
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_phase_gemm_nchw(const Plan &pl, const void *x, const void *wr, const void *bias,
                                  void *y, hipStream_t stream) {
    const DevParams &p = pl.dp;
    if (p.n_blocks <= 0) return hipSuccess;
    if (!p.gemm_nchw || !p.wr_chunked || pl.elem_bytes != 2) return hipErrorInvalidValue;
#ifdef NCHW_TUNE
    return launch_nchw_cfg<uint16_t>(pl, x, wr, bias, y, stream);
#else
    return p.f16 ? launch_nchw_cfg<_Float16>(pl, x, wr, bias, y, stream)
                 : launch_nchw_cfg<uint16_t>(pl, x, wr, bias, y, stream);
#endif
}

}  // namespace convt
