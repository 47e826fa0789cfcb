// Backward data (the input gradient dx) on MFMA for two-byte types with
// stride 2 and dilation 1 on the height and width axes and 16 taps over those
// two axes (4 x 4, 2 x 8, 8 x 2); gfx950, one 256-thread block per CU.
//
// The adjoint of the forward's scatter-add (the KInference convTranspose2d
// page, Summary: out[i*s - p + k*d] += x[i] * w[k]) gathers
//     dx[b][g*Cig + ci][i] = sum over (co, kk) of W[g*Cig + ci][co][kk] * dy[b][g*Cog + co][s*i - p + kk*d].
// Along height and width, tap k = 2m + c lands on dy position
// 2(i + m) + c - p: the plane of residue r[c] = (c - p) mod 2 at index
// j = i + m + floor((c - p) / 2). All taps of one parity read one phase plane
// with a per-tap shift, so for a box of dx positions and 8 dy channels one
// halo box in each of the four (height, width) phase planes serves all 16
// taps: the stride-phase reuse of the huggingface ai.onnx.ConvTranspose
// page's blocked variant (Implementation variants), run backwards.
//
// GEMM: 128 dx channels x a box of 256 dx positions per block, K = dy
// channels x taps. Waves 2 x 2, each 64 channels x 128 positions: 4 x 2
// fragments of v_mfma_f32_32x32x16 with the positions as the MFMA's rows, so
// that a lane's accumulators hold 4 consecutive positions of one channel. A
// K step pairs two taps: lanes 0-31 carry 8 dy channels of the first, lanes
// 32-63 the same channels of the second. A stage is one chunk of 8 dy
// channels at one depth tap: 16 taps, 8 K steps.
//
// Operands in LDS (two stage buffers):
//  * weights: [tap slot][128 rows][8 dy channels] of 16-byte rows, slots in
//    W's own height x width tap order. A thread loads 16 bytes (8 taps) of
//    its dx channel's row for each of the chunk's 8 dy channels and
//    transposes the 8 x 8 block of two-byte values in registers into 8 slot
//    rows (byte permutes); W is read as stored.
//  * halo: four phase planes of E1 x E2 rows of 16 bytes (8 dy channels of
//    one plane position). dy is channel-planar with an even row length, so a
//    4-byte load of positions (2J, 2J + 1) of a row holds plane index J of
//    both width residues: a thread loads such pairs from 8 channels and
//    permutes them into one row of each width plane.
//
// Pipeline: register-staged buffer loads (the range check reads zero outside
// dy and W, past the channel chunks and for depth taps outside dy); stage s
// computes from buffer s % 2 while stage s+1 (loaded one stage earlier) is
// written into the other buffer and stage s+2 is loaded; the block meets at
// one barrier per stage, before the last K step, whose operands are already
// in registers.
//
// Epilogue: the accumulators rounded once to the element type, written into
// LDS as [channel][box position], then stored as 16-byte pieces of dx rows.
#include <type_traits>

#include "kcommon.h"
#include "launch.h"

namespace convt {

namespace {
constexpr int kBwdThreads = 256;
}  // namespace

template <typename T, bool KS>
__global__ __launch_bounds__(kBwdThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void allphase_bwd_kernel(BwdAPArgs a, const T *__restrict__ dy, const T *__restrict__ w,
                         T *__restrict__ dx) {
    // KS (the K split): a 128-position box, waves (w & 1, w >> 1) = (channel
    // half, K half), each holding all 128 positions and taking four of a
    // stage's eight K steps; the two K halves' sums meet in LDS at the end
    constexpr int BM = 128;                    // dx channels per block
    constexpr int BN = KS ? 128 : 256;         // dx positions per block (the box)
    constexpr int MT = 2, NT = 4;              // fragments per wave: channels, positions
    constexpr int NK = KS ? 4 : 8;             // K steps per wave and stage
    constexpr int NSLOT = 16;                  // height x width taps
    constexpr int WSUB = NSLOT * BM * 16;      // a stage's weight rows
    constexpr int PROWS = KS ? kBwdPlaneRowsKS : kBwdPlaneRows;
    constexpr int PLANE = (PROWS + 1) * 16;
    constexpr int STAGE = WSUB + 4 * PLANE;
    constexpr int MAIN = 2 * STAGE;
    constexpr int PITCH = 2 * BN + 16;         // epilogue staging bytes per channel
    constexpr int EPI = BM * PITCH;
    constexpr int RED = KS ? 2 * 64 * MT * NT * 64 : 0;  // the K-split sums of two waves, float32
    constexpr int LDS_A = MAIN > EPI ? MAIN : EPI;
    constexpr int LDS_BYTES = LDS_A > RED ? LDS_A : RED;
    constexpr int XU = KS ? 2 : 3;             // halo units per thread and stage
    static_assert(XU * kBwdThreads >= 2 * PROWS, "halo units cover two planes' rows");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    using HT = typename std::conditional<std::is_same<T, _Float16>::value, _Float16, __bf16>::type;
    using Frag = typename std::conditional<std::is_same<T, _Float16>::value, f16x8, bf16x8>::type;

    __shared__ __attribute__((aligned(1024))) unsigned char lds[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = KS ? wave & 1 : wave >> 1;  // channel half
    const int wn = KS ? 0 : wave & 1;          // position half
    const int kh = KS ? wave >> 1 : 0;         // K half
    const int kv = lane >> 5;                 // lane half: first or second tap of a K step

    // ---- block coordinates: channel tile fastest, then the box (width,
    // height, depth position), group, batch
    uint32_t bid = (uint32_t)remap_block(blockIdx.x, a.n_blocks, a.xcd_remap);
    uint32_t qq = fast_div(bid, a.div_ci);
    const int ci_t = (int)(bid - qq * (uint32_t)a.n_ci_tiles);
    bid = qq;
    qq = fast_div(bid, a.div_t2);
    const int t2 = (int)(bid - qq * (uint32_t)a.nt[2]);
    bid = qq;
    qq = fast_div(bid, a.div_t1);
    const int t1 = (int)(bid - qq * (uint32_t)a.nt[1]);
    bid = qq;
    qq = fast_div(bid, a.div_t0);
    const int i00 = (int)(bid - qq * (uint32_t)a.nt[0]);  // the box's depth position
    bid = qq;
    qq = fast_div(bid, a.div_g);
    const int g = (int)(bid - qq * (uint32_t)a.G);
    const int b = (int)qq;

    const int T1 = a.T1, T2 = a.T2, E1 = a.E1, E2 = a.E2;
    const int i01 = t1 * T1, i02 = t2 * T2;
    const int ci0 = ci_t * BM;
    const int O1 = a.O[1], O2 = a.O[2], K0 = a.K[0], K2 = a.K[2];

    // ---- halo units: u = tid + 256k is (height residue rh, plane row jh,
    // column pair jw), jw fastest; it loads dy row 2(i01 + tmin1 + jh) + rh,
    // positions 2J and 2J + 1 with J = i02 + tmin2 + jw, of 8 channels, and
    // writes row (jh, jw) of planes (rh, 0) and (rh, 1). xoff: byte offset in
    // a dy channel (out of range outside dy); xdst: LDS offset of the first
    // row within a stage (units past the halo write the spare last row of
    // planes 0 and 1).
    const int npl = E1 * E2;
    uint32_t xoff[XU];
    int xdst[XU];
#pragma unroll
    for (int k = 0; k < XU; ++k) {
        const int u = tid + kBwdThreads * k;
        xoff[k] = kOutOfRange;
        xdst[k] = WSUB + PROWS * 16;
        if (u < 2 * npl) {
            const int rh = u >= npl ? 1 : 0;
            const int rem = u - rh * npl;
            const int jh = div_small(rem, E2), jw = rem - jh * E2;
            xdst[k] = WSUB + 2 * rh * PLANE + (jh * E2 + jw) * 16;
            const int oh = 2 * (i01 + a.tmin1 + jh) + rh;
            const int J = i02 + a.tmin2 + jw;
            if (oh >= 0 && oh < O1 && J >= 0 && 2 * J < O2) xoff[k] = (uint32_t)(oh * O2 + 2 * J) * 2u;
        }
    }
    const uint32_t ypl2 = (uint32_t)a.y_plane * 2u;
    const uint32_t yslice = (uint32_t)(O1 * O2) * 2u;  // one dy depth slice
    const uint32_t ybytes = (uint32_t)a.Cog * ypl2;
    const __amdgpu_buffer_rsrc_t xrs =
        make_rsrc(dy + ((int64_t)b * a.Co + (int64_t)g * a.Cog) * a.y_plane, ybytes);
    // stage cl = (chunk c, depth tap kd): the chunk's first channel and the
    // dy depth slice, as a wave-uniform offset; a depth outside dy gives the
    // resource's size (every lane then reads zero, with no 32-bit wrap)
    auto x_stage = [&](int cl) __attribute__((always_inline)) {
        const uint32_t c = fast_div((uint32_t)cl, a.div_k0);
        const int kd = cl - (int)c * K0;
        const int e0 = a.S0 * i00 - a.P0 + kd * a.D0;
        return (e0 >= 0 && e0 < a.O[0]) ? c * 8u * ypl2 + (uint32_t)e0 * yslice : ybytes;
    };

    // ---- weight unit of this thread: dx channel ci0 + wci, tap octet wo (8
    // of the 16 height x width taps); its 8 loads are the chunk's 8 dy
    // channels. In LDS, octet wo's rows are stored at row wci ^ 12wo,
    // spreading the lanes of one write over the LDS banks (12 keeps a
    // 32-row operand fragment one contiguous group).
    const int ktot = a.ktot;
    const uint32_t wrow = (uint32_t)a.Cog * (uint32_t)ktot * 2u;  // bytes between dx channels
    const uint32_t wbytes = (uint32_t)a.Cig * wrow;
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(w + (int64_t)g * a.Cig * a.Cog * ktot, wbytes);
    const int wo = tid & 1, wci = tid >> 1;
    const uint32_t woff = ci0 + wci < a.Cig ? (uint32_t)(ci0 + wci) * wrow + (uint32_t)wo * 16u : kOutOfRange;
    const int wdst = wo * 8 * (BM * 16) + (wci ^ (12 * wo)) * 16;
    // dy channel 8c + e of stage cl at its depth tap (stored order): the
    // offset within a dx channel's row, or the resource's size past Cog
    auto w_stage = [&](int cl, int e) __attribute__((always_inline)) {
        const uint32_t c = fast_div((uint32_t)cl, a.div_k0);
        const int kd = cl - (int)c * K0;
        const int kds = a.flip ? K0 - 1 - kd : kd;
        const int co = (int)c * 8 + e;
        return co < a.Cog ? ((uint32_t)co * (uint32_t)ktot + (uint32_t)kds * NSLOT) * 2u : wbytes;
    };

    // ---- MFMA operands. K step i of a stage (i + 4 kh with the K split):
    // taps 2i (lanes 0-31) and 2i + 1 (lanes 32-63) in (height, width)
    // order. Per lane: the tap's weight slot row (this lane's channel row of
    // the wave's half) and its halo plane and shift.
    int aslot[NK], boff[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int t = 2 * (i + kh * NK) + kv;
        const int kh = t / K2, kw = t - (t / K2) * K2;
        const int sh = a.flip ? a.K[1] - 1 - kh : kh, sw = a.flip ? K2 - 1 - kw : kw;
        const int sl = sh * K2 + sw;
        aslot[i] = sl * (BM * 16) + (wm * 64 + ((lane & 31) ^ (12 * (sl >> 3)))) * 16;
        const int ch = kh & 1, cw = kw & 1;
        boff[i] = WSUB + (a.r1[ch] * 2 + a.r2[cw]) * PLANE +
                  (((kh >> 1) + a.u1[ch]) * E2 + (kw >> 1) + a.u2[cw]) * 16;
    }
    // halo row (bytes) of box position n = wn*128 + nt*32 + (lane & 31) at
    // zero shift: n's bits split into a per-lane and a wave-uniform part
    // that never carry into each other (T2 a power of two)
    auto halo_row = [&](int n) __attribute__((always_inline)) {
        return ((n >> a.lgT2) * E2 + (n & (T2 - 1))) * 16;
    };
    const int brow = halo_row(lane & 31);
    int bnt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bnt[nt] = __builtin_amdgcn_readfirstlane(halo_row(wn * 128 + nt * 32));

    // ---- register stages
    struct XRegs {
        uint32_t v[XU][8];
    };
    // a stage's wave-uniform load offsets, computed once ahead of its K steps
    // and held in scalar registers (the empty asm keeps the selects from
    // being turned into branches inside the K steps, which would split their
    // scheduling regions)
    struct StageOffs {
        uint32_t x, w[8];
    };
    auto stage_offs = [&](int cl) __attribute__((always_inline)) {
        StageOffs o;
        o.x = __builtin_amdgcn_readfirstlane(x_stage(cl));
        asm volatile("" : "+s"(o.x));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o.w[e] = __builtin_amdgcn_readfirstlane(w_stage(cl, e));
            asm volatile("" : "+s"(o.w[e]));
        }
        return o;
    };
    u32x4 WR[8];
    XRegs X0, X1;
    auto load_w = [&](const StageOffs &so) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            WR[e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, woff, so.w[e], 0));
    };
    auto load_x = [&](XRegs &xr, int k, const StageOffs &so) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            xr.v[k][e] = __builtin_amdgcn_raw_buffer_load_b32(xrs, xoff[k], so.x + (uint32_t)e * ypl2, 0);
    };
    // rows 4h .. 4h+3 of the unit's 8 x 8 block (dy channel e holds taps
    // 2j, 2j + 1 in word j) as slot rows (tap t holds channels 2j, 2j + 1 in
    // word j)
    auto store_w = [&](unsigned char *stage, int h) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int t = 4 * h + tt, j = t >> 1;
            u32x4 r;
            if (t & 1)
                r = {hi_pair(WR[0][j], WR[1][j]), hi_pair(WR[2][j], WR[3][j]), hi_pair(WR[4][j], WR[5][j]),
                     hi_pair(WR[6][j], WR[7][j])};
            else
                r = {lo_pair(WR[0][j], WR[1][j]), lo_pair(WR[2][j], WR[3][j]), lo_pair(WR[4][j], WR[5][j]),
                     lo_pair(WR[6][j], WR[7][j])};
            *(u32x4 *)(stage + wdst + t * (BM * 16)) = r;
        }
    };
    // the unit's two plane rows: even positions (width residue 0) and odd
    auto store_x = [&](const XRegs &xr, int k, unsigned char *stage) __attribute__((always_inline)) {
        const uint32_t *d = xr.v[k];
        const u32x4 r0 = {lo_pair(d[0], d[1]), lo_pair(d[2], d[3]), lo_pair(d[4], d[5]), lo_pair(d[6], d[7])};
        const u32x4 r1 = {hi_pair(d[0], d[1]), hi_pair(d[2], d[3]), hi_pair(d[4], d[5]), hi_pair(d[6], d[7])};
        *(u32x4 *)(stage + xdst[k]) = r0;
        *(u32x4 *)(stage + xdst[k] + PLANE) = r1;
    };

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.0f;
    Frag fa[2][MT], fb[2][NT];
    auto read_frags = [&](Frag (&A)[MT], Frag (&B)[NT], const unsigned char *stage, int i)
        __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            A[mt] = __builtin_bit_cast(Frag, *(const u32x4 *)(stage + aslot[i] + mt * 512));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            B[nt] = __builtin_bit_cast(Frag, *(const u32x4 *)(stage + boff[i] + brow + bnt[nt]));
    };
    // D[position][channel]: the positions' fragment is the MFMA's first operand
    auto mfma = [&](const Frag (&A)[MT], const Frag (&B)[NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if constexpr (std::is_same<T, _Float16>::value)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(B[nt], A[mt], acc[mt][nt], 0, 0, 0);
                else
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B[nt], A[mt], acc[mt][nt], 0, 0, 0);
            }
    };
    // issue order within a K step: each MFMA followed by at most one LDS
    // read, one global load, one LDS write and NV VALU ops
    auto interleave = [&](auto nv) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MT * NT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
            __builtin_amdgcn_sched_group_barrier(0x002, decltype(nv)::value, 0);  // VALU
        }
    };
    auto barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    using V1 = std::integral_constant<int, 1>;
    using V2 = std::integral_constant<int, 2>;
    using V3 = std::integral_constant<int, 3>;
    // stage s from buffer cur: writes stage s+1 (halo xs, weights in WR) to
    // buffer nxt and loads stage cl = s+2 (halo into xl, weights into WR)
    auto stage_body = [&](unsigned char *cur, unsigned char *nxt, const XRegs &xs, XRegs &xl, int cl)
        __attribute__((always_inline)) {
        const StageOffs so = stage_offs(cl);
        if constexpr (KS) {
            __builtin_amdgcn_sched_barrier(0);
            read_frags(fa[1], fb[1], cur, 1);
            mfma(fa[0], fb[0]);
            store_x(xs, 0, nxt);
            load_x(xl, 0, so);
            interleave(V1{});
            __builtin_amdgcn_sched_barrier(0);
            read_frags(fa[0], fb[0], cur, 2);
            mfma(fa[1], fb[1]);
            store_x(xs, 1, nxt);
            load_x(xl, 1, so);
            store_w(nxt, 0);
            interleave(V3{});
            __builtin_amdgcn_sched_barrier(0);
            read_frags(fa[1], fb[1], cur, 3);
            mfma(fa[0], fb[0]);
            store_w(nxt, 1);
            load_w(so);
            interleave(V2{});
        } else {
            __builtin_amdgcn_sched_barrier(0);
            read_frags(fa[1], fb[1], cur, 1);
            mfma(fa[0], fb[0]);
            store_x(xs, 0, nxt);
            load_x(xl, 0, so);
            interleave(V1{});
            __builtin_amdgcn_sched_barrier(0);
            read_frags(fa[0], fb[0], cur, 2);
            mfma(fa[1], fb[1]);
            store_x(xs, 1, nxt);
            load_x(xl, 1, so);
            interleave(V1{});
            __builtin_amdgcn_sched_barrier(0);
            read_frags(fa[1], fb[1], cur, 3);
            mfma(fa[0], fb[0]);
            store_x(xs, 2, nxt);
            load_x(xl, 2, so);
            interleave(V1{});
            __builtin_amdgcn_sched_barrier(0);
            read_frags(fa[0], fb[0], cur, 4);
            mfma(fa[1], fb[1]);
            store_w(nxt, 0);
            interleave(V2{});
            __builtin_amdgcn_sched_barrier(0);
            read_frags(fa[1], fb[1], cur, 5);
            mfma(fa[0], fb[0]);
            store_w(nxt, 1);
            load_w(so);
            interleave(V2{});
            __builtin_amdgcn_sched_barrier(0);
            read_frags(fa[0], fb[0], cur, 6);
            mfma(fa[1], fb[1]);
            interleave(V1{});
            __builtin_amdgcn_sched_barrier(0);
            read_frags(fa[1], fb[1], cur, 7);
            mfma(fa[0], fb[0]);
            interleave(V1{});
        }
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        read_frags(fa[0], fb[0], nxt, 0);
        mfma(fa[1], fb[1]);
#pragma unroll
        for (int i = 0; i < MT * NT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    unsigned char *buf0 = lds, *buf1 = lds + STAGE;
    const StageOffs so0 = stage_offs(0), so1 = stage_offs(1);
    load_w(so0);
#pragma unroll
    for (int k = 0; k < XU; ++k) load_x(X0, k, so0);
#pragma unroll
    for (int k = 0; k < XU; ++k) load_x(X1, k, so1);
    store_w(buf0, 0);
    store_w(buf0, 1);
#pragma unroll
    for (int k = 0; k < XU; ++k) store_x(X0, k, buf0);
    load_w(so1);
    barrier();
    read_frags(fa[0], fb[0], buf0, 0);
    for (int s = 0; s < a.nstages; s += 2) {
        stage_body(buf0, buf1, X1, X0, s + 2);
        stage_body(buf1, buf0, X0, X1, s + 3);
    }

    // ---- epilogue: past this barrier no wave reads the stage buffers (the
    // last stage's trailing operand reads included); lane l of fragment
    // (mt, nt) holds channel wm*64 + mt*32 + (l & 31) at positions
    // wn*128 + nt*32 + 8q + 4(l / 32) + (0..3) in elements 4q .. 4q+3
    barrier();
    if constexpr (KS) {
        // the second K half's sums go through LDS to the first's waves, 16
        // bytes per lane and instruction, lanes contiguous
        float4 *red = (float4 *)lds + wm * (MT * NT * 4 * 64) + lane;
        if (kh == 1) {
#pragma unroll
            for (int f = 0; f < MT * NT; ++f)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16 &v = acc[f / NT][f % NT];
                    red[(f * 4 + q) * 64] = float4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
                }
        }
        barrier();
        if (kh == 0) {
#pragma unroll
            for (int f = 0; f < MT * NT; ++f)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 o = red[(f * 4 + q) * 64];
                    f32x16 &v = acc[f / NT][f % NT];
                    v[4 * q] += o.x;
                    v[4 * q + 1] += o.y;
                    v[4 * q + 2] += o.z;
                    v[4 * q + 3] += o.w;
                }
        }
        barrier();
    }
    if (kh == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int ci = wm * 64 + mt * 32 + (lane & 31);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int pos = wn * 128 + nt * 32 + 8 * q + 4 * kv;
                const u32x2 v = {pack_half2<HT>(acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1]),
                                 pack_half2<HT>(acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3])};
                *(u32x2 *)(lds + ci * PITCH + pos * 2) = v;
            }
    }
    }
    barrier();

    // ---- stores: piece pc (16 bytes, 8 positions) is channel pc / (BN / 8),
    // box positions 8 (pc % (BN / 8)) ..; the box's rows are T1 rows of T2 positions,
    // whole pieces since T2 and the dx row length are multiples of 8.
    // Channels past Cig and positions past dx take the out-of-range offset.
    const uint32_t xpl2 = (uint32_t)a.x_plane * 2u;
    const __amdgpu_buffer_rsrc_t drs =
        make_rsrc(dx + ((int64_t)b * a.Ci + (int64_t)g * a.Cig) * a.x_plane, (uint32_t)a.Cig * xpl2);
    const int I1 = a.I[1], I2 = a.I[2];
#pragma unroll 4
    for (int i = 0; i < BM * BN / 8 / kBwdThreads; ++i) {
        const int pc = tid + kBwdThreads * i;
        const int ci = pc / (BN / 8), rem = pc % (BN / 8);
        const int pos = rem * 8;
        const int row = pos >> a.lgT2, col = pos & (T2 - 1);
        const u32x4 v = *(const u32x4 *)(lds + ci * PITCH + rem * 16);
        uint32_t off = kOutOfRange;
        if (ci0 + ci < a.Cig && i01 + row < I1 && i02 + col < I2)
            off = (uint32_t)(ci0 + ci) * xpl2 + (uint32_t)((i00 * I1 + i01 + row) * I2 + i02 + col) * 2u;
        __builtin_amdgcn_raw_buffer_store_b128(v, drs, off, 0, 0);
    }
}

template <typename T>
static hipError_t launch_bwd_allphase_t(const Plan &pl, const void *dy, const void *w, void *dx,
                                        hipStream_t stream) {
    const BwdAPArgs &a = pl.bap;
    if (a.ksplit)
        hipLaunchKernelGGL((allphase_bwd_kernel<T, true>), dim3(a.n_blocks), dim3(kBwdThreads), 0, stream, a,
                           (const T *)dy, (const T *)w, (T *)dx);
    else
        hipLaunchKernelGGL((allphase_bwd_kernel<T, false>), dim3(a.n_blocks), dim3(kBwdThreads), 0, stream, a,
                           (const T *)dy, (const T *)w, (T *)dx);
    return hipGetLastError();
}

hipError_t launch_allphase_bwd(const Plan &pl, const void *dy, const void *w, void *dx,
                               hipStream_t stream) {
    if (pl.bap.n_blocks <= 0) return hipSuccess;
    if (pl.route_bwd != CONVT_ROUTE_PHASE_GEMM_ALLPHASE || pl.elem_bytes != 2) return hipErrorInvalidValue;
    return pl.dp.f16 ? launch_bwd_allphase_t<_Float16>(pl, dy, w, dx, stream)
                     : launch_bwd_allphase_t<uint16_t>(pl, dy, w, dx, stream);
}

}  // namespace convt
