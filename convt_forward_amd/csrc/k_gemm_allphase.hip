// All-phase implicit-gather GEMM for two-byte inputs with stride 2 on the
// height and width axes (gfx950, one 256-thread block per CU).
//
// Output s*q + r of an axis gathers x[q + off(kk)] * w[kk] over the taps kk
// of residue r (the stride phases), so each phase is a dense correlation over
// q. Here one block computes all four (height, width) residues of a q box for
// 128 output channels and one depth residue: the huggingface
// ai.onnx.ConvTranspose page's grouped stride-phase blocked variant
// (Implementation variants) makes each gathered input serve a whole block of
// outputs, and the same holds here across the phases. Per phase it is the
// implicit GEMM the page describes for stride 1 (Implementation variants),
//     D[co][q] = sum over (tap, ci) of W[g*Cig + ci][co][tap] * x[b][g*Cig+ci][q + off(tap)],
// with x read as zero outside its extents (the implicit padding).
//
// Tile: wave v (0..3) holds the residue pair (rh, rw) = (v / 2, v % 2) as a
// 128 x 128 accumulator tile (128 channels x the 128 positions of the q box,
// 4 x 4 fragments of v_mfma_f32_32x32x16). One K step pairs two of the
// phase's taps: lanes 0-31 carry 8 input channels of the first tap, lanes
// 32-63 the same channels of the second. A pipeline stage covers 8 input
// channels (SC = 8 / TW chunks of them) and every tap of the block's phases.
//
// Operands in LDS, two stage buffers:
//  * weights: for each chunk, [tap slot][128 channels][8 input channels] rows
//    of 16 bytes, slots in W's own tap order (the block's depth taps x all
//    height and width taps). W is read as it is stored: a thread loads 16
//    bytes (8 consecutive taps) from each of 8 input-channel rows of one
//    output channel and transposes the 8 x 8 block of two-byte values in
//    registers with byte permutes into 8 slot rows. No reordered copy of W
//    is made.
//  * input halo: the q box grown by the union of the four phases' tap
//    windows, as 16-byte rows (8 channels of one position). x is
//    channel-planar, so a thread loads 4-byte pairs of neighbouring
//    positions from 8 channels and permutes them into two position rows;
//    the halo's first column and its width are even, so a pair lies in one
//    row of x (the planner requires an even x row length).
//
// Pipeline: buffer loads into registers (out-of-range channels and
// positions read zero through the range check), compiler-visible so its
// wait counts stay exact. Stage s computes from buffer s % 2 in four K steps;
// during them the wave writes stage s+1's halo (loaded two stages earlier)
// and weights (loaded one stage earlier) into buffer (s+1) % 2 and issues
// the loads of stage s+2. The block meets at a barrier before the last K
// step, whose operands are already in registers, so the first operand reads
// of stage s+1 overlap its MFMAs.
//
// Epilogue: acc (started at the bias) + activation, rounded once to the
// element type, written into LDS in output order (the four phases
// interleave into whole output rows), then stored as 16-byte pieces of
// output rows: each wave instruction writes 1 KiB of one output channel.
#include <type_traits>

#include "kcommon.h"
#include "launch.h"

namespace convt {

namespace {

// Row swizzle of weight octet q (of the NP octets a W row contributes): its
// slot rows are stored at row co ^ rot. Consecutive lanes of a 16-byte LDS
// write differ in octet first, then channel; these values keep every 8
// consecutive lanes on distinct 16-byte bank groups modulo 8 and every 16 on
// distinct groups modulo 16 (both for NP = 2 and NP = 4), and stay below 16
// so that a 32-row operand fragment remains one contiguous 32-row group.
template <int NP>
__device__ __forceinline__ int octet_rot(int q) {
    return NP == 2 ? 12 * q : 2 * q + 8 * (q & 1);
}

constexpr int kAPThreads = 256;

}  // namespace

template <typename T, int TW, int MT, bool ACT>
__global__ __launch_bounds__(kAPThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void allphase_gemm_kernel(AllPhaseArgs a, const T *__restrict__ x, const T *__restrict__ w,
                          const T *__restrict__ bias, T *__restrict__ y) {
    constexpr int SC = 8 / TW;         // 8-channel chunks per stage
    constexpr int NPAIR = TW / 2;      // K steps (tap pairs) per chunk
    static_assert(SC * NPAIR == 4, "four K steps per stage");
    static_assert(MT == 4 || MT == 2, "128 x 128 or 64 x 256 wave tiles");
    constexpr int NT = 16 / MT;        // fragments along the positions
    constexpr int BM = 32 * MT;        // output channels per block
    constexpr int BN = 32 * NT;        // q positions per block (each wave holds all of them)
    constexpr int WU = BM / 64;        // weight units (8 channels x 8 taps) per thread and stage
    constexpr int XU = MT == 4 ? 1 : 2;  // halo units (2 positions x 8 channels) per thread and stage
    constexpr int NSLOT = 4 * TW;      // weight taps one chunk brings in (the block's four phases)
    constexpr int WSUB = NSLOT * BM * 16;
    constexpr int WBUF = SC * WSUB;
    constexpr int XROWS = 512 * XU / SC;  // halo rows of one chunk
    constexpr int XSUB = XROWS * 16;
    constexpr int STAGE = WBUF + SC * XSUB;
    constexpr int MAIN = 2 * STAGE;
    constexpr int PITCH = 8 * BN + 16;  // epilogue staging bytes per channel (+16 spreads LDS banks)
    constexpr int EPI = BM * PITCH;
    constexpr int BIAS_OFF = MAIN > EPI ? MAIN : EPI;
    constexpr int SINK = BIAS_OFF + BM * 4;
    using HT = typename std::conditional<std::is_same<T, _Float16>::value, _Float16, __bf16>::type;
    using Frag = typename std::conditional<std::is_same<T, _Float16>::value, f16x8, bf16x8>::type;

    __shared__ __attribute__((aligned(1024))) unsigned char lds[SINK + 32];
    float *bias_s = (float *)(lds + BIAS_OFF);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rh = wave >> 1, rw = wave & 1;  // this wave's height and width residues
    const int kv = lane >> 5;                 // lane half: first or second tap of a K step

    // ---- block coordinates: channel tile fastest, then depth residue, q
    // tiles (width, height, depth), group, batch
    uint32_t bid = (uint32_t)remap_block(blockIdx.x, a.n_blocks, a.xcd_remap);
    uint32_t qq = fast_div(bid, a.div_co);
    const int co_t = (int)(bid - qq * (uint32_t)a.n_co_tiles);
    bid = qq;
    qq = fast_div(bid, a.div_rd);
    const int rd = (int)(bid - qq * (uint32_t)a.n_rd);
    bid = qq;
    qq = fast_div(bid, a.div_t2);
    const int t2 = (int)(bid - qq * (uint32_t)a.nt[2]);
    bid = qq;
    qq = fast_div(bid, a.div_t1);
    const int t1 = (int)(bid - qq * (uint32_t)a.nt[1]);
    bid = qq;
    qq = fast_div(bid, a.div_t0);
    const int t0 = (int)(bid - qq * (uint32_t)a.nt[0]);
    bid = qq;
    qq = fast_div(bid, a.div_g);
    const int g = (int)(bid - qq * (uint32_t)a.G);
    const int b = (int)qq;

    const int T0 = a.T[0], T1 = a.T[1], T2 = a.T[2];
    const int q00 = t0 * T0, q01 = t1 * T1, q02 = t2 * T2;
    const int co0 = co_t * BM;
    const int offd = a.offd[rd];
    const int E0 = T0 + (a.nd - 1) * a.ostep_d, E1 = a.E1, E2 = a.E2, E2p = a.E2p;
    const int npairs = E0 * E1 * (E2 >> 1);  // position pairs of one chunk's halo


    // ---- halo units of this thread: u = tid + 256k (k < XU) is (chunk sc,
    // position pair) with pairs fastest; xoff: byte offset of its 8 channels'
    // first pair in the (batch, group) slice (out of range outside x, or past
    // the halo); xdst: LDS offset of its first row within a stage, or -1 past
    // the halo
    const uint32_t plane2 = (uint32_t)a.x_plane * 2u;
    uint32_t xoff[XU];
    int xdst[XU];
#pragma unroll
    for (int k = 0; k < XU; ++k) {
        const int u = tid + kAPThreads * k;
        xoff[k] = kOutOfRange;
        xdst[k] = -1;
        if (u < SC * npairs) {
            const int sc = u >= npairs ? 1 : 0;
            const int pr = u - sc * npairs;
            const int hp = E2 >> 1;
            const int prh = div_small(pr, hp), cp = pr - prh * hp;
            const int e0 = div_small(prh, E1), e1 = prh - e0 * E1;
            const int row = (e0 * E1 + e1) * E2p + 2 * cp;
            xdst[k] = WBUF + sc * XSUB + row * 16;
            const int i0 = q00 + offd + e0, i1 = q01 + a.uh + e1, i2 = q02 + a.uw + 2 * cp;
            if (i0 >= 0 && i0 < a.I[0] && i1 >= 0 && i1 < a.I[1] && i2 >= 0 && i2 < a.I[2])
                xoff[k] = (uint32_t)((i0 * a.I[1] + i1) * a.I[2] + i2) * 2u + (uint32_t)(sc * 8) * plane2;
        }
    }
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x + ((int64_t)b * a.Ci + (int64_t)g * a.Cig) * a.x_plane,
                                                 (uint32_t)a.Cig * plane2);
    const uint32_t xstage = (uint32_t)(8 * SC) * plane2;  // bytes between stages' channels

    // ---- weight units of this thread: u = tid + 256k (k < WU) is octet j
    // (of the NPAIR 8-tap octets of a W row that the block uses: depth tap
    // jd, octet o of its plane) of output channel co0 + co in chunk sc, octets
    // fastest, so that a wave's loads cover runs of whole rows; the 8 loads of
    // a unit are the 8 input channels of its chunk. In LDS, octet j's slot
    // rows are stored at row co ^ octet_rot(j), spreading the lanes of one
    // write over the LDS banks.
    const int K12 = a.K[1] * a.K[2];
    const int noct = K12 >> 3;  // 8-tap octets of one depth plane
    const uint32_t wrow = (uint32_t)a.Cog * (uint32_t)a.ktot * 2u;  // bytes between input channels
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(w + (int64_t)g * a.Cig * a.Cog * a.ktot, (uint32_t)a.Cig * wrow);
    uint32_t woff[WU];
    int wdst[WU];
#pragma unroll
    for (int k = 0; k < WU; ++k) {
        const int u = tid + kAPThreads * k;
        const int j = u % NPAIR, co = (u / NPAIR) % BM, sc = u / (NPAIR * BM);
        const int jd = j / noct, o = j - jd * noct;
        int kd = a.kd0[rd] - a.kstep_d * jd;
        if (a.flip) kd = a.K[0] - 1 - kd;
        woff[k] = (uint32_t)((co0 + co) * a.ktot + kd * K12 + o * 8) * 2u + (uint32_t)(sc * 8) * wrow;
        wdst[k] = sc * WSUB + (jd * K12 + o * 8) * (BM * 16) + (co ^ octet_rot<NPAIR>(j)) * 16;
    }
    const uint32_t wstage = (uint32_t)(8 * SC) * wrow;

    // ---- MFMA operands. K step i of a stage: chunk i / NPAIR, taps 2p and
    // 2p + 1 (p = i % NPAIR) of this wave's phase, taps in (depth, height,
    // width) order. Per lane half: the slot's byte offset in a chunk's weight
    // tiles and the tap's halo row shift.
    const int nw = a.K[2] >> 1, nh = a.K[1] >> 1;
    int aslot[NPAIR], boff[NPAIR];
#pragma unroll
    for (int p = 0; p < NPAIR; ++p) {
        const int t = 2 * p + kv;
        const int jw = t % nw, jh = (t / nw) % nh, jd = t / (nw * nh);
        int kh = a.kh0[rh] - 2 * jh, kw = a.kw0[rw] - 2 * jw;
        if (a.flip) {
            kh = a.K[1] - 1 - kh;
            kw = a.K[2] - 1 - kw;
        }
        // the slot's rows are swizzled by its octet (slot / 8), within 32-row groups
        const int slot = jd * K12 + kh * a.K[2] + kw;
        aslot[p] = slot * (BM * 16) + (((lane & 31) ^ octet_rot<NPAIR>(slot >> 3)) * 16);
        boff[p] = ((jd * a.ostep_d * E1 + a.offh0[rh] + jh - a.uh) * E2p + a.offw0[rw] + jw - a.uw) * 16;
    }
    // halo row (bytes) of this lane's position n = nt * 32 + fpos for a zero
    // tap shift (fpos: the lane's place in the fragment, frag16_pos for
    // 16-wide boxes, whose halo rows are E2p = 24 apart): the box extents are
    // powers of two with T2 >= 16, so the lane's 5 bits and nt's bits never
    // carry into each other and the row splits into a per-lane part and a
    // wave-uniform part per fragment
    auto halo_row = [&](int n) __attribute__((always_inline)) {
        const int c2 = n & (T2 - 1), c1 = (n >> a.lgT2) & (T1 - 1), c0 = n >> (a.lgT1 + a.lgT2);
        return ((c0 * E1 + c1) * E2p + c2) * 16;
    };
    const int fpos = T2 == 16 ? frag16_pos(lane & 31) : (lane & 31);
    const int brow = halo_row(fpos);
    int bnt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bnt[nt] = __builtin_amdgcn_readfirstlane(halo_row(nt * 32));

    // ---- register stages
    struct WRegs {
        u32x4 v[WU][8];
    };
    struct XRegs {
        uint32_t v[XU][8];
    };
    WRegs WR;
    XRegs X0, X1;
    auto load_w = [&](int k, int c) __attribute__((always_inline)) {
        const uint32_t cs = (uint32_t)c * wstage;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            WR.v[k][e] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, woff[k], cs + (uint32_t)e * wrow, 0));
    };
    auto load_x = [&](XRegs &xr, int k, int c) __attribute__((always_inline)) {
        const uint32_t cs = (uint32_t)c * xstage;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            xr.v[k][e] = __builtin_amdgcn_raw_buffer_load_b32(xrs, xoff[k], cs + (uint32_t)e * plane2, 0);
    };
    // unit k's 8 x 8 block (input channel e holds taps 2j, 2j + 1 in word j)
    // as 8 slot rows (tap t holds channels 2j, 2j + 1 in word j)
    auto store_w = [&](int k, unsigned char *stage) __attribute__((always_inline)) {
        const u32x4 *L = WR.v[k];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int j = t >> 1;
            u32x4 r;
            if (t & 1)
                r = {hi_pair(L[0][j], L[1][j]), hi_pair(L[2][j], L[3][j]), hi_pair(L[4][j], L[5][j]),
                     hi_pair(L[6][j], L[7][j])};
            else
                r = {lo_pair(L[0][j], L[1][j]), lo_pair(L[2][j], L[3][j]), lo_pair(L[4][j], L[5][j]),
                     lo_pair(L[6][j], L[7][j])};
            *(u32x4 *)(stage + wdst[k] + t * (BM * 16)) = r;
        }
    };
    // the pair's two position rows (8 channels each); units past the halo
    // write the sink (a select, not a branch, keeps the K step in one
    // scheduling region)
    auto store_x = [&](const XRegs &xr, int k, unsigned char *stage) __attribute__((always_inline)) {
        const uint32_t *d = xr.v[k];
        const u32x4 r0 = {lo_pair(d[0], d[1]), lo_pair(d[2], d[3]), lo_pair(d[4], d[5]), lo_pair(d[6], d[7])};
        const u32x4 r1 = {hi_pair(d[0], d[1]), hi_pair(d[2], d[3]), hi_pair(d[4], d[5]), hi_pair(d[6], d[7])};
        unsigned char *p0 = xdst[k] >= 0 ? stage + xdst[k] : lds + SINK;
        *(u32x4 *)p0 = r0;
        *(u32x4 *)(p0 + 16) = r1;
    };

    f32x16 acc[MT][NT];
    Frag fa[2][MT], fb[2][NT];
    auto read_frags = [&](Frag (&A)[MT], Frag (&B)[NT], const unsigned char *stage, int i)
        __attribute__((always_inline)) {
        const int sc = i / NPAIR, p = i % NPAIR;
        const unsigned char *wt = stage + sc * WSUB + aslot[p];
        const unsigned char *xt = stage + WBUF + sc * XSUB + boff[p];  // + brow + bnt[nt]
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) A[mt] = __builtin_bit_cast(Frag, *(const u32x4 *)(wt + mt * 512));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) B[nt] = __builtin_bit_cast(Frag, *(const u32x4 *)(xt + brow + bnt[nt]));
    };
    auto mfma = [&](const Frag (&A)[MT], const Frag (&B)[NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if constexpr (std::is_same<T, _Float16>::value)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[mt], B[nt], acc[mt][nt], 0, 0, 0);
                else
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[mt], B[nt], acc[mt][nt], 0, 0, 0);
            }
    };
    // issue order within a K step: each MFMA followed by at most one LDS
    // read, one global load, one LDS write and NV VALU ops
    auto interleave = [&](auto nv) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
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
    // stage s from buffer cur: writes stage s+1 (halo xs, weights in WR) to
    // buffer nxt and loads stage cl = s+2 (halo into xl, weights into WR),
    // one part per K step
    auto stage_body = [&](unsigned char *cur, unsigned char *nxt, const XRegs &xs, XRegs &xl, int cl)
        __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        read_frags(fa[1], fb[1], cur, 1);
        mfma(fa[0], fb[0]);
        store_x(xs, 0, nxt);
        load_x(xl, 0, cl);
        interleave(std::integral_constant<int, 2>{});
        __builtin_amdgcn_sched_barrier(0);
        read_frags(fa[0], fb[0], cur, 2);
        mfma(fa[1], fb[1]);
        store_w(0, nxt);
        load_w(0, cl);
        interleave(std::integral_constant<int, 2>{});
        __builtin_amdgcn_sched_barrier(0);
        read_frags(fa[1], fb[1], cur, 3);
        mfma(fa[0], fb[0]);
        if constexpr (WU == 2) {
            store_w(1, nxt);
            load_w(1, cl);
        } else {
            store_x(xs, 1, nxt);
            load_x(xl, 1, cl);
        }
        interleave(std::integral_constant<int, 2>{});
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        read_frags(fa[0], fb[0], nxt, 0);
        mfma(fa[1], fb[1]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    unsigned char *buf0 = lds, *buf1 = lds + STAGE;
#pragma unroll
    for (int k = 0; k < WU; ++k) load_w(k, 0);
#pragma unroll
    for (int k = 0; k < XU; ++k) load_x(X0, k, 0);
#pragma unroll
    for (int k = 0; k < XU; ++k) load_x(X1, k, 1);
    // the bias of the block's channels, requested behind the first stages'
    // loads through a range-checked load (zero past Cog or without a bias),
    // not a branch, so that nothing waits on it before they are issued
    const __amdgpu_buffer_rsrc_t brs =
        make_rsrc(a.has_bias ? (const void *)(bias + g * a.Cog) : (const void *)bias,
                  a.has_bias ? (uint32_t)a.Cog * 2u : 0u);
    const uint16_t bias_raw = __builtin_amdgcn_raw_buffer_load_b16(
        brs, tid < BM ? (uint32_t)(co0 + tid) * 2u : kOutOfRange, 0, 0);
#pragma unroll
    for (int k = 0; k < WU; ++k) store_w(k, buf0);
#pragma unroll
    for (int k = 0; k < XU; ++k) store_x(X0, k, buf0);
    if (tid < BM) bias_s[tid] = half_to_f32<HT>(bias_raw);
#pragma unroll
    for (int k = 0; k < WU; ++k) load_w(k, 1);
    barrier();
    // the accumulators start at the bias of their output channel (lane l of
    // fragment (mt, nt) holds rows mt*32 + 8*(j/4) + 4*(l/32) + j%4)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float bv = bias_s[mt * 32 + 8 * (j >> 2) + 4 * kv + (j & 3)];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt][j] = bv;
        }
    read_frags(fa[0], fb[0], buf0, 0);
    for (int s = 0; s < a.nstages; s += 2) {
        stage_body(buf0, buf1, X1, X0, s + 2);
        stage_body(buf1, buf0, X0, X1, s + 3);
    }

    // ---- epilogue: every wave has stopped reading the stage buffers once
    // it passes this barrier (the last stage's trailing operand reads
    // included), so they become the staging area
    barrier();
    auto stage_out = [&](auto act_tag) __attribute__((always_inline)) {
        constexpr int A = decltype(act_tag)::value;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n = nt * 32 + fpos;
            const int c2 = n & (T2 - 1), c1 = (n >> a.lgT2) & (T1 - 1), c0 = n >> (a.lgT1 + a.lgT2);
            const int pos = ((c0 * 2 * T1 + 2 * c1 + rh) * 2 * T2 + 2 * c2 + rw) * 2;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int j = 0; j < 16; j += 2) {
                    const int co = mt * 32 + 8 * (j >> 2) + 4 * kv + (j & 3);
                    float v0 = acc[mt][nt][j], v1 = acc[mt][nt][j + 1];
                    if constexpr (A != CONVT_ACT_NONE) {
                        v0 = activate<true>(A, v0);
                        v1 = activate<true>(A, v1);
                    }
                    const uint32_t pk = pack_half2<HT>(v0, v1);
                    *(uint16_t *)(lds + co * PITCH + pos) = (uint16_t)pk;
                    *(uint16_t *)(lds + (co + 1) * PITCH + pos) = (uint16_t)(pk >> 16);
                }
        }
    };
    if constexpr (ACT) {
        switch (a.act) {
            case CONVT_ACT_RELU: stage_out(std::integral_constant<int, CONVT_ACT_RELU>{}); break;
            case CONVT_ACT_SIGMOID: stage_out(std::integral_constant<int, CONVT_ACT_SIGMOID>{}); break;
            case CONVT_ACT_TANH: stage_out(std::integral_constant<int, CONVT_ACT_TANH>{}); break;
            case CONVT_ACT_SILU: stage_out(std::integral_constant<int, CONVT_ACT_SILU>{}); break;
            case CONVT_ACT_GELU: stage_out(std::integral_constant<int, CONVT_ACT_GELU>{}); break;
            default: stage_out(std::integral_constant<int, CONVT_ACT_NONE>{}); break;
        }
    } else {
        stage_out(std::integral_constant<int, CONVT_ACT_NONE>{});
    }
    barrier();

    // ---- stores: per channel the block's outputs are T0 * 2T1 rows of 2T2
    // (a multiple of 32) outputs, 8 * BN bytes in staging order; piece pc (16
    // bytes) of channel co = pc / (BN / 2). Channels past Cog fall outside the store
    // resource (which ends at Cog); rows past the output (or q past the depth
    // residue's count) take the out-of-range offset.
    const uint32_t ypl2 = (uint32_t)a.y_plane * 2u;
    const __amdgpu_buffer_rsrc_t yrs =
        make_rsrc(y + ((int64_t)b * a.Co + (int64_t)g * a.Cog) * a.y_plane, (uint32_t)a.Cog * ypl2);
    const int lgp = a.lgT2 - 2;  // pieces per output row: T2 / 4
    const int qnd = a.qnd[rd];
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {
        const int pc = tid + kAPThreads * i;
        constexpr int LGPC = MT == 4 ? 6 : 7;  // log2 of the pieces per channel, BN / 2
        const int co = pc >> LGPC, rem = pc & ((1 << LGPC) - 1);
        const int row = rem >> lgp, cp = rem & ((1 << lgp) - 1);
        const int c0 = row >> (a.lgT1 + 1), r1 = row & (2 * T1 - 1);
        const int od = a.S0 * (q00 + c0) + rd, oh = 2 * q01 + r1, ow = 2 * q02 + 8 * cp;
        const u32x4 v = *(const u32x4 *)(lds + co * PITCH + rem * 16);
        uint32_t off = kOutOfRange;
        if (q00 + c0 < qnd && oh < a.O[1] && ow < a.O[2])
            off = (uint32_t)(co0 + co) * ypl2 + (uint32_t)((od * a.O[1] + oh) * a.O[2] + ow) * 2u;
        __builtin_amdgcn_raw_buffer_store_b128(v, yrs, off, 0, 0);
    }
}

template <typename T, int TW, int MT>
static hipError_t launch_allphase_t(const Plan &pl, const void *x, const void *w, const void *bias,
                                    void *y, hipStream_t stream) {
    const AllPhaseArgs &a = pl.ap;
    const dim3 grid(a.n_blocks), block(kAPThreads);
    if (a.act != CONVT_ACT_NONE)
        hipLaunchKernelGGL((allphase_gemm_kernel<T, TW, MT, true>), grid, block, 0, stream, a, (const T *)x,
                           (const T *)w, (const T *)bias, (T *)y);
    else
        hipLaunchKernelGGL((allphase_gemm_kernel<T, TW, MT, false>), grid, block, 0, stream, a, (const T *)x,
                           (const T *)w, (const T *)bias, (T *)y);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_allphase_cfg(const Plan &pl, const void *x, const void *w, const void *bias,
                                      void *y, hipStream_t stream) {
    const int tw = pl.ap_tw, mt = pl.ap_mt;
    if (tw == 4 && mt == 4) return launch_allphase_t<T, 4, 4>(pl, x, w, bias, y, stream);
    if (tw == 4 && mt == 2) return launch_allphase_t<T, 4, 2>(pl, x, w, bias, y, stream);
    if (tw == 8 && mt == 4) return launch_allphase_t<T, 8, 4>(pl, x, w, bias, y, stream);
    if (tw == 8 && mt == 2) return launch_allphase_t<T, 8, 2>(pl, x, w, bias, y, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_allphase(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                           hipStream_t stream) {
    if (pl.ap.n_blocks <= 0) return hipSuccess;
    if (pl.route != CONVT_ROUTE_PHASE_GEMM_ALLPHASE || pl.elem_bytes != 2) return hipErrorInvalidValue;
    return pl.dp.f16 ? launch_allphase_cfg<_Float16>(pl, x, w, bias, y, stream)
                     : launch_allphase_cfg<uint16_t>(pl, x, w, bias, y, stream);
}

}  // namespace convt
