// Host planner: validation, output sizes, stride-phase tables, route and tile
// choice, workspace size. Makes no HIP call, so it runs without a GPU.
#include <string.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>
#include <numeric>

#include "convt_internal.h"

namespace convt {

namespace {

int64_t gcd64(int64_t a, int64_t b) { return std::gcd(a, b); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Python-style modulo (result in [0, m)).
int64_t pmod(int64_t a, int64_t m) {
    int64_t r = a % m;
    return r < 0 ? r + m : r;
}

bool mul_ok(int64_t a, int64_t b, int64_t limit, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > limit / a) return false;
    *out = a * b;
    return true;
}

}  // namespace

// Residue r of one axis: outputs s*q + r, q in [0, q_count); taps kk with
// (r + p - kk*d) divisible by s; kk_first is the largest such kk (the first in
// ascending-offset order) and off_first its offset (r + p - kk_first*d) / s.
AxisResidue axis_residue(int64_t I, int64_t K, int64_t S, int64_t P, int64_t D, int64_t O,
                         int64_t r) {
    (void)I;
    AxisResidue a{0, 0, -1, 0};
    a.q_count = r < O ? ceil_div(O - r, S) : 0;
    // Solve kk*d == r + p (mod s) for kk in [0, K).
    const int64_t g = gcd64(S, D);
    const int64_t kstep = S / g;
    int64_t first = -1;
    for (int64_t kk = 0; kk < std::min<int64_t>(K, kstep); ++kk) {
        if (pmod(r + P - kk * D, S) == 0) {
            first = kk;
            break;
        }
    }
    if (first < 0) return a;
    a.n_taps = (K - 1 - first) / kstep + 1;
    a.kk_first = first + (a.n_taps - 1) * kstep;
    a.off_first = (r + P - a.kk_first * D) / S;  // exact
    return a;
}

namespace {

void fill_axis(DevAxis *ax, int64_t I, int64_t K, int64_t S, int64_t P, int64_t D, int64_t O) {
    memset(ax, 0, sizeof(*ax));
    ax->I = (int32_t)I;
    ax->O = (int32_t)O;
    ax->S = (int32_t)S;
    ax->K = (int32_t)K;
    ax->P = (int32_t)P;
    ax->D = (int32_t)D;
    const int64_t g = gcd64(S, D);
    ax->kstep = (int32_t)(S / g);
    ax->ostep = (int32_t)(D / g);
    if (S > kMaxS) return;
    int32_t cum = 0;
    bool any = false;
    for (int64_t r = 0; r < S; ++r) {
        AxisResidue a = axis_residue(I, K, S, P, D, O, r);
        ax->n[r] = (int32_t)a.n_taps;
        ax->cum[r] = cum;
        cum += (int32_t)a.n_taps;
        ax->kk0[r] = (int32_t)a.kk_first;
        ax->off0[r] = (int32_t)a.off_first;
        ax->qn[r] = (int32_t)a.q_count;
        ax->qmax = std::max<int32_t>(ax->qmax, (int32_t)a.q_count);
        if (a.n_taps > 0) {
            const int32_t lo = (int32_t)a.off_first;
            const int32_t hi = (int32_t)(a.off_first + (a.n_taps - 1) * ax->ostep);
            ax->span_max = std::max<int32_t>(ax->span_max, hi - lo);
            ax->umin = any ? std::min(ax->umin, lo) : lo;
            ax->umax = any ? std::max(ax->umax, hi) : hi;
            any = true;
        }
    }
}

// Raw buffer resources address a (batch, group) slice with 32-bit offsets
// and treat offsets >= 2^31 as out of range; every slice must stay below.
bool buffer_fits(int64_t bytes) { return bytes >= 0 && bytes < ((int64_t)1 << 31) - (1 << 20); }

bool slices_fit(const DevParams &dp, int esz) {
    return buffer_fits((int64_t)dp.Cig * dp.x_plane * esz) &&
           buffer_fits((int64_t)dp.Cog * dp.y_plane * esz) &&
           // the reordered weights of a group, with every padding the tile
           // configurations and tap groups can add
           buffer_fits(((int64_t)dp.ktot + 3 * dp.nphase) * (dp.Cog + 255) * (dp.Cig + 63) * esz) &&
           // a (batch, group) slice of the channel-chunked copy of x
           buffer_fits((int64_t)(dp.Cig + 15) * dp.x_plane * 2);
}

bool strides_fit(const DevParams &dp) {
    for (int a = 0; a < 3; ++a)
        if (dp.ax[a].S > kMaxS) return false;
    return dp.ph_tab_ok != 0;
}

// Fill the packed per-phase table (phases in lexicographic residue order).
// Leaves ph_tab_ok = 0 when a phase does not fit the packed fields.
void fill_phase_table(DevParams *dp) {
    dp->ph_tab_ok = 0;
    for (int a = 0; a < 3; ++a)
        if (dp->ax[a].S > kMaxS) return;
    const int64_t np = (int64_t)dp->ax[0].S * dp->ax[1].S * dp->ax[2].S;
    if (np > kMaxPhaseTab) return;
    int P = 0, tapbase = 0;
    for (int r0 = 0; r0 < dp->ax[0].S; ++r0)
        for (int r1 = 0; r1 < dp->ax[1].S; ++r1)
            for (int r2 = 0; r2 < dp->ax[2].S; ++r2, ++P) {
                const int r[3] = {r0, r1, r2};
                PhaseRec &pr = dp->ph[P];
                int ntaps = 1;
                for (int a = 0; a < 3; ++a) {
                    const DevAxis &ax = dp->ax[a];
                    const int n = ax.n[r[a]], qn = ax.qn[r[a]], off = ax.off0[r[a]];
                    if (n >= (1 << 23) || qn >= (1 << 16) || off < -32768 || off > 32767) return;
                    pr.rn[a] = r[a] | (n << 8);
                    pr.qo[a] = (qn & 0xffff) | (int32_t)((uint32_t)(off & 0xffff) << 16);
                    ntaps *= n;
                }
                pr.ntaps = ntaps;
                pr.tapbase = tapbase;
                tapbase += ntaps;
            }
    dp->ph_tab_ok = 1;
}

// ---- phase GEMM tiling ----------------------------------------------------
// A block computes BN positions of one phase for BM output channels. The q
// tile is a (td, th, tw) box with td*th*tw == BN; its input halo grows by the
// tap span of the phase on each axis and must fit the LDS halo buffer.
// Backward data (bwd): the tile is a box of dx positions and its halo in a
// phase plane of dy grows by the phase's tap span (at most span_max); a
// block runs every phase's taps.
bool choose_gemm_tile(DevParams *dp, int ndim, int BN, int halo_max, bool bwd) {
    int64_t best_cost = std::numeric_limits<int64_t>::max();
    int bd = 0, bh = 0, bw = 0;
    for (int tw = 1; tw <= BN; tw *= 2) {
        for (int th = 1; th * tw <= BN; th *= 2) {
            if (BN % (th * tw)) continue;
            const int td = BN / (th * tw);
            if (ndim < 3 && td != 1) continue;
            if (ndim < 2 && th != 1) continue;
            const int64_t hd = td + dp->ax[0].span_max;
            const int64_t hh = th + dp->ax[1].span_max;
            const int64_t hw = tw + dp->ax[2].span_max;
            if (hd * hh * hw > halo_max) continue;
            // the backward kernel packs box coordinates in 10 + 11 + 11 bits
            if (bwd && (hd > 1023 || hh > 2047 || hw > 2047)) continue;
            const int64_t nt = ceil_div(dp->ax[0].qmax, td) * ceil_div(dp->ax[1].qmax, th) *
                               ceil_div(dp->ax[2].qmax, tw);
            // MFMA work of a tile (masked positions included) dominates; halo
            // loads add a smaller term per position, and the epilogue one per
            // output row that 32 consecutive positions (the lanes of one
            // store) touch.
            const int64_t avg_taps =
                bwd ? dp->ktot : std::max<int64_t>(1, dp->ktot / std::max(1, dp->nphase));
            const int64_t rows_per_store = std::max(1, 32 / tw);
            const int64_t cost = nt * (BN * avg_taps * 4 + hd * hh * hw + BN * rows_per_store);
            if (cost < best_cost) {
                best_cost = cost;
                bd = td;
                bh = th;
                bw = tw;
            }
        }
    }
    if (!bw) return false;
    dp->td = bd;
    dp->th = bh;
    dp->tw = bw;
    dp->hd = bd + dp->ax[0].span_max;
    dp->hh = bh + dp->ax[1].span_max;
    dp->hw = bw + dp->ax[2].span_max;
    dp->nt_d = (int32_t)ceil_div(dp->ax[0].qmax, bd);
    dp->nt_h = (int32_t)ceil_div(dp->ax[1].qmax, bh);
    dp->nt_w = (int32_t)ceil_div(dp->ax[2].qmax, bw);
    return true;
}

// Taps per pipeline stage: phases are padded with zero taps to whole
// groups; the model weighs the padded MFMA work against a per-stage overhead
// (barrier, operand refill) of about 0.3 tap.
int choose_gemm_gs(const DevParams &dp) {
    int best_gs = 1;
    double best_cost = 0;
    for (int gs = 1; gs <= tiles::kGemmTapGroup; ++gs) {
        int64_t padded = 0;
        for (int P = 0; P < dp.nphase; ++P) padded += ceil_div(dp.ph[P].ntaps, gs) * gs;
        const double cost = (double)padded * (1.0 + 0.3 / gs);
        if (gs == 1 || cost < best_cost * 0.999) {
            best_gs = gs;
            best_cost = cost;
        }
    }
    return best_gs;
}

// Pick the tile configuration with the smallest modelled time: blocks run in
// rounds of two per CU, each round costing its blocks' padded MFMA work,
// scaled up where the wave tile's LDS operand reads would outrun the MFMAs
// and by a per-MFMA overhead that small wave tiles amortise worse.
int pick_gemm_cfg(DevParams *dp, int dtype, int ndim, bool bwd, int gs, double *t_out);

// Padded tap work of gs taps per stage, with the per-stage overhead of
// choose_gemm_gs.
double tap_work(const DevParams &dp, int gs) {
    int64_t padded = 0;
    for (int P = 0; P < dp.nphase; ++P) padded += ceil_div(dp.ph[P].ntaps, gs) * gs;
    return (double)padded * (1.0 + 0.3 / gs);
}

// Forward: the preferred taps per stage first, then fewer (smaller weight
// buffers leave more LDS to the halo) until some configuration fits.
// Backward data, whose halos are larger: every (taps per stage,
// configuration) pair, by modelled time.
int pick_gemm_cfg(DevParams *dp, int dtype, int ndim, bool bwd) {
    if (!bwd) {
        for (int gs = choose_gemm_gs(*dp); gs >= 1; --gs) {
            const int c = pick_gemm_cfg(dp, dtype, ndim, false, gs, nullptr);
            if (c >= 0) return c;
        }
        return -1;
    }
    int best = -1;
    double best_t = 0;
    DevParams best_dp{};
    for (int gs = tiles::kGemmTapGroup; gs >= 1; --gs) {
        DevParams tmp = *dp;
        double t = 0;
        const int c = pick_gemm_cfg(&tmp, dtype, ndim, true, gs, &t);
        if (c < 0) continue;
        t *= tap_work(*dp, gs);
        if (best < 0 || t < best_t * 0.999) {
            best = c;
            best_t = t;
            best_dp = tmp;
        }
    }
    if (best >= 0) *dp = best_dp;
    return best;
}

int pick_gemm_cfg(DevParams *dp, int dtype, int ndim, bool bwd, int gs, double *t_out) {
    const bool bf16 = dtype == CONVT_DTYPE_BF16 || dtype == CONVT_DTYPE_F16;  // two-byte configs
    int best = -1;
    double best_t = 0;
    DevParams best_dp{};
    for (int c = 0; c < tiles::kGemmCfgCount; ++c) {
        const tiles::GemmTile &t = tiles::kGemmCfg[c];
        if ((t.bf16 != 0) != bf16 || !tiles::gemm_cfg_valid(t, gs)) continue;
        DevParams tmp = *dp;
        if (!choose_gemm_tile(&tmp, ndim, t.bn, tiles::gemm_halo_cap(t, gs), bwd)) continue;
        const int64_t co_tiles = ceil_div(tmp.Cog, t.bm);
        const int64_t blocks = (int64_t)tmp.nt_d * tmp.nt_h * tmp.nt_w * co_tiles *
                               (bwd ? 1 : tmp.nphase) * tmp.G * tmp.B;
        const int wgn = t.nw / t.wgm;
        const double mt = t.bm / t.wgm / 32.0, nt = t.bn / (double)wgn / 32.0;
        // LDS read time over MFMA time per tap (float32 MFMAs take 4x the
        // cycles per byte of operands)
        const double lds_ratio = 0.67 * (mt + nt) / (mt * nt) * (bf16 ? 1.0 : 0.25);
        const double eff = std::max(1.0, lds_ratio) * (1.0 + 0.25 / (mt * nt));
        const double rounds = std::ceil((double)blocks / (256.0 * t.occ));
        // a round's blocks share the CU's SIMDs (nw/4 waves per SIMD each)
        double time = rounds * t.occ * (t.nw / 4.0) * (double)t.bm * t.bn * eff / 2.0;
        // backward data: every stage copies a new halo (a phase plane's box,
        // gathered from dy at stride s) while the weight tiles are contiguous;
        // taller tiles spread each halo copy over more rows (measured: 128 x
        // 128 beats 64 x 256 by 4-7% on the 2-D and 3-D bfloat16 workloads)
        if (bwd) time *= 1.0 + 16.0 / t.bm;
        if (best < 0 || time < best_t * 0.999) {
            best = c;
            best_t = time;
            best_dp = tmp;
        }
    }
    if (best >= 0) {
        *dp = best_dp;
        dp->gemm_cfg = best;
        dp->gemm_gs = gs;
        if (t_out) *t_out = best_t;
    }
    return best;
}

bool gemm_eligible(const DevParams &dp, int dtype, int ndim, bool bwd = false) {
    if (!strides_fit(dp) || dp.ktot > 4096) return false;
    if (!slices_fit(dp, dtype == CONVT_DTYPE_F32 ? 4 : 2)) return false;
    if (dtype != CONVT_DTYPE_F32 && dtype != CONVT_DTYPE_BF16 && dtype != CONVT_DTYPE_F16)
        return false;
    DevParams tmp = dp;
    return pick_gemm_cfg(&tmp, dtype, ndim, bwd) >= 0;
}

// ---- two-byte phase GEMM reading x in NC[D]HW ------------------------------
// Halo extents of phase P for a (T0, T1, T2) box: the box grown by the
// phase's tap span per axis; on the last axis the halo starts at the
// phase's first offset rounded down to even and its width is rounded up to
// even (the kernel reads x in pairs of positions).
int64_t nchw_halo(const DevParams &dp, int P, int T0, int T1, int T2) {
    const PhaseRec &pr = dp.ph[P];
    const int n0 = pr.rn[0] >> 8, n1 = pr.rn[1] >> 8, n2 = pr.rn[2] >> 8;
    const int off2 = pr.qo[2] >> 16;
    const int64_t E0 = T0 + (int64_t)(n0 > 0 ? n0 - 1 : 0) * dp.ax[0].ostep;
    const int64_t E1 = T1 + (int64_t)(n1 > 0 ? n1 - 1 : 0) * dp.ax[1].ostep;
    int64_t E2 = T2 + (int64_t)(n2 > 0 ? n2 - 1 : 0) * dp.ax[2].ostep + (off2 & 1);
    E2 = (E2 + 1) & ~(int64_t)1;
    return E0 * E1 * E2;
}

// ---- all-phase two-byte GEMM -------------------------------------------
FastDiv fast_div_of(uint32_t d) {
    uint32_t s = 0;
    while (((uint64_t)1 << s) < d) ++s;
    const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << s) - d)) / d + 1;
    return FastDiv{(uint32_t)m, s};
}

// Plan the all-phase kernel (k_gemm_allphase.hip) for a forward problem with
// a two-byte element type, or return false if it does not apply: it needs
// stride 2 and dilation 1 on the height and width axes with even kernel
// extents there (every residue then has K/2 taps), the same tap count for
// every depth residue, 4 or 8 taps per phase (a stage is then 8 input
// channels x all taps of the block's four phases, 64 KiB of weights), whole
// 8-tap octets per depth plane of W, W in [C_in][C_out/groups][k...], an
// even x row length (pairs of positions) and an output row length that is
// a multiple of 8 (16-byte output pieces). min_cog: fewer output channels
// per group are left to the other kernels.
bool choose_allphase(Plan *pl, const DevParams &dp, int ndim, int dtype, int64_t min_cog) {
    if (dtype != CONVT_DTYPE_BF16 && dtype != CONVT_DTYPE_F16) return false;
    if (ndim < 2 || dp.w_layout != CONVT_FILTER_CI_CO_K || dp.Cog < min_cog) return false;
    const DevAxis &a0 = dp.ax[0], &a1 = dp.ax[1], &a2 = dp.ax[2];
    if (a1.S != 2 || a2.S != 2 || a1.D != 1 || a2.D != 1 || a1.K % 2 || a2.K % 2) return false;
    if (a0.S > kMaxS) return false;
    const int nd = a0.n[0];
    for (int r = 0; r < a0.S; ++r)
        if (a0.n[r] != nd) return false;
    if (nd < 1) return false;
    const int tw = nd * (a1.K / 2) * (a2.K / 2);
    if (tw != 4 && tw != 8) return false;
    if ((a1.K * a2.K) % 8 != 0 || a2.I % 2 != 0 || a2.O % 8 != 0) return false;
    const int sc = 8 / tw;
    const int64_t cig_span = dp.Cig + 3 * 8 * sc;  // channels the prefetch may address
    if (!buffer_fits(cig_span * dp.x_plane * 2) ||
        !buffer_fits(cig_span * dp.Cog * dp.ktot * 2 + (int64_t)256 * dp.ktot * 2) ||
        !buffer_fits(((int64_t)dp.Cog + 128) * dp.y_plane * 2))  // rows up to a tile past Cog
        return false;
    const int uw = a2.umin & ~1;
    double best = 0;
    int bt[3] = {0, 0, 0}, bmt = 0;
    // wave tiles of 64 channels x 256 positions (mt 2) or 128 x 128 (mt 4);
    // a block holds 32 * mt channels and a q box of 512 / mt positions, and
    // stages up to 512 * (halo units per thread: 2 or 1) / sc halo rows
    for (int mt = 2; mt <= 4; mt += 2) {
        const int bn = 512 / mt, bm = 32 * mt;
        const int64_t rows_cap = 512 * (mt == 4 ? 1 : 2) / sc;
        for (int t2 = 16; t2 <= bn; t2 *= 2) {
            for (int t1 = 1; t1 * t2 <= bn; t1 *= 2) {
                const int t0 = bn / (t1 * t2);
                if (ndim < 3 && t0 != 1) continue;
                const int64_t e0 = t0 + (int64_t)(nd - 1) * a0.ostep;
                const int64_t e1 = t1 + a1.umax - a1.umin;
                const int64_t e2 = (t2 + a2.umax - uw + 1) & ~(int64_t)1;
                // 16-wide boxes: halo rows 24 apart (allphase_halo_pitch)
                if (t2 == 16 && e2 > 24) continue;
                const int64_t rows = e0 * e1 * (t2 == 16 ? 24 : e2);
                if (rows > rows_cap) continue;
                const int64_t nt = ceil_div(a0.qmax, t0) * ceil_div(a1.qmax, t1) * ceil_div(a2.qmax, t2);
                const int64_t blocks = nt * ceil_div(dp.Cog, bm) * a0.S * dp.G * dp.B;
                // one block per CU; a stage: 2048 MFMA cycles per wave, plus
                // the staging of its weights (64 KiB for 128 channels) and
                // halo, which the MFMAs hide only in part
                const double stage = 2048.0 + 8.0 * bm + 2.0 * (double)rows;
                const double t = std::ceil((double)blocks / 256.0) * stage;
                if (bt[2] == 0 || t < best * 0.999) {
                    best = t;
                    bt[0] = t0;
                    bt[1] = t1;
                    bt[2] = t2;
                    bmt = mt;
                }
            }
        }
    }
    if (bt[2] == 0) return false;
    AllPhaseArgs &ap = pl->ap;
    ap = AllPhaseArgs{};
    ap.Ci = dp.Ci;
    ap.Co = dp.Co;
    ap.Cig = dp.Cig;
    ap.Cog = dp.Cog;
    ap.G = dp.G;
    for (int a = 0; a < 3; ++a) {
        ap.I[a] = dp.ax[a].I;
        ap.O[a] = dp.ax[a].O;
        ap.K[a] = dp.ax[a].K;
        ap.T[a] = bt[a];
        ap.nt[a] = (int32_t)ceil_div(dp.ax[a].qmax, bt[a]);
    }
    ap.ktot = dp.ktot;
    ap.lgT1 = __builtin_ctz((unsigned)bt[1]);
    ap.lgT2 = __builtin_ctz((unsigned)bt[2]);
    ap.n_co_tiles = (int32_t)ceil_div(dp.Cog, 32 * bmt);
    ap.n_rd = a0.S;
    const int64_t blocks = (int64_t)ap.nt[0] * ap.nt[1] * ap.nt[2] * ap.n_co_tiles * ap.n_rd * dp.G * dp.B;
    if (blocks > ((int64_t)1 << 31) - 1) return false;
    ap.n_blocks = (int32_t)blocks;
    ap.xcd_remap = blocks % 8 == 0 ? 1 : 0;
    ap.div_co = fast_div_of((uint32_t)ap.n_co_tiles);
    ap.div_rd = fast_div_of((uint32_t)ap.n_rd);
    ap.div_t2 = fast_div_of((uint32_t)ap.nt[2]);
    ap.div_t1 = fast_div_of((uint32_t)ap.nt[1]);
    ap.div_t0 = fast_div_of((uint32_t)ap.nt[0]);
    ap.div_g = fast_div_of((uint32_t)dp.G);
    const int64_t stages = ceil_div(ceil_div(dp.Cig, 8), sc);
    ap.nstages = (int32_t)((stages + 1) / 2 * 2);
    ap.x_plane = dp.x_plane;
    ap.y_plane = dp.y_plane;
    ap.has_bias = dp.has_bias;
    ap.act = dp.act;
    ap.flip = dp.w_flip;
    for (int r = 0; r < 2; ++r) {
        ap.kh0[r] = a1.kk0[r];
        ap.offh0[r] = a1.off0[r];
        ap.kw0[r] = a2.kk0[r];
        ap.offw0[r] = a2.off0[r];
    }
    ap.uh = a1.umin;
    ap.uw = uw;
    ap.E1 = bt[1] + a1.umax - a1.umin;
    ap.E2 = (bt[2] + a2.umax - uw + 1) & ~1;
    ap.E2p = bt[2] == 16 ? 24 : ap.E2;
    ap.S0 = a0.S;
    ap.nd = nd;
    ap.kstep_d = a0.kstep;
    ap.ostep_d = a0.ostep;
    for (int r = 0; r < a0.S; ++r) {
        ap.kd0[r] = a0.kk0[r];
        ap.offd[r] = a0.off0[r];
        ap.qnd[r] = a0.qn[r];
    }
    pl->ap_tw = tw;
    pl->ap_mt = bmt;
    return true;
}

// Choose the kernel's configuration (tiles::kNchwCfg: waves along C_out,
// taps per stage, halo units per thread) and q box for a forward problem
// with a two-byte element type, or return false if the problem does not
// suit it: an odd x row length (pairs of positions must lie within one
// row), phases whose tap counts no configuration takes without padding more
// than a third, at most 64 output channels per group (half of the 128-row
// tiles would be padding) or no box whose halo the per-thread staging holds.
bool choose_nchw(DevParams *dp, int ndim) {
    if (!strides_fit(*dp) || !slices_fit(*dp, 2)) return false;
    if (dp->ax[2].I % 2 != 0 || dp->Cog <= 64) return false;
    // the stores address rows up to 256 past a wave's first channel, and
    // masked positions sit 2^31 out; every such offset stays below 2^32; the
    // input channels are padded to whole pairs of 16-channel chunks
    if (!buffer_fits(((int64_t)dp->Cog + 256) * dp->y_plane * 2)) return false;
    if (!buffer_fits(((int64_t)dp->Cig + 31) * dp->x_plane * 2)) return false;
    int maxt = 0;
    int64_t taps = 0;
    for (int P = 0; P < dp->nphase; ++P) {
        maxt = std::max(maxt, (int)dp->ph[P].ntaps);
        taps += dp->ph[P].ntaps;
    }
    double best = 0;
    int bcfg = -1, bd = 0, bh = 0, bw = 0;
    int64_t bcap = 0;
    for (int c = 0; c < tiles::kNchwCfgCount; ++c) {
        const tiles::NchwCfg &cf = tiles::kNchwCfg[c];
        if (cf.gs < maxt) continue;
        // the padding taps run MFMAs on zero weights: at most a third extra
        if ((int64_t)cf.gs * dp->nphase * 3 > taps * 4) continue;
        const int BN = 4 / cf.wgm * 128;
        const int64_t co_tiles = ceil_div(dp->Cog, 128 * cf.wgm);
        for (int tw = 16; tw <= BN; tw *= 2) {
            for (int th = 1; th * tw <= BN; th *= 2) {
                const int td = BN / (th * tw);
                if (td * th * tw != BN) continue;
                if (ndim < 3 && td != 1) continue;
                if (ndim < 2 && th != 1) continue;
                int64_t cap = 0;
                for (int P = 0; P < dp->nphase; ++P)
                    cap = std::max(cap, nchw_halo(*dp, P, td, th, tw));
                if (cap > (int64_t)256 * cf.xu) continue;
                const int64_t nt = ceil_div(dp->ax[0].qmax, td) * ceil_div(dp->ax[1].qmax, th) *
                                   ceil_div(dp->ax[2].qmax, tw);
                const int64_t blocks = nt * co_tiles * dp->nphase * dp->G * dp->B;
                // blocks run one per CU; a block's time per chunk: its MFMAs
                // (512 cycles per tap per wave, scaled by the rows it holds)
                // plus the halo it stages
                const double rounds = std::ceil((double)blocks / 256.0);
                const double t = rounds * (512.0 * cf.gs * cf.wgm + 2.0 * cap + 300.0) / cf.wgm;
                if (bcfg < 0 || t < best * 0.999) {
                    best = t;
                    bcfg = c;
                    bd = td;
                    bh = th;
                    bw = tw;
                    bcap = cap;
                }
            }
        }
    }
    if (bcfg < 0) return false;
    dp->gemm_nchw = 1;
    dp->nchw_cfg = bcfg;
    dp->nchw_wgm = tiles::kNchwCfg[bcfg].wgm;
    dp->nchw_xcap = (int32_t)bcap;
    dp->gemm_gs = tiles::kNchwCfg[bcfg].gs;
    dp->gemm_cfg = 0;
    dp->td = bd;
    dp->th = bh;
    dp->tw = bw;
    dp->hd = bd + dp->ax[0].span_max;
    dp->hh = bh + dp->ax[1].span_max;
    dp->hw = bw + dp->ax[2].span_max;
    dp->nt_d = (int32_t)ceil_div(dp->ax[0].qmax, bd);
    dp->nt_h = (int32_t)ceil_div(dp->ax[1].qmax, bh);
    dp->nt_w = (int32_t)ceil_div(dp->ax[2].qmax, bw);
    return true;
}

// ---- grouped route tiling -------------------------------------------------
// A block computes every phase of a tile of q rows (qh) at one qd, over the
// full q width, for the Cog channels of one group, and stages the output
// rows in LDS so that they leave as dense rows.
bool choose_grouped_tile(DevParams *dp) {
    const DevAxis &ad = dp->ax[0], &ah = dp->ax[1], &aw = dp->ax[2];
    // the halo covers the union of every phase's input window
    const int64_t span_w = aw.umax - aw.umin;
    const int64_t hw = aw.qmax + span_w;
    const int64_t hd = 1 + (ad.umax - ad.umin);
    // Halo row columns: input position i at column i - pmin, so halo
    // position 0 (input position umin) is at column hshift. The pitch covers
    // every column a 16-position segment reads and, when x rows are whole
    // 8-position (16-byte) chunks that the kernel copies as such, the whole
    // input row; columns of positions outside the row hold zeros. An odd
    // pitch puts the same column of neighbouring rows (and slices) on
    // different LDS banks.
    const int64_t pmin = std::min<int64_t>(aw.umin, 0);
    const int64_t hshift = aw.umin - pmin;
    const int64_t nk = aw.I % 8 == 0 ? aw.I / 8 : 0;
    const int64_t hwp =
        std::max<int64_t>(hshift + ceil_div(aw.qmax, 16) * 16 + span_w, nk ? aw.I - pmin : 0) | 1;
    // Output staging, per wave: a chunk of nsc segments of one output row for
    // every channel of the group (16 * S2 outputs per segment), aiming at
    // 1 KiB per store instruction; rows padded by 16 bytes against bank
    // conflicts.
    const int64_t seg_bytes = 32 * aw.S;
    const int64_t nseg = ceil_div(aw.qmax, 16);
    const int64_t nsc_max = std::min<int64_t>(nseg, 1024 / (std::max(dp->Cog, 1) * seg_bytes));
    const int64_t nsc = nsc_max >= 4 ? 4 : nsc_max >= 2 ? 2 : 1;  // the kernel's unrolled sizes
    const int64_t st_pitch = nsc * seg_bytes + 16;
    // (one more row per wave takes the padding lanes' writes). Width stride
    // 2 with at most 8 channels per group and whole segment pairs needs no
    // staging: the kernel moves a pair's second segment into the padding
    // lanes (DPP) and stores whole 128-byte rows straight from registers.
    const bool pair_dpp = aw.S == 2 && dp->Cog <= 8 && nseg % 2 == 0;
    const int64_t st_bytes =
        pair_dpp ? 0 : (int64_t)tiles::kGrpThreads / 64 * (dp->Cog + 1) * st_pitch;
    auto al = [](int64_t v) { return (v + 15) / 16 * 16; };
    // the group's weights (as W stores them) and the slot table reach LDS by
    // DMA in 1 KiB and 256-byte pieces: their areas are whole pieces. The
    // weight-fragment slab replaces the weights in place: per output channel
    // a row of 16 bytes per slot, an odd number of slots per row (the 16
    // lanes of a fragment read, one channel each, fall on distinct banks)
    const int64_t ns = (int64_t)dp->ktot * (dp->Cig / 8);
    const int64_t slab_bytes = (int64_t)dp->Cog * (ns | 1) * 16;
    const int64_t w_bytes =
        std::max<int64_t>(((int64_t)dp->ktot * dp->Cog * dp->Cig * 2 + 1023) / 1024 * 1024, slab_bytes);
    // slot table: a 16-byte record per phase, then (halo offset, weight
    // offset) per (tap, 8-channel slice)
    const int64_t tab_bytes =
        (16 * (int64_t)dp->nphase + (int64_t)dp->ktot * (dp->Cig / 8) * 8 + 255) / 256 * 256;

    int best = 0;
    int64_t best_halo = 0;
    for (int rows = 1; rows <= 64; rows *= 2) {
        if (rows > ah.qmax && rows > 1) break;
        const int64_t hh = rows + (ah.umax - ah.umin);
        const int64_t halo_bytes = hd * hh * hwp * dp->Cig * 2;
        if (halo_bytes > tiles::kGrpHaloBytes ||
            al(halo_bytes) + al(w_bytes) + al(tab_bytes) + st_bytes > tiles::kGrpLdsBudget)
            break;
        best = rows;
        best_halo = halo_bytes;
        if ((int64_t)rows * aw.qmax >= tiles::kGrpMinPositions) break;
    }
    if (!best || (int64_t)dp->ktot * tiles::kGrpCog * dp->Cig * 2 > tiles::kGrpWBytes) return false;
    // the kernel's grid is (G * B, row tiles, q depths)
    if (ceil_div(ah.qmax, best) > 65535 || ad.qmax > 65535 || (int64_t)dp->G * dp->B > 0x7fffffff)
        return false;
    dp->td = 1;
    dp->th = best;
    dp->tw = aw.qmax;
    dp->hd = (int32_t)hd;
    dp->hh = best + (ah.umax - ah.umin);
    dp->hw = (int32_t)hw;
    dp->grp_hwp = (int32_t)hwp;
    dp->grp_hshift = (int32_t)hshift;
    dp->grp_nk = (int32_t)nk;
    dp->grp_nsc = pair_dpp ? 0 : (int32_t)nsc;  // 0: segment pairs through DPP
    dp->grp_st_pitch = (int32_t)st_pitch;
    dp->nt_d = ad.qmax;
    dp->nt_h = (int32_t)ceil_div(ah.qmax, best);
    dp->nt_w = 1;
    dp->grp_w_off = (int32_t)al(best_halo);
    dp->grp_tab_off = (int32_t)(al(best_halo) + al(w_bytes));
    dp->grp_slab_off = dp->grp_w_off;
    dp->grp_ns = (int32_t)ns;
    dp->grp_st_off = (int32_t)(al(best_halo) + al(w_bytes) + al(tab_bytes));
    dp->grp_lds_bytes = (int32_t)(dp->grp_st_off + st_bytes);
    return true;
}

// The grouped kernel's tables (GrpTables): a record per phase and the (tap,
// slice) slots of each phase in its taps' order, each naming the tap's halo
// window and its weights in the group's part of W as stored (the stored tap
// is the spatially reversed one where W's taps are stored flipped).
bool grouped_tables(Plan *pl) {
    const DevParams &p = pl->dp;
    GrpTables &gt = pl->gt;
    const int noct = p.Cig >> 3;
    if (p.nphase > kMaxPhaseTab || p.ktot > kGrpMaxTaps || 2 * p.nphase + p.ktot * noct > kGrpTabMax)
        return false;
    // element strides of the group's weights: stored tap, input channel,
    // output channel
    int64_t ss, sc, so;
    if (p.w_layout == CONVT_FILTER_K_CI_CO) {  // [k][C_in][Cog]: per tap a [Cig][Cog] run
        ss = (int64_t)p.Cig * p.Cog, sc = p.Cog, so = 1;
    } else if (p.w_layout == CONVT_FILTER_K_CO_CI) {  // [k][C_out][Cig]: per tap a [Cog][Cig] run
        ss = (int64_t)p.Cig * p.Cog, sc = 1, so = p.Cig;
    } else {  // [C_in][Cog][k]: one [Cig][Cog][k] run
        ss = 1, sc = (int64_t)p.Cog * p.ktot, so = p.ktot;
    }
    gt.w_sc = (int32_t)(2 * sc);
    gt.w_so = (int32_t)(2 * so);
    gt.w_tap_pieces = p.w_layout == CONVT_FILTER_CI_CO_K ? 0 : p.Cig * p.Cog / 8;
    const DevAxis &a0 = p.ax[0], &a1 = p.ax[1], &a2 = p.ax[2];
    gt.tab_n = 2 * p.nphase + p.ktot * noct;
    int32_t *slots = gt.tab + 4 * p.nphase;
    for (int P = 0; P < p.nphase; ++P) {
        const PhaseRec &rec = p.ph[P];
        int r[3], n[3], qn[3], off0[3];
        for (int a = 0; a < 3; ++a) {
            r[a] = rec.rn[a] & 0xff;
            n[a] = rec.rn[a] >> 8;
            qn[a] = rec.qo[a] & 0xffff;
            off0[a] = rec.qo[a] >> 16;
        }
        const int nslots = rec.ntaps * noct;
        gt.tab[4 * P + 0] = qn[0];
        gt.tab[4 * P + 1] = qn[1];
        gt.tab[4 * P + 2] = qn[2];
        gt.tab[4 * P + 3] = rec.tapbase * noct | nslots << 16;
        for (int sl = 0; sl < nslots; ++sl) {
            const int tap = sl / noct, oct = sl % noct;
            const int j2 = tap % n[2], j1 = (tap / n[2]) % n[1], j0 = tap / (n[2] * n[1]);
            const int hrow = (off0[0] - a0.umin + j0 * a0.ostep) * p.hh + (off0[1] - a1.umin + j1 * a1.ostep);
            const int col = off0[2] - a2.umin + j2 * a2.ostep + p.grp_hshift;
            // the tap's kernel indices, then its index as W stores it
            const int k0 = a0.kk0[r[0]] - j0 * a0.kstep, k1 = a1.kk0[r[1]] - j1 * a1.kstep,
                      k2 = a2.kk0[r[2]] - j2 * a2.kstep;
            const int st = p.w_flip ? ((a0.K - 1 - k0) * a1.K + (a1.K - 1 - k1)) * a2.K + (a2.K - 1 - k2)
                                    : (k0 * a1.K + k1) * a2.K + k2;
            int32_t *e = slots + 2 * (rec.tapbase * noct + sl);
            e[0] = ((hrow * noct + oct) * p.grp_hwp + col) * 16;
            e[1] = (int32_t)(2 * (st * ss + 8 * oct * sc));
        }
    }
    return true;
}

bool grouped_eligible(const DevParams &dp, int dtype) {
    if ((dtype != CONVT_DTYPE_BF16 && dtype != CONVT_DTYPE_F16) || dp.ktot > 4096) return false;
    if (!slices_fit(dp, 2)) return false;
    if (!strides_fit(dp)) return false;
    if (dp.Cig % 8 != 0 || dp.Cig > 64 || dp.Cog > tiles::kGrpCog) return false;
    if (dp.ax[2].S > tiles::kGrpMaxS2) return false;
    // every phase's K slots (tap x 8-channel slice) fit four MFMA steps
    int64_t max_taps = 1;
    for (int a = 0; a < 3; ++a) {
        int64_t m = 0;
        for (int r = 0; r < dp.ax[a].S; ++r) m = std::max<int64_t>(m, dp.ax[a].n[r]);
        max_taps *= m;
    }
    if (max_taps * (dp.Cig / 8) > 4 * tiles::kGrpMaxKSteps) return false;
    if ((int64_t)dp.ktot * tiles::kGrpCog * dp.Cig * 2 > tiles::kGrpWBytes) return false;
    if (dp.ktot > kGrpMaxTaps || 2 * dp.nphase + dp.ktot * (dp.Cig / 8) > kGrpTabMax) return false;
    // the kernel gathers its group's weights from all of W through one
    // range-checked resource (masked elements take an offset past its end)
    if (!buffer_fits((int64_t)dp.Ci * dp.Cog * dp.ktot * 2)) return false;
    DevParams tmp = dp;
    return choose_grouped_tile(&tmp);
}

bool direct_eligible(const DevParams &dp) {
    if (!strides_fit(dp)) return false;
    const int64_t slab = (int64_t)dp.Cig * dp.Cog * dp.ktot * 4;
    return slab <= tiles::kDirSlabBytes;
}

// The direct backward-data kernel (fp: the forward problem): its LDS holds
// the group's weights, and one buffer resource the group's dy planes.
bool direct_bwd_eligible(const DevParams &fp, int elem_bytes) {
    return tiles::dir_bwd_lds_bytes(fp.Cig, fp.Cog, fp.ktot) <= tiles::kDirBwdLdsBytes &&
           (int64_t)fp.Cog * fp.y_plane * elem_bytes < ((int64_t)1 << 31) && fp.x_plane > 0;
}

// Plan the grouped backward kernel (k_bwd_grouped.hip) for the input
// gradient of a two-byte 2-D problem (fp: the forward problem), or return
// false if it does not apply: output channels per group a multiple of 8 with
// at most 16 (tap, 8-channel slice) slots, at most 16 input channels per
// group, dy rows of whole 16-byte chunks, 32-bit buffer offsets, and the
// direct backward kernel eligible too (it serves calls whose dy or dx is not
// aligned for this one). A tile is R dx rows (a power of two up to 16, about
// 256 dx positions) whose dy halo, weights and fragment slab fit the LDS
// budget and whose halo is at most 256 load units (one per thread).
bool choose_grouped_bwd(Plan *pl, int ndim, int dtype) {
    const DevParams &fp = pl->dp;
    if (dtype != CONVT_DTYPE_BF16 && dtype != CONVT_DTYPE_F16) return false;
    if (ndim != 2) return false;
    const DevAxis &a1 = fp.ax[1], &a2 = fp.ax[2];
    if (fp.Cog < 8 || fp.Cog % 8 != 0 || fp.Cig < 1 || fp.Cig > 16) return false;
    const int64_t noct = fp.Cog / 8, ktot = (int64_t)a1.K * a2.K;
    if (ktot != fp.ktot || ktot * noct > kGbMaxSlots) return false;
    if (a2.O % 8 != 0 || a1.O < 1 || a1.I < 1 || a2.I < 1) return false;
    if (!direct_bwd_eligible(fp, 2)) return false;
    if (!buffer_fits((int64_t)fp.Cog * fp.y_plane * 2) || !buffer_fits((int64_t)fp.Cig * fp.x_plane * 2) ||
        !buffer_fits((int64_t)fp.Ci * fp.Cog * fp.ktot * 2))
        return false;
    // halo columns: every column a dx row's taps read and all of dy's row
    // (staged as whole chunks) after the P2 zero columns. With width stride
    // 2 the even and odd columns go to separate halves, so that the 16
    // lanes of an A fragment (dx positions 2 columns apart) read consecutive
    // cells; the pitch of a (halo row, slice) stays odd.
    const int64_t hwr =
        std::max<int64_t>((int64_t)a2.S * (a2.I - 1) + (int64_t)a2.D * (a2.K - 1) + 1, (int64_t)a2.P + a2.O);
    const int64_t sp = a2.S == 2 ? 2 : 1;
    const int64_t hp = sp == 1 ? (hwr | 1) : (hwr + 1) / 2;
    const int64_t hwp = sp == 1 ? hp : 2 * hp + 1;
    auto cell = [&](int64_t c) { return (c & (sp - 1)) * hp + (c >> (sp - 1)); };
    // the group's W as stored (whole 1 KiB pieces), then the fragment slab
    const int64_t w_bytes = ((int64_t)fp.Cig * fp.Cog * ktot * 2 + 1023) / 1024 * 1024 + 16 * kGbSlabPitch;
    auto halo_rows = [&](int64_t r) { return (int64_t)a1.S * (r - 1) + (int64_t)a1.D * (a1.K - 1) + 1; };
    auto halo_bytes = [&](int64_t r) { return halo_rows(r) * noct * hwp * 16; };
    // halo load units (row, slice, 8-position chunk): one per thread
    auto units = [&](int64_t r) { return halo_rows(r) * noct * (a2.O / 8); };
    int64_t R = 1;
    while (R < 16 && 2 * R * a2.I <= 256 && 2 * R <= a1.I) R *= 2;
    while (R > 1 && (halo_bytes(R) + w_bytes > kGbLdsBudget || units(R) > 256)) R /= 2;
    if (halo_bytes(R) + w_bytes > kGbLdsBudget || units(R) > 256) return false;
    const int64_t nt_h = ceil_div(a1.I, R);
    if (nt_h > 65535 || (int64_t)fp.G * fp.B > 0x7fffffff) return false;
    GrpBwdArgs &g = pl->gb;
    memset(&g, 0, sizeof(g));
    g.G = fp.G; g.Ci = fp.Ci; g.Co = fp.Co; g.Cig = fp.Cig; g.Cog = fp.Cog; g.noct = (int32_t)noct;
    g.I1 = a1.I; g.I2 = a2.I; g.O1 = a1.O; g.O2 = a2.O;
    g.S1 = a1.S; g.S2 = a2.S; g.P1 = a1.P; g.P2 = a2.P; g.D1 = a1.D; g.D2 = a2.D;
    g.K1 = a1.K; g.K2 = a2.K; g.ktot = (int32_t)ktot;
    g.nslots = (int32_t)(ktot * noct);
    g.ks = (g.nslots + 3) / 4;
    g.R = (int32_t)R; g.nt_h = (int32_t)nt_h; g.B = fp.B;
    if ((int64_t)fp.G * fp.B * nt_h > 0x7fffffff) return false;
    g.hr = (int32_t)halo_rows(R); g.hwp = (int32_t)hwp;
    g.hwr = (int32_t)hwr; g.hp = (int32_t)hp; g.sp = (int32_t)sp;
    g.x_plane = fp.x_plane; g.y_plane = fp.y_plane;
    g.w_off = (int32_t)halo_bytes(R);
    g.slab_off = (int32_t)(halo_bytes(R) + w_bytes - 16 * kGbSlabPitch);
    g.lds_bytes = (int32_t)(halo_bytes(R) + w_bytes);
    // element strides of the group's weights: stored tap, input channel,
    // output channel
    int64_t ss, sci, sco;
    if (fp.w_layout == CONVT_FILTER_K_CI_CO) {  // [k][C_in][Cog]: per tap a [Cig][Cog] run
        ss = (int64_t)fp.Cig * fp.Cog, sci = fp.Cog, sco = 1;
    } else if (fp.w_layout == CONVT_FILTER_K_CO_CI) {  // [k][C_out][Cig]: per tap a [Cog][Cig] run
        ss = (int64_t)fp.Cig * fp.Cog, sci = 1, sco = fp.Cig;
    } else {  // [C_in][Cog][k]: one [Cig][Cog][k] run
        ss = 1, sci = (int64_t)fp.Cog * ktot, sco = ktot;
    }
    g.w_sci = (int32_t)(2 * sci);
    g.w_sco = (int32_t)(2 * sco);
    g.w_tap_pieces = fp.w_layout == CONVT_FILTER_CI_CO_K ? 0 : fp.Cig * fp.Cog / 8;
    for (int slot = 0; slot < g.nslots; ++slot) {
        const int t = slot / (int)noct, oct = slot % (int)noct;
        const int kh = t / a2.K, kw = t % a2.K;
        const int st = fp.w_flip ? (a1.K - 1 - kh) * a2.K + (a2.K - 1 - kw) : kh * a2.K + kw;
        g.slot_w[slot] = (int32_t)(2 * (st * ss + 8 * oct * sco));
        g.slot_h[slot] = (int32_t)(((a1.D * kh * noct + oct) * hwp + cell((int64_t)a2.D * kw)) * 16);
    }
    return true;
}

// Plan the backward all-phase kernel (k_bwd_allphase.hip) for the input
// gradient of a two-byte problem (fp: the forward problem), or return false
// if it does not apply: W in the C_in x C_out x taps layout; stride 2 and
// dilation 1 on the height and width axes with even tap counts there and 16
// taps over the two; an even dy row length (a 4-byte pair of dy positions
// lies in one row), dx rows of whole 16-byte pieces; 32-bit buffer offsets
// (dy up to 32 channels past the group, for the stages the pipeline loads
// ahead); at least min_cig dx channels per group. The box is one depth
// position x T1 x T2 = 256 positions (128 with the K split) whose four
// phase-plane halos fit the kernel's planes.
bool choose_bwd_allphase(Plan *pl, int ndim, int dtype, int64_t min_cig) {
    const DevParams &fp = pl->dp;
    if (dtype != CONVT_DTYPE_BF16 && dtype != CONVT_DTYPE_F16) return false;
    if (ndim < 2 || fp.w_layout != CONVT_FILTER_CI_CO_K || fp.Cig < min_cig || fp.Cig < 1 || fp.Cog < 1)
        return false;
    const DevAxis &a0 = fp.ax[0], &a1 = fp.ax[1], &a2 = fp.ax[2];
    if (a1.S != 2 || a2.S != 2 || a1.D != 1 || a2.D != 1 || a1.K % 2 || a2.K % 2 || a1.K * a2.K != 16)
        return false;
    if (a2.O % 2 != 0 || a2.I % 8 != 0 || a1.I < 1 || a0.I < 1) return false;
    if (!buffer_fits(((int64_t)fp.Cog + 32) * fp.y_plane * 2) ||
        !buffer_fits((int64_t)fp.Cig * fp.Cog * fp.ktot * 2) || !buffer_fits((int64_t)fp.Cig * fp.x_plane * 2))
        return false;
    // per axis: tap k = 2m + c reads plane residue (c - p) mod 2 at index
    // i + m + floor((c - p) / 2); tmin = floor(-p / 2) (the c = 0 value)
    auto floor_half = [](int64_t v) { return v >= 0 ? v / 2 : -((1 - v) / 2); };
    BwdAPArgs &ba = pl->bap;
    ba = BwdAPArgs{};
    const DevAxis *hw[2] = {&a1, &a2};
    int32_t tmin[2], r[2][2], u[2][2];
    for (int x = 0; x < 2; ++x) {
        const int64_t p = hw[x]->P;
        tmin[x] = (int32_t)floor_half(-p);
        for (int c = 0; c < 2; ++c) {
            r[x][c] = (int32_t)pmod(c - p, 2);
            u[x][c] = (int32_t)(floor_half(c - p) - tmin[x]);
        }
    }
    // the box and the K split: a block per CU (256 CUs) and per stage about
    // 2048 MFMA cycles per wave plus ~1000 of staging, or with the K split
    // (128-position boxes, two wave pairs sharing a stage's K steps) 1024 +
    // ~730; among equal times the smaller halo
    const int64_t n_ci = ceil_div(fp.Cig, 128), per_img = (int64_t)a0.I * n_ci * fp.G * fp.B;
    int T1 = 0, T2 = 0, KS = 0;
    int64_t E1 = 0, E2 = 0;
    double best = 0;
    for (int ks = 0; ks <= 1; ++ks) {
        const int bn = ks ? 128 : 256;
        for (int t2 = 16; t2 <= 64; t2 *= 2) {
            const int t1 = bn / t2;
            const int64_t e1 = t1 + a1.K / 2 - 1 + u[0][1], e2 = t2 + a2.K / 2 - 1 + u[1][1];
            if (e1 * e2 > (ks ? kBwdPlaneRowsKS : kBwdPlaneRows)) continue;
            const int64_t blocks = ceil_div(a1.I, t1) * ceil_div(a2.I, t2) * per_img;
            const double t = std::ceil((double)blocks / 256.0) * (ks ? 1760.0 : 3050.0);
            if (T2 == 0 || t < best * 0.999 || (t <= best * 1.001 && e1 * e2 < E1 * E2)) {
                T1 = t1;
                T2 = t2;
                E1 = e1;
                E2 = e2;
                KS = ks;
                best = t;
            }
        }
    }
    if (T2 == 0) return false;
    ba.Ci = fp.Ci;
    ba.Co = fp.Co;
    ba.Cig = fp.Cig;
    ba.Cog = fp.Cog;
    ba.G = fp.G;
    for (int a = 0; a < 3; ++a) {
        ba.I[a] = fp.ax[a].I;
        ba.O[a] = fp.ax[a].O;
        ba.K[a] = fp.ax[a].K;
    }
    ba.ktot = fp.ktot;
    ba.T1 = T1;
    ba.T2 = T2;
    ba.lgT2 = __builtin_ctz((unsigned)T2);
    ba.E1 = (int32_t)E1;
    ba.E2 = (int32_t)E2;
    ba.ksplit = KS;
    ba.n_ci_tiles = (int32_t)ceil_div(fp.Cig, 128);
    ba.nt[0] = a0.I;
    ba.nt[1] = (int32_t)ceil_div(a1.I, T1);
    ba.nt[2] = (int32_t)ceil_div(a2.I, T2);
    const int64_t blocks = (int64_t)ba.nt[0] * ba.nt[1] * ba.nt[2] * ba.n_ci_tiles * fp.G * fp.B;
    if (blocks < 1 || blocks > ((int64_t)1 << 31) - 1) return false;
    ba.n_blocks = (int32_t)blocks;
    ba.xcd_remap = blocks % 8 == 0 ? 1 : 0;
    ba.div_ci = fast_div_of((uint32_t)ba.n_ci_tiles);
    ba.div_t2 = fast_div_of((uint32_t)ba.nt[2]);
    ba.div_t1 = fast_div_of((uint32_t)ba.nt[1]);
    ba.div_t0 = fast_div_of((uint32_t)ba.nt[0]);
    ba.div_g = fast_div_of((uint32_t)fp.G);
    const int64_t stages = ceil_div(fp.Cog, 8) * a0.K;
    if (stages > ((int64_t)1 << 30)) return false;
    ba.nstages = (int32_t)((stages + 1) / 2 * 2);
    ba.div_k0 = fast_div_of((uint32_t)a0.K);
    ba.x_plane = fp.x_plane;
    ba.y_plane = fp.y_plane;
    ba.flip = fp.w_flip;
    ba.S0 = a0.S;
    ba.P0 = a0.P;
    ba.D0 = a0.D;
    ba.tmin1 = tmin[0];
    ba.tmin2 = tmin[1];
    for (int c = 0; c < 2; ++c) {
        ba.r1[c] = r[0][c];
        ba.u1[c] = u[0][c];
        ba.r2[c] = r[1][c];
        ba.u2[c] = u[1][c];
    }
    return true;
}

}  // namespace

// ---- backward data ---------------------------------------------------------
// dx[i] gathers dy[s*i - p + kk*d] * W[kk]. Output residue r of the forward
// split holds the taps whose products land on dy positions s*j + r, at
// j = i - off(kk): per phase, a stride-1 correlation of the phase plane
// dy_r[j] = dy[s*j + r] with the phase's taps, and dx is the sum over the
// phases. The backward GEMM runs these sums in one K loop per block.
convt_status plan_backward(Plan *pl, const int64_t I[3], const int64_t K[3], const int64_t S[3],
                           const int64_t P[3], const int64_t D[3], const int64_t O[3]) {
    const convt_problem *p = &pl->prob;
    const DevParams &fp = pl->dp;
    DevParams &b = pl->bdp;
    memset(&b, 0, sizeof(b));
    for (int a = 0; a < 3; ++a) fill_axis(&b.ax[a], I[a], K[a], S[a], P[a], D[a], O[a]);
    fill_phase_table(&b);
    // The input is dy (ax.I = O), the output dx (ax.O = qmax = I); span_max
    // stays the widest phase's tap span.
    for (int a = 0; a < 3; ++a) {
        DevAxis &ax = b.ax[a];
        ax.I = (int32_t)O[a];
        ax.O = (int32_t)I[a];
        ax.qmax = (int32_t)I[a];
    }
    b.B = fp.B;
    b.Ci = fp.Co;
    b.Co = fp.Ci;
    b.G = fp.G;
    b.Cig = fp.Cog;
    b.Cog = fp.Cig;
    b.ktot = fp.ktot;
    b.nphase = fp.nphase;
    b.x_plane = fp.y_plane;
    b.y_plane = fp.x_plane;
    b.has_bias = 0;
    b.w_layout = fp.w_layout;
    b.w_flip = fp.w_flip;
    b.act = CONVT_ACT_NONE;
    b.f16 = fp.f16;
    const int dt = p->dtype;
    const int nd = pl->ndim;
    const bool empty_out = b.B == 0 || b.Co == 0 || b.y_plane == 0;
    const bool no_terms = b.Cig == 0;
    int route = p->route_bwd;
    if (route == CONVT_ROUTE_AUTO) {
        if (empty_out)
            route = CONVT_ROUTE_NONE;
        else if (no_terms)
            route = CONVT_ROUTE_FILL;
        else if (choose_grouped_bwd(pl, nd, dt))
            route = CONVT_ROUTE_GROUPED;
        else if (direct_bwd_eligible(fp, pl->elem_bytes) && (fp.Cig < 32 || fp.Cog < 16))
            // few channels: the backward GEMM's tiles (64 dx channels, chunks
            // of 16 dy channels) would be mostly padding
            route = CONVT_ROUTE_DIRECT;
        else if (choose_bwd_allphase(pl, nd, dt, 65))
            route = CONVT_ROUTE_PHASE_GEMM_ALLPHASE;
        else if (gemm_eligible(b, dt, nd, true))
            route = CONVT_ROUTE_PHASE_GEMM;
        else if (direct_bwd_eligible(fp, pl->elem_bytes))
            route = CONVT_ROUTE_DIRECT;
        else
            route = CONVT_ROUTE_NAIVE;
    } else {
        bool ok = false;
        switch (route) {
            case CONVT_ROUTE_NONE: ok = empty_out; break;
            case CONVT_ROUTE_FILL: ok = !empty_out && no_terms; break;
            case CONVT_ROUTE_PHASE_GEMM:
                ok = !empty_out && !no_terms && gemm_eligible(b, dt, nd, true);
                break;
            case CONVT_ROUTE_PHASE_GEMM_ALLPHASE:
                ok = !empty_out && !no_terms && choose_bwd_allphase(pl, nd, dt, 1);
                break;
            case CONVT_ROUTE_DIRECT:
                ok = !empty_out && !no_terms && direct_bwd_eligible(fp, pl->elem_bytes);
                break;
            case CONVT_ROUTE_GROUPED: ok = !empty_out && !no_terms && choose_grouped_bwd(pl, nd, dt); break;
            case CONVT_ROUTE_NAIVE: ok = !empty_out && !no_terms; break;
            default: ok = false;
        }
        if (!ok) return CONVT_ERR_UNSUPPORTED;
    }
    pl->route_bwd = route;
    pl->info.route_bwd = route;
    pl->info.bwd_workspace_bytes = 0;
    if (route != CONVT_ROUTE_PHASE_GEMM) return CONVT_OK;  // the all-phase kernel needs no workspace

    const int64_t i31 = ((int64_t)1 << 31) - 1, lim = (int64_t)1 << 62;
    pick_gemm_cfg(&b, dt, nd, true);
    const tiles::GemmTile &t = tiles::kGemmCfg[b.gemm_cfg];
    const int64_t bk = 32 / pl->elem_bytes * t.sc;  // K channels (of dy) per stage
    b.cog_pad = (int32_t)(ceil_div(b.Cog, t.bm) * t.bm);
    b.cig_pad = (int32_t)(ceil_div(b.Cig, bk) * bk);
    b.wr_chunked = 1;
    int64_t base = 0, stages = 0;
    b.bwd_nlive = 0;
    for (int ph = 0; ph < b.nphase; ++ph) {
        const int64_t ng = ceil_div(b.ph[ph].ntaps, b.gemm_gs);
        b.ph[ph].tapbase = (int32_t)base;
        base += ng * b.gemm_gs;
        stages += ng * (b.cig_pad / bk);
        if (ng > 0) b.bwd_live[b.bwd_nlive++] = (uint8_t)ph;
    }
    if (base > i31 || stages > i31) return CONVT_ERR_UNSUPPORTED;
    b.ktot_pad = (int32_t)base;
    b.bwd_nstages = (int32_t)stages;
    b.n_co_tiles = (int32_t)ceil_div(b.Cog, t.bm);
    const int64_t blocks = (int64_t)b.nt_d * b.nt_h * b.nt_w * b.n_co_tiles * b.G * b.B;
    if (blocks > i31) return CONVT_ERR_UNSUPPORTED;
    b.n_blocks = (int32_t)blocks;
    b.xcd_remap = blocks % 8 == 0 ? 1 : 0;
    int64_t wr, tmp, ws;
    if (!mul_ok((int64_t)b.G * b.ktot_pad, (int64_t)b.cog_pad * b.cig_pad, lim, &wr))
        return CONVT_ERR_INVALID_ARGUMENT;
    pl->bwd_wr_elems = wr;
    ws = wr * pl->elem_bytes;
    pl->bwd_tab_offset = (ws + 255) / 256 * 256;
    ws = pl->bwd_tab_offset + (int64_t)b.ktot_pad * 4;
    if (dt != CONVT_DTYPE_F32) {
        // the channel-chunked copy of dy: [B][G][chunk][position][32 bytes]
        int64_t xp;
        if (!mul_ok((int64_t)b.B * b.G, (int64_t)b.cig_pad / 16, lim, &tmp) ||
            !mul_ok(tmp, (int64_t)b.x_plane * 32, lim, &xp))
            return CONVT_ERR_INVALID_ARGUMENT;
        pl->bwd_xp_offset = (ws + 255) / 256 * 256;
        pl->bwd_xp_bytes = xp;
        ws = pl->bwd_xp_offset + xp;
    }
    pl->info.bwd_workspace_bytes = ws;
    return CONVT_OK;
}

convt_status make_plan(const convt_problem *p, Plan *pl) {
    memset(pl, 0, sizeof(*pl));
    if (!p) return CONVT_ERR_INVALID_ARGUMENT;
    pl->prob = *p;
    const int nd = p->ndim;
    if (nd < 1 || nd > CONVT_MAX_NDIM) return CONVT_ERR_INVALID_ARGUMENT;
    if (p->has_bias != 0 && p->has_bias != 1) return CONVT_ERR_INVALID_ARGUMENT;
    if (p->route < CONVT_ROUTE_AUTO || p->route > CONVT_ROUTE_PHASE_GEMM_ALLPHASE)
        return CONVT_ERR_INVALID_ARGUMENT;
    if (p->has_padding_hi != 0 && p->has_padding_hi != 1) return CONVT_ERR_INVALID_ARGUMENT;
    if (p->filter_layout < CONVT_FILTER_CI_CO_K || p->filter_layout > CONVT_FILTER_K_CO_CI ||
        (p->taps_flipped != 0 && p->taps_flipped != 1))
        return CONVT_ERR_INVALID_ARGUMENT;
    if (p->activation < CONVT_ACT_NONE || p->activation > CONVT_ACT_GELU || p->reserved1 != 0)
        return CONVT_ERR_INVALID_ARGUMENT;
    if (p->route_bwd < CONVT_ROUTE_AUTO || p->route_bwd > CONVT_ROUTE_PHASE_GEMM_ALLPHASE)
        return CONVT_ERR_INVALID_ARGUMENT;
    const int64_t B = p->x_shape[0], Ci = p->x_shape[1];
    const int64_t G = p->groups;
    if (B < 0 || Ci < 0 || G < 1) return CONVT_ERR_INVALID_ARGUMENT;
    if (p->w_shape[0] != Ci || p->w_shape[1] < 0) return CONVT_ERR_INVALID_ARGUMENT;
    if (Ci % G != 0) return CONVT_ERR_INVALID_ARGUMENT;
    const int64_t Cog = p->w_shape[1];
    const int64_t Cig = Ci / G;
    const int64_t lim = (int64_t)1 << 62;
    int64_t Co;
    if (!mul_ok(Cog, G, lim, &Co)) return CONVT_ERR_INVALID_ARGUMENT;

    int64_t I[3] = {1, 1, 1}, K[3] = {1, 1, 1}, S[3] = {1, 1, 1}, P[3] = {0, 0, 0},
            D[3] = {1, 1, 1}, OP[3] = {0, 0, 0}, O[3] = {1, 1, 1};
    const int lead = 3 - nd;
    for (int j = 0; j < nd; ++j) {
        const int a = lead + j;
        I[a] = p->x_shape[2 + j];
        K[a] = p->w_shape[2 + j];
        S[a] = p->stride[j];
        P[a] = p->padding[j];
        // the high padding only shortens the axis: the kernels see the low
        // padding P and the output size O
        const int64_t PH = p->has_padding_hi ? p->padding_hi[j] : P[a];
        D[a] = p->dilation[j];
        OP[a] = p->output_padding[j];
        if (I[a] < 0 || K[a] < 1 || S[a] < 1 || P[a] < 0 || PH < 0 || D[a] < 1 || OP[a] < 0)
            return CONVT_ERR_INVALID_ARGUMENT;
        if (OP[a] >= std::max(S[a], D[a])) return CONVT_ERR_INVALID_ARGUMENT;
        // sizes are bounded so that the output-size arithmetic cannot overflow
        if (I[a] > ((int64_t)1 << 31) || K[a] > ((int64_t)1 << 20) || S[a] > ((int64_t)1 << 20) ||
            D[a] > ((int64_t)1 << 20) || P[a] > ((int64_t)1 << 40) || PH > ((int64_t)1 << 40))
            return CONVT_ERR_INVALID_ARGUMENT;
        O[a] = (I[a] - 1) * S[a] - (P[a] + PH) + D[a] * (K[a] - 1) + OP[a] + 1;
        if (O[a] < 1) return CONVT_ERR_INVALID_ARGUMENT;
    }
    // The kernels index an axis in 32-bit arithmetic: an output position o
    // reaches the input through o + p - kk*d (from -d(k-1) up to
    // (I-1)s + d(k-1) + op), and each residue's first input offset is
    // (r + p - kk*d)/s. Problems whose terms do not fit are valid but not
    // served.
    for (int j = 0; j < nd; ++j) {
        const int a = lead + j;
        const int64_t PH = p->has_padding_hi ? p->padding_hi[j] : P[a];
        const int64_t lim30 = (int64_t)1 << 30;
        if (P[a] > lim30 || PH > lim30 || D[a] * (K[a] - 1) > lim30 ||
            (I[a] > 0 ? (I[a] - 1) * S[a] : 0) + D[a] * (K[a] - 1) + std::max(S[a], D[a]) >= ((int64_t)1 << 31))
            return CONVT_ERR_UNSUPPORTED;
    }
    if (p->dtype < CONVT_DTYPE_F32 || p->dtype > CONVT_DTYPE_I64)
        return CONVT_ERR_INVALID_ARGUMENT;
    if (p->dtype != CONVT_DTYPE_F32 && p->dtype != CONVT_DTYPE_BF16 && p->dtype != CONVT_DTYPE_F16)
        return CONVT_ERR_UNSUPPORTED;

    // element counts
    int64_t xpl = I[0], ypl = O[0], ktot = K[0], nph = S[0], t;
    for (int a = 1; a < 3; ++a) {
        if (!mul_ok(xpl, I[a], lim, &xpl) || !mul_ok(ypl, O[a], lim, &ypl) ||
            !mul_ok(ktot, K[a], lim, &ktot) || !mul_ok(nph, S[a], lim, &nph))
            return CONVT_ERR_INVALID_ARGUMENT;
    }
    int64_t xn, yn, wn;
    if (!mul_ok(B, Ci, lim, &t) || !mul_ok(t, xpl, lim, &xn)) return CONVT_ERR_INVALID_ARGUMENT;
    if (!mul_ok(B, Co, lim, &t) || !mul_ok(t, ypl, lim, &yn)) return CONVT_ERR_INVALID_ARGUMENT;
    if (!mul_ok(Ci, Cog, lim, &t) || !mul_ok(t, ktot, lim, &wn)) return CONVT_ERR_INVALID_ARGUMENT;
    const int64_t i31 = ((int64_t)1 << 31) - 1;
    if (xpl > i31 || ypl > i31 || ktot > i31) return CONVT_ERR_INVALID_ARGUMENT;
    if (B > i31 || Ci > i31 || Co > i31) return CONVT_ERR_INVALID_ARGUMENT;
    (void)xn;
    (void)wn;

    pl->ndim = nd;
    pl->elem_bytes = p->dtype == CONVT_DTYPE_F32 ? 4 : 2;
    convt_plan_info &info = pl->info;
    info.out_shape[0] = B;
    info.out_shape[1] = Co;
    for (int j = 0; j < nd; ++j) info.out_shape[2 + j] = O[lead + j];
    info.c_out = Co;
    info.n_phases = nph;
    {
        // 2 * B * C_in * Cog * prod(k) * prod(I), saturating
        long double f = 2.0L * B * Ci * Cog * ktot * xpl;
        info.useful_flops = f > (long double)INT64_MAX ? INT64_MAX : (int64_t)f;
    }

    DevParams &dp = pl->dp;
    for (int a = 0; a < 3; ++a) fill_axis(&dp.ax[a], I[a], K[a], S[a], P[a], D[a], O[a]);
    fill_phase_table(&dp);
    dp.B = (int32_t)B;
    dp.Ci = (int32_t)Ci;
    dp.Co = (int32_t)Co;
    dp.G = (int32_t)G;
    dp.Cig = (int32_t)Cig;
    dp.Cog = (int32_t)Cog;
    dp.ktot = (int32_t)ktot;
    dp.nphase = nph > i31 ? i31 : (int32_t)nph;
    dp.x_plane = (int32_t)xpl;
    dp.y_plane = (int32_t)ypl;
    dp.has_bias = p->has_bias;
    dp.w_layout = p->filter_layout;
    dp.w_flip = p->taps_flipped;
    dp.act = p->activation;
    dp.f16 = p->dtype == CONVT_DTYPE_F16;

    // ---- route ------------------------------------------------------------
    const bool empty_out = (B == 0 || Co == 0);
    const bool no_terms = (Cig == 0 || xpl == 0);
    int route = p->route;
    const int dt = p->dtype;
    if (route == CONVT_ROUTE_AUTO) {
        if (empty_out)
            route = CONVT_ROUTE_NONE;
        else if (no_terms)
            route = CONVT_ROUTE_FILL;
        else if (grouped_eligible(dp, dt) && (G > 1 || Cog <= 16))
            route = CONVT_ROUTE_GROUPED;
        else if (direct_eligible(dp) && (Cig * ktot <= 64 || Cog <= 4))
            route = CONVT_ROUTE_DIRECT;
        else if (gemm_eligible(dp, dt, nd))
            route = CONVT_ROUTE_PHASE_GEMM;
        else if (direct_eligible(dp))
            route = CONVT_ROUTE_DIRECT;
        else
            route = CONVT_ROUTE_NAIVE;
    } else {
        // A forced route must be able to serve the problem.
        bool ok = false;
        switch (route) {
            case CONVT_ROUTE_NONE: ok = empty_out; break;
            case CONVT_ROUTE_FILL: ok = !empty_out && no_terms; break;
            case CONVT_ROUTE_PHASE_GEMM: ok = !empty_out && !no_terms && gemm_eligible(dp, dt, nd); break;
            case CONVT_ROUTE_PHASE_GEMM_PACKED:
                ok = !empty_out && !no_terms && dt != CONVT_DTYPE_F32 && gemm_eligible(dp, dt, nd);
                break;
            case CONVT_ROUTE_PHASE_GEMM_ALLPHASE:
                ok = !empty_out && !no_terms && choose_allphase(pl, dp, nd, dt, 1);
                break;
            case CONVT_ROUTE_GROUPED: ok = !empty_out && !no_terms && grouped_eligible(dp, dt); break;
            case CONVT_ROUTE_DIRECT: ok = !empty_out && !no_terms && direct_eligible(dp); break;
            case CONVT_ROUTE_NAIVE: ok = !empty_out && !no_terms; break;
            default: ok = false;
        }
        if (!ok) return CONVT_ERR_UNSUPPORTED;
    }
    pl->route = route;
    info.route = route;

    // ---- tiles and workspace ------------------------------------------------
    // two-byte problems that the all-phase kernel serves go to it
    if (p->route == CONVT_ROUTE_AUTO && route == CONVT_ROUTE_PHASE_GEMM && choose_allphase(pl, dp, nd, dt, 65))
        route = CONVT_ROUTE_PHASE_GEMM_ALLPHASE;
    if (route == CONVT_ROUTE_PHASE_GEMM_ALLPHASE) {
        pl->route = route;
        info.route = route;
        pl->wr_elems = 0;
        info.workspace_bytes = 0;
        return plan_backward(pl, I, K, S, P, D, O);
    }
    int64_t blocks = 0;
    // the two-byte GEMM reads x in place when the problem suits that kernel
    if (route == CONVT_ROUTE_PHASE_GEMM && dt != CONVT_DTYPE_F32 && !choose_nchw(&dp, nd))
        route = CONVT_ROUTE_PHASE_GEMM_PACKED;
    pl->route = route;
    info.route = route;
    if (route == CONVT_ROUTE_PHASE_GEMM && dp.gemm_nchw) {
        const int bm = 128 * dp.nchw_wgm;
        dp.cog_pad = (int32_t)(ceil_div(Cog, bm) * bm);
        // whole pairs of 16-channel chunks (the kernel runs two per loop trip)
        dp.cig_pad = (int32_t)(ceil_div(Cig, 32) * 32);
        dp.wr_chunked = 1;
        {
            // each phase's taps padded to gemm_gs (one stage per chunk)
            int64_t base = 0;
            for (int P = 0; P < dp.nphase; ++P) {
                dp.ph[P].tapbase = (int32_t)base;
                base += ceil_div(dp.ph[P].ntaps, dp.gemm_gs) * dp.gemm_gs;
            }
            if (base > i31) return CONVT_ERR_UNSUPPORTED;
            dp.ktot_pad = (int32_t)base;
        }
        dp.n_co_tiles = (int32_t)ceil_div(Cog, bm);
        blocks = (int64_t)dp.nt_d * dp.nt_h * dp.nt_w * dp.n_co_tiles * nph * G * B;
    } else if (route == CONVT_ROUTE_PHASE_GEMM || route == CONVT_ROUTE_PHASE_GEMM_PACKED) {
        pick_gemm_cfg(&dp, dt, nd, false);
        const tiles::GemmTile &t = tiles::kGemmCfg[dp.gemm_cfg];
        // channels of a stage: SC chunks of 32 bytes
        const int64_t bk = 32 / pl->elem_bytes * t.sc;
        dp.cog_pad = (int32_t)(ceil_div(Cog, t.bm) * t.bm);
        dp.cig_pad = (int32_t)(ceil_div(Cig, bk) * bk);
        dp.wr_chunked = 1;
        {
            // each phase's taps padded to whole groups of gemm_gs
            int64_t base = 0;
            for (int P = 0; P < dp.nphase; ++P) {
                dp.ph[P].tapbase = (int32_t)base;
                base += ceil_div(dp.ph[P].ntaps, dp.gemm_gs) * dp.gemm_gs;
            }
            if (base > i31) return CONVT_ERR_UNSUPPORTED;
            dp.ktot_pad = (int32_t)base;
        }
        dp.n_co_tiles = (int32_t)ceil_div(Cog, t.bm);
        blocks = (int64_t)dp.nt_d * dp.nt_h * dp.nt_w * dp.n_co_tiles * nph * G * B;
    } else if (route == CONVT_ROUTE_GROUPED) {
        choose_grouped_tile(&dp);
        {
            // MFMA K steps of the widest phase, rounded up to 1, 2 or 4
            int64_t ks = 1;
            for (int P = 0; P < dp.nphase; ++P) {
                const int64_t need = (dp.ph[P].ntaps * (Cig / 8) + 3) / 4;
                while (ks < need) ks *= 2;
            }
            dp.grp_ksteps = (int32_t)ks;
        }
        dp.cog_pad = tiles::kGrpCog;
        dp.cig_pad = (int32_t)Cig;
        dp.n_co_tiles = 1;
        blocks = (int64_t)dp.nt_d * dp.nt_h * G * B;
        if (!grouped_tables(pl)) return CONVT_ERR_UNSUPPORTED;
    }
    if (blocks > i31) return CONVT_ERR_UNSUPPORTED;
    dp.n_blocks = (int32_t)blocks;
    // the grouped kernel runs a 3-D grid in plain order
    dp.xcd_remap = (blocks % 8 == 0 && route != CONVT_ROUTE_GROUPED) ? 1 : 0;
    const bool gemm = route == CONVT_ROUTE_PHASE_GEMM || route == CONVT_ROUTE_PHASE_GEMM_PACKED;
    // (the grouped kernel reads W as stored and takes its tables with its
    // arguments: no workspace)
    if (gemm) {
        int64_t wr;
        const int64_t taps = dp.ktot_pad;
        if (!mul_ok((int64_t)G * taps, (int64_t)dp.cog_pad * dp.cig_pad, lim, &wr))
            return CONVT_ERR_INVALID_ARGUMENT;
        pl->wr_elems = wr;
        info.workspace_bytes = wr * pl->elem_bytes;
        // the per-tap halo shift table (int32 per padded tap of a group)
        pl->tab_offset = (info.workspace_bytes + 255) / 256 * 256;
        info.workspace_bytes = pl->tab_offset + (int64_t)dp.ktot_pad * 4;
        if (route == CONVT_ROUTE_PHASE_GEMM_PACKED) {
            // the channel-chunked copy of x: [B][G][chunk][position][32 bytes]
            int64_t xp;
            if (!mul_ok(B * G, (int64_t)dp.cig_pad / 16, lim, &t) || !mul_ok(t, xpl * 32, lim, &xp))
                return CONVT_ERR_INVALID_ARGUMENT;
            pl->xp_offset = (info.workspace_bytes + 255) / 256 * 256;
            pl->xp_bytes = xp;
            info.workspace_bytes = pl->xp_offset + xp;
        }
    } else {
        pl->wr_elems = 0;
        info.workspace_bytes = 0;
    }
    return plan_backward(pl, I, K, S, P, D, O);
}

}  // namespace convt
