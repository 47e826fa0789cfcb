// Internal plan structures shared by the host planner, the C ABI and the
// kernels. Plain data only (no HIP types), so the planner builds and runs
// without a GPU.
#pragma once

#include <stdint.h>

#include "convt.h"

namespace convt {

// Largest per-axis stride the phase-table routes take (the kernels carry one
// table row per output residue). Larger strides go to the naive route.
constexpr int kMaxS = 16;

// Stride-phase table of one spatial axis.
//
// The scatter y[i*s - p + kk*d] += x[i] * w[kk] splits by output residue
// r = o mod s: output s*q + r receives x[q + off] * w[kk] for the taps kk with
// (r + p - kk*d) divisible by s, off = (r + p - kk*d) / s. Those taps form an
// arithmetic progression with step kstep = s / gcd(s, d); along it the offset
// moves by ostep = d / gcd(s, d). Taps are kept in ascending offset order,
// i.e. descending kk: the tap-reversed orientation of the weights.
struct DevAxis {
    int32_t I, O, S, K, P, D;
    int32_t kstep, ostep;
    int32_t qmax;        // largest q_count over residues
    int32_t span_max;    // largest (n - 1) * ostep over residues
    int32_t umin, umax;  // smallest / largest input offset over all residues (union window)
    int32_t n[kMaxS];    // taps of residue r
    int32_t cum[kMaxS];  // taps of residues < r
    int32_t kk0[kMaxS];  // first tap of residue r in plan order (its largest kk)
    int32_t off0[kMaxS]; // input offset of that tap (the residue's smallest)
    int32_t qn[kMaxS];   // q_count of residue r: outputs s*q + r with q < qn
};

// One stride phase, packed so that a kernel fetches it with a single 32-byte
// scalar load: per axis, rn = residue | taps << 8 and qo = q_count (low 16
// bits) | first input offset << 16 (signed); then the phase's tap count and
// the index of its first tap in the reordered weights.
constexpr int kMaxPhaseTab = 64;
struct PhaseRec {
    int32_t rn[3];
    int32_t qo[3];
    int32_t ntaps, tapbase;
};

// Everything a kernel needs, passed by value. Axis 0 is depth, 1 height,
// 2 width; problems of rank < 3 get leading unit axes (I = O = K = S = D = 1,
// P = 0), which leave the sums unchanged.
struct DevParams {
    DevAxis ax[3];
    int32_t B, Ci, Co, G, Cig, Cog;
    int32_t cig_pad, cog_pad;  // padded extents of the reordered weights
    int32_t ktot;              // prod(K): taps over all phases
    int32_t nphase;            // prod(S)
    int32_t x_plane, y_plane;  // spatial elements of one x / y channel plane
    int32_t has_bias;
    int32_t w_layout;          // convt_filter_layout of W
    int32_t w_flip;            // 1: W's taps are stored spatially reversed
    int32_t act;               // convt_activation of the forward output
    int32_t f16;               // two-byte elements are IEEE half (else bfloat16)
    // Tiling of the main kernel (meaning depends on the route).
    int32_t td, th, tw;        // q-tile extents
    int32_t hd, hh, hw;        // halo box extents (largest over phases)
    int32_t nt_d, nt_h, nt_w;  // tiles per axis
    int32_t n_co_tiles;
    int32_t n_blocks;          // grid of the main kernel
    int32_t xcd_remap;         // 1: block ids remapped so each XCD takes a contiguous range
    int32_t grp_w_off, grp_tab_off, grp_lds_bytes;  // grouped route: LDS layout (bytes)
    int32_t grp_hwp;           // grouped route: halo row pitch in 16-byte cells (>= hw)
    int32_t grp_hshift;        // grouped route: pitch column of halo position 0
    int32_t grp_nk;            // grouped route: 8-position chunks of an x row (0: rows are
                               // not whole chunks); chunk k sits at column 8k + hshift - umin
    int32_t grp_nsc;           // grouped route: q segments (16 positions) per staged chunk
                               // (0: segment pairs leave through DPP, no staging)
    int32_t grp_slab_off;      // grouped route: LDS offset (bytes) of the weight-fragment slab
                               // [Cog][slot (pitch grp_ns | 1)][8 input channels]
    int32_t grp_ns;            // grouped route: (tap, 8-channel slice) slots of all phases
    int32_t grp_st_off;        // grouped route: LDS offset (bytes) of the per-wave output staging
    int32_t grp_st_pitch;      // grouped route: staging bytes per channel (chunk bytes + 16)
    int32_t grp_ksteps;        // grouped route: MFMA K steps per phase (1, 2 or 4)
    int32_t gemm_cfg;          // phase GEMM: index into tiles::kGemmCfg
    int32_t gemm_gs;           // phase GEMM: taps per pipeline stage (1..kGemmTapGroup)
    int32_t wr_chunked;        // 1: the route reorders W into [g][tap][chunk][co][32 B] (0: W read as stored)
    int32_t ktot_pad;          // taps per group in the reordered weights (phase GEMM: each
                               // phase padded with zero taps to a multiple of gemm_gs)
    int32_t ph_tab_ok;         // 1: ph[] holds every phase (nphase <= kMaxPhaseTab)
    int32_t gemm_nchw;         // phase GEMM: 1 = two-byte kernel reading x in NC[D]HW directly
    int32_t nchw_cfg;          // ... its configuration (tiles::kNchwCfg)
    int32_t nchw_wgm;          // ... its waves along the output channels (1: 128 rows, 2: 256)
    int32_t nchw_xcap;         // ... halo positions one LDS halo buffer holds
    int32_t bwd_nstages;       // backward-data GEMM: pipeline stages of a block (all phases)
    int32_t bwd_nlive;         // backward-data GEMM: phases with taps
    uint8_t bwd_live[kMaxPhaseTab];  // their indices, ascending
    PhaseRec ph[kMaxPhaseTab];
};

// Division by a run-time constant d >= 1 for every 32-bit dividend n:
// n / d = (mulhi(n, m) + n) >> s in 33-bit arithmetic, with s = ceil(log2 d)
// and m = floor(2^32 (2^s - d) / d) + 1 (the round-up multiplier of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).
struct FastDiv {
    uint32_t m, s;
};

// All-phase GEMM (two-byte types; stride 2 and dilation 1 on the height and
// width axes): a block computes every (height, width) residue of a q box for
// 128 output channels and one depth residue, reading x in NC[D]HW and W in
// [C_in][C_out/groups][k...] directly. Axes as in DevParams (0 depth, 1
// height, 2 width; unit depth for 2-D problems).
struct AllPhaseArgs {
    int32_t Ci, Co, Cig, Cog, G;
    int32_t I[3], O[3], K[3];
    int32_t ktot;               // K0 * K1 * K2
    int32_t T[3];               // q box (T0 * T1 * T2 = 128; T1, T2 powers of two, T2 >= 16)
    int32_t lgT1, lgT2;
    int32_t n_co_tiles, n_rd;   // 128-channel tiles; depth residues
    int32_t n_blocks, xcd_remap;
    FastDiv div_co, div_rd, div_t2, div_t1, div_t0, div_g;  // block-index decode
    int32_t nt[3];              // q tiles per axis
    int32_t nstages;            // pipeline stages (chunk groups), even
    int32_t x_plane, y_plane;
    int32_t has_bias, act, flip;
    // height / width: the taps of residue r are k = k0[r] - 2j at input
    // offset off0[r] + j (j < K/2); the halo starts at offset uh (height)
    // and uw (width, even) from the q box and spans E1 x E2 positions (E2
    // even), its rows E2p apart in LDS (24 for 16-wide boxes, else E2)
    int32_t kh0[2], offh0[2], kw0[2], offw0[2];
    int32_t uh, uw, E1, E2, E2p;
    // depth: residue rd's taps are k = kd0[rd] - kstep_d j at input offset
    // offd[rd] + ostep_d j (j < nd, the same count for every residue); its q
    // count is qnd[rd]
    int32_t S0, nd, kstep_d, ostep_d;
    int32_t kd0[kMaxS], offd[kMaxS], qnd[kMaxS];
};

// Backward data on the all-phase kernel (two-byte types; stride 2, dilation
// 1 and an even tap count on the height and width axes, 16 taps over the
// two): a block computes 128 dx channels x a box of one depth position and
// T1 x T2 = 256 positions (128 with the K split: the waves then share each
// stage's K steps in two pairs), its K loop running over (8-channel chunk of
// dy, depth tap) stages of all 16 height x width taps.
constexpr int kBwdPlaneRows = 383;    // halo rows per phase plane, at most (one more row absorbs idle units)
constexpr int kBwdPlaneRowsKS = 255;  // ... with the K split (a 128-position box)
// route_bwd GROUPED (k_bwd_grouped.hip): the input gradient of a 2-D grouped
// problem with few channels, as a strided correlation of dy on MFMA. A block
// owns one (batch, group) and R dx rows over the full dx width; dy's halo for
// those rows goes to LDS as 16-byte cells of 8 dy channels
// [halo row][slice][column].
constexpr int kGbMaxSlots = 16;     // (tap, 8-channel dy slice) slots: four MFMA K steps
constexpr int kGbLdsBudget = 28672;  // LDS per block (halo + weights + fragment slab)
constexpr int kGbSlabPitch = 17 * 16; // bytes per input channel in the fragment slab
struct GrpBwdArgs {
    int32_t G, Ci, Co, Cig, Cog, noct;  // the forward problem's channels; noct = Cog / 8
    int32_t I1, I2, O1, O2;             // dx and dy extents (height, width)
    int32_t S1, S2, P1, P2, D1, D2;     // stride, low padding, dilation
    int32_t K1, K2, ktot, nslots, ks;   // taps; slots = ktot * noct; K steps
    int32_t R, nt_h, B;                 // dx rows per tile, row tiles, batch; tiles =
                                        // G * B * nt_h, row tiles fastest, groups slowest
    int32_t hr, hwp;                    // halo rows, pitch of a (halo row, slice) in cells (odd)
    int32_t hwr, hp, sp;                // halo columns; with width stride 2 (sp = 2) the even
                                        // columns take cells 0 .. hp-1 and the odd ones hp ..,
                                        // column c at cell (c % sp) * hp + c / sp; else sp = 1
    int32_t x_plane, y_plane;           // dx and dy plane elements
    int32_t w_off, slab_off, lds_bytes; // LDS: halo from 0, W from w_off, the fragment
                                        // slab [input channel][17 slots][16 B] from slab_off
    int32_t w_sci, w_sco, w_tap_pieces; // W as stored: bytes between input / output
                                        // channels of a group; 16-byte pieces per tap
                                        // when taps are outermost, else 0
    int32_t slot_w[kGbMaxSlots];        // per slot: byte offset of its stored tap and
                                        // slice's first output channel in the group's W
    int32_t slot_h[kGbMaxSlots];        // per slot: halo byte offset of the tap for dx
                                        // row 0, position 0
};

struct BwdAPArgs {
    int32_t Ci, Co, Cig, Cog, G;  // the forward problem's channels: dx has Ci (groups of Cig), dy Co
    int32_t I[3], O[3], K[3];     // dx extents, dy extents, taps
    int32_t ktot;
    int32_t T1, T2, lgT2;         // the box (powers of two, T1 * T2 = 256, or 128 with ksplit)
    int32_t E1, E2;               // halo rows of one phase plane: E1 x E2 <= kBwdPlaneRows(KS)
    int32_t ksplit;               // 1: 128-position box, the K steps split between wave pairs
    int32_t n_ci_tiles;           // 128-channel tiles of Cig
    int32_t nt[3];                // boxes per axis (nt[0] = I[0]: one depth position per box)
    int32_t n_blocks, xcd_remap;
    FastDiv div_ci, div_t2, div_t1, div_t0, div_g;  // block-index decode
    int32_t nstages;              // ceil(Cog / 8) * K[0], rounded up to even
    FastDiv div_k0;               // stage -> (chunk, depth tap)
    int32_t x_plane, y_plane;     // dx plane (I0 I1 I2), dy plane (O0 O1 O2)
    int32_t flip;
    int32_t S0, P0, D0;           // depth: dx position i reads dy depth S0*i - P0 + kd*D0
    // height / width: tap k = 2m + c reads the dy phase plane of residue
    // r[c] (positions 2j + r[c]) at j = i + tmin + m + u[c]; the halo of a
    // box starting at i0 covers j in [i0 + tmin, i0 + tmin + E)
    int32_t tmin1, tmin2;
    int32_t r1[2], u1[2], r2[2], u2[2];
};

// Grouped route: the kernel's slot table, built by the planner and passed
// with the kernel's arguments (the kernel copies it to LDS together with its
// group's weights as W stores them, and reads its weight fragments there).
constexpr int kGrpTabMax = 2 * kMaxPhaseTab + 64;  // int2 entries: 2 per phase, then the slots
constexpr int kGrpMaxTaps = 64;                    // taps of the grouped route (its weight slab bound)
static_assert(kGrpTabMax <= 256, "the grouped kernel's table fits one 4-byte copy per lane of 8 waves");
struct GrpTables {
    int32_t tab_n;                    // int2 entries used
    int32_t tab[2 * kGrpTabMax];      // per phase an int4 record (q counts; first slot | slot
                                      // count << 16), then per (tap, 8-channel slice) slot the
                                      // halo byte offset of the tap's window and the byte offset
                                      // in the group's weights (as stored) of the tap's first
                                      // channel of the slice, output channel 0
    int32_t w_sc, w_so;               // bytes between consecutive input / output channels of
                                      // the group's weights as stored
    int32_t w_tap_pieces;             // 16-byte pieces per tap when W stores the group's
                                      // weights tap by tap (taps outermost), else 0 (one run)
};

struct Plan {
    convt_problem prob;
    convt_plan_info info;
    DevParams dp;
    int32_t ndim;
    int32_t route;
    int64_t wr_elems;   // elements of the reordered weights (workspace, from offset 0)
    int64_t tab_offset; // phase GEMM: byte offset of the per-tap halo shift table (int32 per tap)
    int64_t xp_offset;  // bfloat16 phase GEMM: byte offset of the channel-chunked copy of x
    int64_t xp_bytes;   // its size (0 when not used)
    int32_t elem_bytes; // 4 (float32) or 2 (bfloat16)
    GrpTables gt;       // CONVT_ROUTE_GROUPED: the kernel's tables
    AllPhaseArgs ap;    // CONVT_ROUTE_PHASE_GEMM_ALLPHASE: the kernel's arguments
    int32_t ap_tw;      // ... taps per phase and chunk (4 or 8)
    int32_t ap_mt;      // ... 32-channel fragments per wave (4: 128 x 128 wave tiles, 2: 64 x 256)
    // Backward data. bdp is the problem as the backward kernels see it: the
    // input is dy (ax[a].I = O, channels Co in groups of Cog), the output is
    // dx (ax[a].O = I, channels Ci in groups of Cig); the axes keep the
    // forward's stride-phase tables (residues, taps, offsets).
    int32_t route_bwd;
    DevParams bdp;
    int64_t bwd_wr_elems;    // elements of the backward-reordered weights (offset 0)
    int64_t bwd_tab_offset;  // byte offset of the per-tap halo shift table
    int64_t bwd_xp_offset;   // bfloat16: byte offset of the channel-chunked copy of dy
    int64_t bwd_xp_bytes;    // its size (0 when not used)
    BwdAPArgs bap;           // route_bwd PHASE_GEMM_ALLPHASE: the kernel's arguments
    GrpBwdArgs gb;           // route_bwd GROUPED: the kernel's arguments
};

// Tile constants of the kernels, shared with the planner so that it sizes
// grids and halos the way the kernels expect.
namespace tiles {
// Phase GEMM: tile configurations. A block has nw waves (4: two blocks
// share a CU and cover each other's barrier waits; one 8-wave block per CU
// measured slower, its waves all meeting at every barrier), laid out as
// WGM x nw/WGM; each wave holds
// a 32-aligned sub-tile of the BM output channels x BN positions. A K chunk
// is 32 bytes of input channels (16 bfloat16 or 8 float32); a pipeline stage
// covers SC consecutive chunks and gs (1..4) taps. The weight tiles of a
// stage stream through a ring of kGemmWRing LDS buffers of 32-byte rows; the
// input halo of SC chunks (HALO positions at most) streams through a ring of
// xb buffers that share the rest of the block's LDS budget (20 KiB per wave:
// a CU's 160 KiB over its 8 resident waves):
// bfloat16 as one 32-byte row per position (from the channel-chunked copy of
// x), float32 as one row of 4-byte elements per channel (straight from x).
struct GemmTile {
    int bm, bn, wgm, bf16, sc, xb;  // xb: halo ring buffers (3: two groups in flight, 2: one)
    int nw;                         // waves per block (4 or 8)
    int occ;                        // blocks per CU the LDS budget and registers allow (2 or 4)
};
// A CU's 160 KiB of LDS shared by its resident blocks.
constexpr int kGemmLdsPerCU = 160 * 1024;
constexpr int kGemmTapGroup = 4;   // taps per pipeline stage, at most (the planner picks 1..4)
constexpr int kGemmWRing = 3;      // weight-tile buffers: two stages in flight
constexpr int kGemmWRowBytes = 32; // weight row: one chunk of channels
constexpr int kGemmCfgCount = 7;
constexpr GemmTile kGemmCfg[kGemmCfgCount] = {
    {128, 256, 1, 1, 1, 3, 4, 2},  // 0: bf16, waves 128 x 64
    {64, 256, 1, 1, 1, 3, 4, 2},   // 1: bf16, waves 64 x 64
    {128, 128, 1, 1, 1, 3, 4, 2},  // 2: bf16, waves 128 x 32
    {64, 256, 1, 0, 1, 3, 4, 2},   // 3: f32, waves 64 x 64
    {64, 128, 1, 0, 2, 3, 4, 2},   // 4: f32, waves 64 x 32, two chunks per stage
    {128, 128, 1, 0, 1, 3, 4, 2},  // 5: f32, waves 128 x 32
    {128, 256, 1, 1, 1, 2, 4, 2},  // 6: bf16, waves 128 x 64, larger halos (3-D tiles)
};
constexpr int gemm_lds_budget(const GemmTile &t) { return kGemmLdsPerCU / t.occ; }
constexpr int gemm_chunk_ch(const GemmTile &t) { return t.bf16 ? 16 : 8; }
// one stage's weight tiles
constexpr int gemm_wbuf_bytes(const GemmTile &t, int gs) {
    return t.sc * gs * t.bm * kGemmWRowBytes;
}
// bytes available to the halo of one chunk in one ring slot
constexpr int gemm_xsub_avail(const GemmTile &t, int gs) {
    return (gemm_lds_budget(t) - kGemmWRing * gemm_wbuf_bytes(t, gs)) / t.xb / t.sc;
}
// halo positions one chunk's buffer holds: bfloat16 in whole 1 KiB pieces of
// 32 rows, float32 in whole pieces of 64 positions per channel row
constexpr int gemm_halo_cap(const GemmTile &t, int gs) {
    return t.bf16 ? gemm_xsub_avail(t, gs) / 1024 * 32 : (gemm_xsub_avail(t, gs) / 8 - 32) / 4 / 64 * 64;
}
// float32 halo: byte stride of a channel row (padded by 32 bytes so that the
// two halves of a wave, reading rows 4 apart, fall on different LDS banks)
constexpr int gemm_xrow_bytes(const GemmTile &t, int gs) { return gemm_halo_cap(t, gs) * 4 + 32; }
// one chunk's halo buffer
constexpr int gemm_xsub_bytes(const GemmTile &t, int gs) {
    return t.bf16 ? gemm_halo_cap(t, gs) / 32 * 1024 : gemm_chunk_ch(t) * gemm_xrow_bytes(t, gs);
}
// whether a configuration can run with gs taps per stage (its halo buffers
// hold at least one copy piece)
constexpr bool gemm_cfg_valid(const GemmTile &t, int gs) {
    return gemm_halo_cap(t, gs) >= (t.bf16 ? 32 : 64);
}
constexpr int gemm_lds_bytes(const GemmTile &t, int gs) {
    return kGemmWRing * gemm_wbuf_bytes(t, gs) + t.xb * t.sc * gemm_xsub_bytes(t, gs);
}
static_assert(gemm_lds_bytes(kGemmCfg[0], 4) <= gemm_lds_budget(kGemmCfg[0]), "LDS");
static_assert(gemm_lds_bytes(kGemmCfg[2], 4) <= gemm_lds_budget(kGemmCfg[2]), "LDS");
static_assert(gemm_lds_bytes(kGemmCfg[3], 4) <= gemm_lds_budget(kGemmCfg[3]), "LDS");
static_assert(gemm_lds_bytes(kGemmCfg[5], 4) <= gemm_lds_budget(kGemmCfg[5]), "LDS");

static_assert(gemm_halo_cap(kGemmCfg[0], 4) >= 256 && gemm_halo_cap(kGemmCfg[5], 4) >= 128,
              "halo buffers hold at least the tile");
// Two-byte phase GEMM reading x directly (k_gemm_nchw.hip): four waves of
// 128 x 128 accumulators, WGM of them along the output channels; a stage is
// one 16-channel chunk with all GS taps of the phase. LDS: two stages of
// weight tiles [GS][128 * WGM][32 bytes], two halo buffers of xcap rows of
// 32 bytes, and the block's bias in float32. A thread stages at most
// kNchwMaxUnits halo units (2 positions x 8 channels) per stage.
constexpr int kNchwMaxUnits = 4;
constexpr int kNchwLds = 160 * 1024;
constexpr int64_t nchw_lds_bytes(int wgm, int gs, int xu) {
    return 2 * (int64_t)gs * 128 * wgm * 32 + 2 * (int64_t)xu * 256 * 32 + 128 * wgm * 4;
}
struct NchwCfg {
    int wgm;  // waves along the output channels (block rows 128 * wgm)
    int gs;   // taps per stage (every phase padded to it)
    int xu;   // halo units per thread (the halo holds at most 256 * xu positions)
};
constexpr int kNchwCfgCount = 4;
constexpr NchwCfg kNchwCfg[kNchwCfgCount] = {
    {2, 4, 2},  // 0: 2-D kernel 4 stride 2 (2 x 2 taps per phase), C_out/groups > 128
    {1, 4, 2},  // 1: the same, C_out/groups <= 128
    {1, 8, 4},  // 2: 3-D kernel 4 stride 2 (2 x 2 x 2 taps per phase)
    {1, 9, 3},  // 3: 2-D kernel 3 stride 1 (3 x 3 taps)
};
static_assert(nchw_lds_bytes(2, 4, 2) <= kNchwLds && nchw_lds_bytes(1, 8, 4) <= kNchwLds &&
                  nchw_lds_bytes(1, 9, 3) <= kNchwLds,
              "LDS");
// Grouped route
constexpr int kGrpThreads = 256;
constexpr int kGrpCog = 16;           // MFMA N (output channels of a group, padded)
constexpr int kGrpOutStageBytes = 32768;
constexpr int kGrpHaloBytes = 32768;
constexpr int kGrpWBytes = 16384;      // the group's reordered weights, staged in LDS
constexpr int kGrpMaxKSteps = 4;       // MFMA K steps (32 each) per phase
constexpr int kGrpMinPositions = 512;  // q positions per block the tile choice aims for
constexpr int kGrpLdsBudget = 20480;   // LDS per block, for 8 blocks per CU
constexpr int kGrpMaxS2 = 4;           // stride of the last axis (residues kept in registers)
// Direct route
constexpr int kDirThreads = 256;
constexpr int kDirSlabBytes = 32768;  // weight slab of one group in LDS (float32)
constexpr int kDirXStageBytes = 32768; // the group's input planes, staged beside it when they fit
// Direct backward-data kernel (few channels): input channels per pass, and
// its LDS (weights [tap][Cog padded to 8][Cig padded to a pass] as float32,
// then 16 bytes per tap)
constexpr int dir_bwd_ci(int cig) { return cig <= 4 ? 4 : cig <= 8 ? 8 : 16; }
constexpr int64_t dir_bwd_lds_bytes(int cig, int cog, int ktot) {
    return (int64_t)ktot * ((cog + 7) / 8 * 8) * ((cig + dir_bwd_ci(cig) - 1) / dir_bwd_ci(cig) * dir_bwd_ci(cig)) * 4 +
           (int64_t)ktot * 16;
}
constexpr int64_t kDirBwdLdsBytes = 49152;
constexpr int kDirCoChunk = 16;       // output channels accumulated per pass
}  // namespace tiles

convt_status make_plan(const convt_problem *p, Plan *out);

// Per-axis residue data computed on the host (any stride; used for
// inspection and to fill DevAxis).
struct AxisResidue {
    int64_t q_count, n_taps, kk_first, off_first;
};
AxisResidue axis_residue(int64_t I, int64_t K, int64_t S, int64_t P, int64_t D, int64_t O,
                         int64_t r);

}  // namespace convt
