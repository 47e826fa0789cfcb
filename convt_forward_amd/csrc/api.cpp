// C ABI of the library (declared in include/convt.h).
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include <new>

#include "convt.h"
#include "convt_internal.h"
#include "launch.h"

struct convt_plan_s {
    convt::Plan plan;
};

namespace {

int64_t numel(const int64_t *shape, int n) {
    int64_t v = 1;
    for (int i = 0; i < n; ++i) v *= shape[i];
    return v;
}

convt_status device_status(hipError_t e) { return e == hipSuccess ? CONVT_OK : CONVT_ERR_DEVICE; }

bool needs_weights_in_workspace(int route) {
    return route == CONVT_ROUTE_PHASE_GEMM || route == CONVT_ROUTE_PHASE_GEMM_PACKED;
}

// The two-byte phase GEMM that reads x in place takes neighbouring positions
// in pairs as 32-bit words.
bool x_misaligned(const convt::Plan &pl, const void *x) {
    return ((pl.route == CONVT_ROUTE_PHASE_GEMM && pl.dp.gemm_nchw) || pl.route == CONVT_ROUTE_PHASE_GEMM_ALLPHASE) &&
           ((uintptr_t)x % 4) != 0;
}

// The all-phase GEMM reads W in 16-byte pieces.
bool w_misaligned(const convt::Plan &pl, const void *w) {
    return pl.route == CONVT_ROUTE_PHASE_GEMM_ALLPHASE && ((uintptr_t)w % 16) != 0;
}

}  // namespace

extern "C" {

convt_status convt_plan(const convt_problem *problem, convt_plan_t *out, convt_plan_info *info) {
    if (out) *out = nullptr;
    if (!problem || !out) return CONVT_ERR_INVALID_ARGUMENT;
    convt_plan_s *h = new (std::nothrow) convt_plan_s;
    if (!h) return CONVT_ERR_DEVICE;
    const convt_status st = convt::make_plan(problem, &h->plan);
    if (st != CONVT_OK) {
        delete h;
        return st;
    }
    if (info) *info = h->plan.info;
    *out = h;
    return CONVT_OK;
}

void convt_destroy(convt_plan_t plan) { delete plan; }

convt_status convt_prepare_weights(convt_plan_t plan, const void *w, void *workspace, void *stream) {
    if (!plan) return CONVT_ERR_INVALID_ARGUMENT;
    const convt::Plan &pl = plan->plan;
    if (!needs_weights_in_workspace(pl.route) || pl.wr_elems == 0) return CONVT_OK;
    const int nd = pl.ndim;
    if (!w && numel(pl.prob.w_shape, 2 + nd) > 0) return CONVT_ERR_INVALID_ARGUMENT;
    if (!workspace || ((uintptr_t)workspace % 16) != 0) return CONVT_ERR_INVALID_ARGUMENT;
    return device_status(convt::launch_reorder(pl, w, workspace, (hipStream_t)stream));
}

convt_status convt_forward_prepared(convt_plan_t plan, const void *x, const void *w,
                                    const void *bias, void *y, void *workspace, void *stream) {
    if (!plan) return CONVT_ERR_INVALID_ARGUMENT;
    const convt::Plan &pl = plan->plan;
    const int nd = pl.ndim;
    const hipStream_t s = (hipStream_t)stream;
    const int64_t yn = numel(pl.info.out_shape, 2 + nd);
    if (pl.route == CONVT_ROUTE_NONE || yn == 0) return CONVT_OK;
    if (!y) return CONVT_ERR_INVALID_ARGUMENT;
    if (pl.prob.has_bias && !bias) return CONVT_ERR_INVALID_ARGUMENT;
    if (!pl.prob.has_bias && bias) return CONVT_ERR_INVALID_ARGUMENT;
    const bool x_needed = pl.route != CONVT_ROUTE_FILL;
    if (x_needed && !x && numel(pl.prob.x_shape, 2 + nd) > 0) return CONVT_ERR_INVALID_ARGUMENT;
    switch (pl.route) {
        case CONVT_ROUTE_FILL:
            return device_status(convt::launch_fill(pl, bias, y, s));
        case CONVT_ROUTE_NAIVE:
            if (!w) return CONVT_ERR_INVALID_ARGUMENT;
            return device_status(convt::launch_naive(pl, x, w, bias, y, s));
        case CONVT_ROUTE_DIRECT:
            if (!w) return CONVT_ERR_INVALID_ARGUMENT;
            return device_status(convt::launch_direct(pl, x, w, bias, y, s));
        case CONVT_ROUTE_PHASE_GEMM_ALLPHASE:
            if (!w || x_misaligned(pl, x) || w_misaligned(pl, w)) return CONVT_ERR_INVALID_ARGUMENT;
            return device_status(convt::launch_allphase(pl, x, w, bias, y, s));
        case CONVT_ROUTE_PHASE_GEMM:
        case CONVT_ROUTE_PHASE_GEMM_PACKED: {
            if (!workspace || ((uintptr_t)workspace % 16) != 0) return CONVT_ERR_INVALID_ARGUMENT;
            if (pl.dp.gemm_nchw) {
                if (x_misaligned(pl, x)) return CONVT_ERR_INVALID_ARGUMENT;
                return device_status(convt::launch_phase_gemm_nchw(pl, x, workspace, bias, y, s));
            }
            const void *xin = x;
            if (pl.xp_bytes > 0) {
                // bfloat16: stage the channel-chunked copy of x after the weights
                void *xp = (char *)workspace + pl.xp_offset;
                const convt_status st = device_status(convt::launch_pack_x(pl, x, xp, s));
                if (st != CONVT_OK) return st;
                xin = xp;
            }
            return device_status(convt::launch_phase_gemm(pl, xin, workspace, bias, y, s));
        }
        case CONVT_ROUTE_GROUPED:
            if (!w) return CONVT_ERR_INVALID_ARGUMENT;
            return device_status(convt::launch_grouped(pl, x, w, bias, y, s));
        default:
            return CONVT_ERR_UNSUPPORTED;
    }
}

convt_status convt_forward(convt_plan_t plan, const void *x, const void *w, const void *bias,
                           void *y, void *workspace, void *stream) {
    if (!plan) return CONVT_ERR_INVALID_ARGUMENT;
    const convt::Plan &pl = plan->plan;
    const int nd = pl.ndim;
    if (pl.route == CONVT_ROUTE_NONE || numel(pl.info.out_shape, 2 + nd) == 0) return CONVT_OK;
    // argument checks first, so that nothing is enqueued for a bad call
    if (!y) return CONVT_ERR_INVALID_ARGUMENT;
    if (pl.prob.has_bias != (bias != nullptr)) return CONVT_ERR_INVALID_ARGUMENT;
    if (pl.route != CONVT_ROUTE_FILL && !x) return CONVT_ERR_INVALID_ARGUMENT;
    if (pl.route != CONVT_ROUTE_FILL && !w) return CONVT_ERR_INVALID_ARGUMENT;
    if (needs_weights_in_workspace(pl.route) &&
        (!workspace || ((uintptr_t)workspace % 16) != 0))
        return CONVT_ERR_INVALID_ARGUMENT;
    if (x_misaligned(pl, x) || w_misaligned(pl, w)) return CONVT_ERR_INVALID_ARGUMENT;
    if (pl.route == CONVT_ROUTE_PHASE_GEMM_PACKED && pl.xp_bytes > 0 && pl.wr_elems > 0) {
        // two-byte elements: the weight reorder and the channel-chunked copy
        // of x in one launch, then the GEMM
        const hipStream_t s = (hipStream_t)stream;
        void *xp = (char *)workspace + pl.xp_offset;
        const convt_status st = device_status(convt::launch_prep(pl, w, workspace, x, xp, s));
        if (st != CONVT_OK) return st;
        return device_status(convt::launch_phase_gemm(pl, xp, workspace, bias, y, s));
    }
    convt_status st = convt_prepare_weights(plan, w, workspace, stream);
    if (st != CONVT_OK) return st;
    return convt_forward_prepared(plan, x, w, bias, y, workspace, stream);
}

convt_status convt_backward_data(convt_plan_t plan, const void *dy, const void *w, void *dx,
                                 void *workspace, void *stream) {
    if (!plan) return CONVT_ERR_INVALID_ARGUMENT;
    const convt::Plan &pl = plan->plan;
    const int nd = pl.ndim;
    const hipStream_t s = (hipStream_t)stream;
    if (pl.route_bwd == CONVT_ROUTE_NONE || numel(pl.prob.x_shape, 2 + nd) == 0) return CONVT_OK;
    if (!dx) return CONVT_ERR_INVALID_ARGUMENT;
    if (pl.route_bwd == CONVT_ROUTE_FILL)
        return device_status(convt::launch_fill_dp(pl.bdp, pl.elem_bytes, nullptr, dx, s));
    if (!dy || !w) return CONVT_ERR_INVALID_ARGUMENT;
    switch (pl.route_bwd) {
        case CONVT_ROUTE_NAIVE:
            return device_status(convt::launch_naive_bwd(pl, dy, w, dx, s));
        case CONVT_ROUTE_DIRECT:
            return device_status(convt::launch_direct_bwd(pl, dy, w, dx, s));
        case CONVT_ROUTE_GROUPED:
            // dy read in 16-byte pieces, W copied in 16-byte pieces; otherwise
            // the direct kernel (eligible for every plan of this route)
            if ((uintptr_t)dy % 16 != 0 || (uintptr_t)w % 16 != 0)
                return device_status(convt::launch_direct_bwd(pl, dy, w, dx, s));
            return device_status(convt::launch_grouped_bwd(pl, dy, w, dx, s));
        case CONVT_ROUTE_PHASE_GEMM_ALLPHASE:
            // dy read in 4-byte pairs, W in 16-byte pieces, dx stored in 16-byte pieces
            if ((uintptr_t)dy % 4 != 0 || (uintptr_t)w % 16 != 0 || (uintptr_t)dx % 16 != 0)
                return CONVT_ERR_INVALID_ARGUMENT;
            return device_status(convt::launch_allphase_bwd(pl, dy, w, dx, s));
        case CONVT_ROUTE_PHASE_GEMM: {
            if (!workspace || ((uintptr_t)workspace % 16) != 0) return CONVT_ERR_INVALID_ARGUMENT;
            if (pl.bwd_xp_bytes > 0) {
                // two-byte elements: the weight reorder and the channel-chunked
                // copy of dy (after the weights) in one launch
                void *xp = (char *)workspace + pl.bwd_xp_offset;
                const convt_status st = device_status(convt::launch_prep_bwd(pl, w, workspace, dy, xp, s));
                if (st != CONVT_OK) return st;
                return device_status(convt::launch_phase_gemm_bwd(pl, xp, workspace, dx, s));
            }
            const convt_status st = device_status(convt::launch_reorder_bwd(pl, w, workspace, s));
            if (st != CONVT_OK) return st;
            return device_status(convt::launch_phase_gemm_bwd(pl, dy, workspace, dx, s));
        }
        default:
            return CONVT_ERR_UNSUPPORTED;
    }
}

const char *convt_status_string(convt_status status) {
    switch (status) {
        case CONVT_OK: return "ok";
        case CONVT_ERR_INVALID_ARGUMENT: return "invalid argument";
        case CONVT_ERR_UNSUPPORTED: return "unsupported request";
        case CONVT_ERR_DEVICE: return "device error";
        default: return "unknown status";
    }
}

const char *convt_route_name(int32_t route) {
    switch (route) {
        case CONVT_ROUTE_AUTO: return "auto";
        case CONVT_ROUTE_NONE: return "none";
        case CONVT_ROUTE_FILL: return "fill";
        case CONVT_ROUTE_PHASE_GEMM: return "phase_gemm";
        case CONVT_ROUTE_PHASE_GEMM_PACKED: return "phase_gemm_packed";
        case CONVT_ROUTE_PHASE_GEMM_ALLPHASE: return "phase_gemm_allphase";
        case CONVT_ROUTE_GROUPED: return "grouped";
        case CONVT_ROUTE_DIRECT: return "direct";
        case CONVT_ROUTE_NAIVE: return "naive";
        default: return "unknown";
    }
}

convt_status convt_plan_axis_phase(convt_plan_t plan, int32_t axis, int64_t residue,
                                   int64_t *q_count, int64_t *n_taps, int64_t *taps,
                                   int64_t *offsets, int64_t cap) {
    if (!plan) return CONVT_ERR_INVALID_ARGUMENT;
    const convt::Plan &pl = plan->plan;
    if (axis < 0 || axis >= pl.ndim) return CONVT_ERR_INVALID_ARGUMENT;
    const convt_problem &p = pl.prob;
    const int64_t I = p.x_shape[2 + axis], K = p.w_shape[2 + axis], S = p.stride[axis],
                  P = p.padding[axis], D = p.dilation[axis];
    const int64_t O = pl.info.out_shape[2 + axis];
    if (residue < 0 || residue >= S) return CONVT_ERR_INVALID_ARGUMENT;
    if (cap < 0 || (cap > 0 && (!taps || !offsets))) return CONVT_ERR_INVALID_ARGUMENT;
    const convt::AxisResidue a = convt::axis_residue(I, K, S, P, D, O, residue);
    if (q_count) *q_count = a.q_count;
    if (n_taps) *n_taps = a.n_taps;
    // ascending offset order: kk from kk_first downwards in steps of s / gcd(s, d)
    int64_t g = S, h = D;
    while (h) {
        const int64_t t = g % h;
        g = h;
        h = t;
    }
    const int64_t kstep = S / g;
    for (int64_t j = 0; j < a.n_taps && j < cap; ++j) {
        const int64_t kk = a.kk_first - j * kstep;
        taps[j] = kk;
        offsets[j] = (residue + P - kk * D) / S;
    }
    return CONVT_OK;
}

convt_status convt_plan_query(convt_plan_t plan, convt_plan_info *info) {
    if (!plan || !info) return CONVT_ERR_INVALID_ARGUMENT;
    *info = plan->plan.info;
    return CONVT_OK;
}

int32_t convt_version(void) { return 320; }

}  // extern "C"
