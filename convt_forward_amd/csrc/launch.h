// Host-side launchers of the kernels. Each enqueues its kernel(s) on `stream`
// and returns the launch status; none synchronises.
#pragma once

#include <hip/hip_runtime_api.h>

#include "convt_internal.h"

namespace convt {

hipError_t launch_reorder(const Plan &pl, const void *w, void *wr, hipStream_t stream);
hipError_t launch_pack_x(const Plan &pl, const void *x, void *xp, hipStream_t stream);
hipError_t launch_fill(const Plan &pl, const void *bias, void *y, hipStream_t stream);
hipError_t launch_naive(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                        hipStream_t stream);
hipError_t launch_direct(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                         hipStream_t stream);
// wr: the workspace (reordered weights at offset 0, tap table at tab_offset)
hipError_t launch_phase_gemm(const Plan &pl, const void *x, const void *wr, const void *bias,
                             void *y, hipStream_t stream);
// two-byte phase GEMM reading x in NC[D]HW (plans with dp.gemm_nchw)
hipError_t launch_phase_gemm_nchw(const Plan &pl, const void *x, const void *wr, const void *bias,
                                  void *y, hipStream_t stream);
// all-phase two-byte GEMM (CONVT_ROUTE_PHASE_GEMM_ALLPHASE): x and W as the
// caller stores them, no workspace
hipError_t launch_allphase(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                           hipStream_t stream);
// grouped kernel: W as stored (it gathers its group's slab itself), no workspace
hipError_t launch_grouped(const Plan &pl, const void *x, const void *w, const void *bias, void *y,
                          hipStream_t stream);

// Backward data (dx from dy). The channel-chunked copy and the fill use the
// kernels of the forward with the backward problem's parameters.
hipError_t launch_pack_dp(const DevParams &p, const void *x, void *xp, hipStream_t stream);
hipError_t launch_fill_dp(const DevParams &p, int elem_bytes, const void *bias, void *y,
                          hipStream_t stream);
hipError_t launch_reorder_bwd(const Plan &pl, const void *w, void *wr, hipStream_t stream);
hipError_t launch_naive_bwd(const Plan &pl, const void *dy, const void *w, void *dx,
                            hipStream_t stream);
hipError_t launch_direct_bwd(const Plan &pl, const void *dy, const void *w, void *dx,
                             hipStream_t stream);
hipError_t launch_phase_gemm_bwd(const Plan &pl, const void *dy, const void *wr, void *dx,
                                 hipStream_t stream);
// backward all-phase GEMM (route_bwd PHASE_GEMM_ALLPHASE): dy and W as the
// caller stores them, no workspace
hipError_t launch_grouped_bwd(const Plan &pl, const void *dy, const void *w, void *dx, hipStream_t stream);
hipError_t launch_allphase_bwd(const Plan &pl, const void *dy, const void *w, void *dx,
                               hipStream_t stream);

// Two-byte phase GEMM: the weight reorder and the channel-chunked input copy
// of the forward (resp. backward) problem in one launch; xp at the plan's
// xp_offset (resp. bwd_xp_offset) of the workspace wr.
hipError_t launch_prep(const Plan &pl, const void *w, void *wr, const void *x, void *xp,
                       hipStream_t stream);
hipError_t launch_prep_bwd(const Plan &pl, const void *w, void *wr, const void *dy, void *xp,
                           hipStream_t stream);

}  // namespace convt
