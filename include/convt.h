/*
 * convt.h — C ABI of the MI355X (gfx950) ConvTranspose forward library.
 *
 * The operation is the transposed ("fractionally strided") convolution of an
 * NC[D]HW input, with stride, padding, dilation, output_padding, groups and an
 * optional bias, as defined by the scatter-add
 *     y[b, oc, i*s - p + kk*d] += x[b, ci, i] * W[ci, oc - g*Cog, kk]
 * over each spatial axis (SKaiNET pull request "feat(ops): implement
 * convTranspose2d", Summary; extended per axis to 1-D and 3-D), with output
 * size per axis (I - 1)*s - 2*p + d*(k - 1) + output_padding + 1 (same page,
 * Summary; AWS Neuron conv3d_transpose page, Dimensions), or, when the two
 * ends of an axis are padded differently (AWS Neuron page, :param padding:),
 * (I - 1)*s - (p_lo + p_hi) + d*(k - 1) + output_padding + 1, where the low
 * padding p_lo is the p of the scatter and the high padding p_hi only
 * shortens the axis (y is the window [p_lo, p_lo + O) of the unpadded
 * result), channel ci of group g
 * feeding output channels g*Cog ... g*Cog + Cog - 1 and C_out = Cog * groups
 * (SKaiNET page, "groups-aware C_out"), bias added once per output channel
 * (huggingface ai.onnx.ConvTranspose page, Description; AWS Neuron page,
 * :param bias:).
 *
 * Layouts (all row-major, contiguous, element strides implied by the shapes):
 *   x    [B, C_in, I_1..I_n]            device memory
 *   W    [C_in, C_out/groups, k_1..k_n] device memory, forward (not flipped)
 *                                       orientation, the layout the SKaiNET
 *                                       page states
 *   bias [C_out]                        device memory, optional
 *   y    [B, C_out, O_1..O_n]           device memory, written by the library
 * x, W, bias and y share one element type (float32, bfloat16 or float16; the output
 * type follows the inputs as on the huggingface page, "Use with"). Products
 * are accumulated in float32 and the result is rounded once to the output
 * type, after the bias is added.
 *
 * Ownership: the caller allocates and owns every device buffer, including the
 * workspace (its size is reported by convt_plan). The library allocates no
 * device memory and keeps no pointer after a call returns. A plan is host
 * memory owned by the library until convt_destroy; it is immutable after
 * convt_plan, so one plan may serve concurrent calls on different streams as
 * long as each call has its own workspace and output.
 *
 * Errors: every entry point returns a convt_status. Argument errors are
 * detected on the host before anything is enqueued. Device work is
 * asynchronous on the given stream: a launch failure is reported as
 * CONVT_ERR_DEVICE, a fault inside a kernel surfaces at the caller's next
 * synchronisation.
 *
 * Stream arguments are hipStream_t values passed as void* (NULL = the null
 * stream), so this header needs no HIP header.
 */
#ifndef CONVT_H
#define CONVT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CONVT_MAX_NDIM 3

typedef enum convt_status {
    CONVT_OK = 0,
    /* a validation rule failed (see convt_plan), a NULL where a pointer is
     * required, or a bias pointer that disagrees with has_bias */
    CONVT_ERR_INVALID_ARGUMENT = 1,
    /* a well-formed request this library does not compute: a non-float element
     * type (the SKaiNET page's dtype guard: such requests fail loudly rather
     * than corrupt), or a forced route that cannot serve the problem */
    CONVT_ERR_UNSUPPORTED = 2,
    /* the HIP runtime refused a launch */
    CONVT_ERR_DEVICE = 3
} convt_status;

typedef enum convt_dtype {
    CONVT_DTYPE_F32 = 0,
    CONVT_DTYPE_BF16 = 1,
    /* IEEE half (the huggingface page's shader-f16 variants) */
    CONVT_DTYPE_F16 = 2,
    /* the codes below name element types that are refused with
     * CONVT_ERR_UNSUPPORTED */
    CONVT_DTYPE_I8 = 3,
    CONVT_DTYPE_I32 = 4,
    CONVT_DTYPE_I64 = 5
} convt_dtype;

/* Which device route serves a plan. CONVT_ROUTE_AUTO lets the planner pick
 * from the shapes and the element type (the huggingface page picks one
 * implementation per call the same way, "Implementation variants"); any other
 * value forces that route, or fails with CONVT_ERR_UNSUPPORTED if the route
 * cannot serve the problem. */
typedef enum convt_route {
    CONVT_ROUTE_AUTO = 0,
    CONVT_ROUTE_NONE = 1,       /* the output is empty: nothing to launch */
    CONVT_ROUTE_FILL = 2,       /* no input channels: y = bias (or 0) */
    CONVT_ROUTE_PHASE_GEMM = 3, /* stride-phase implicit-gather GEMM on MFMA */
    CONVT_ROUTE_GROUPED = 4,    /* grouped / few-channel stride-phase kernel, MFMA, LDS-staged output;
                                   as route_bwd, its input gradient on MFMA (see
                                   convt_backward_data) */
    CONVT_ROUTE_DIRECT = 5,     /* small-channel direct kernel, weight slab in LDS */
    CONVT_ROUTE_NAIVE = 6,      /* one thread per output, gathers its terms */
    CONVT_ROUTE_PHASE_GEMM_PACKED = 7, /* two-byte types: the phase GEMM on a channel-chunked copy
                                         of x that each call writes into the workspace (the
                                         PHASE_GEMM route reads x in place when the problem
                                         suits that kernel, and plans this one otherwise);
                                         forward only */
    CONVT_ROUTE_PHASE_GEMM_ALLPHASE = 8 /* two-byte types, stride 2 and dilation 1 on the two
                                           innermost axes: one block computes all four of their
                                           stride phases of an output tile, reading x and W as
                                           stored (no workspace, one launch per call); AUTO
                                           plans it where it applies; as route_bwd, the input
                                           gradient's counterpart (16 taps over those axes) */
} convt_route;

/* How W is laid out in memory (the AWS Neuron conv3d_transpose page's
 * filter_shape, extended to groups). Element (ci, ocl, kk) is the weight
 * from input channel ci (global) to output channel g*Cog + ocl of ci's group
 * g, at tap kk (row-major over the kernel axes):
 *   CI_CO_K  [C_in][C_out/groups][k...]   (the SKaiNET page's layout; default)
 *   K_CI_CO  [k...][C_in][C_out/groups]   (the Neuron page's KDHW_CI_CO)
 *   K_CO_CI  [k...][C_out][C_in/groups]   (the Neuron page's KDHW_CO_CI)
 * w_shape in convt_problem stays [C_in, C_out/groups, k...] whatever the
 * layout. With taps_flipped = 1 the stored tap kk holds the forward tap
 * (k_1-1-kk_1, ..., k_n-1-kk_n): the caller has spatially reversed the
 * filter (the Neuron page's flip_filter_taps_in_kernel = False). */
typedef enum convt_filter_layout {
    CONVT_FILTER_CI_CO_K = 0,
    CONVT_FILTER_K_CI_CO = 1,
    CONVT_FILTER_K_CO_CI = 2
} convt_filter_layout;

/* Activation applied to each output after the bias, in float32 before the
 * single rounding to the output type (the AWS Neuron conv3d_transpose
 * page's activation_fn, which names no functions; this set is the reading
 * adopted): ReLU max(v, 0); logistic sigmoid 1/(1 + e^-v); tanh;
 * SiLU v/(1 + e^-v); GELU v/2 (1 + erf(v/sqrt 2)). convt_backward_data
 * ignores it (it is the gradient of the convolution alone). */
typedef enum convt_activation {
    CONVT_ACT_NONE = 0,
    CONVT_ACT_RELU = 1,
    CONVT_ACT_SIGMOID = 2,
    CONVT_ACT_TANH = 3,
    CONVT_ACT_SILU = 4,
    CONVT_ACT_GELU = 5
} convt_activation;

/* The problem, in the terms the pages use. Only the first 2 + ndim entries
 * of the shape arrays and the first ndim entries of the attribute arrays are
 * read. padding is the low (leading) padding of each axis; the high
 * (trailing) padding equals it unless has_padding_hi is 1, in which case it
 * is padding_hi (the AWS Neuron page's pad_*_lo / pad_*_hi pairs). A
 * zero-initialised tail (has_padding_hi = 0) keeps symmetric padding. */
typedef struct convt_problem {
    int32_t ndim;                               /* 1, 2 or 3 spatial axes */
    int32_t dtype;                              /* convt_dtype of x, W, bias and y */
    int64_t x_shape[2 + CONVT_MAX_NDIM];        /* [B, C_in, I...] */
    int64_t w_shape[2 + CONVT_MAX_NDIM];        /* [C_in, C_out/groups, k...] */
    int64_t stride[CONVT_MAX_NDIM];             /* >= 1 */
    int64_t padding[CONVT_MAX_NDIM];            /* >= 0 */
    int64_t dilation[CONVT_MAX_NDIM];           /* >= 1 */
    int64_t output_padding[CONVT_MAX_NDIM];     /* 0 <= op < max(stride, dilation) */
    int64_t groups;                             /* >= 1, divides C_in */
    int32_t has_bias;                           /* 0 or 1 */
    int32_t route;                              /* convt_route; CONVT_ROUTE_AUTO normally */
    int32_t has_padding_hi;                     /* 0: high padding = padding; 1: = padding_hi */
    int32_t route_bwd;                          /* convt_route of convt_backward_data; AUTO normally */
    int64_t padding_hi[CONVT_MAX_NDIM];         /* >= 0; read only when has_padding_hi = 1 */
    int32_t filter_layout;                      /* convt_filter_layout of W */
    int32_t taps_flipped;                       /* 1: W's taps are spatially reversed */
    int32_t activation;                         /* convt_activation applied to y */
    int32_t reserved1;                          /* must be 0 */
} convt_problem;

typedef struct convt_plan_info {
    int64_t out_shape[2 + CONVT_MAX_NDIM];      /* [B, C_out, O...] (first 2 + ndim entries) */
    int64_t c_out;                              /* w_shape[1] * groups */
    int64_t workspace_bytes;                    /* device workspace the caller must pass (may be 0) */
    int64_t n_phases;                           /* product of the strides */
    int64_t useful_flops;                       /* 2 * B * C_in * (C_out/groups) * prod(k) * prod(I) */
    int32_t route;                              /* the convt_route chosen */
    int32_t route_bwd;                          /* the route of convt_backward_data */
    int64_t bwd_workspace_bytes;                /* device workspace convt_backward_data needs */
} convt_plan_info;

typedef struct convt_plan_s *convt_plan_t;

/*
 * Validate a problem and build a plan. Host only: no device call is made.
 *
 * Validation (SKaiNET page, commit message and Summary: stride, padding,
 * outputPadding < max(stride, dilation) per axis, dilation, groups
 * divisibility, bias shape, dtype guard; plus shape consistency):
 *   ndim in 1..3; all sizes >= 0; kernel sizes >= 1; stride >= 1;
 *   padding >= 0 (both ends); has_padding_hi in {0, 1}; route and route_bwd
 *   valid convt_route codes; filter_layout a convt_filter_layout;
 *   taps_flipped in {0, 1}; activation a convt_activation; reserved1 == 0;
 *   dilation >= 1; 0 <= output_padding < max(stride, dilation);
 *   groups >= 1 dividing C_in; w_shape[0] == C_in; every output size >= 1;
 *   has_bias in {0, 1}; element counts of x, W and y below 2^62 and each
 *   plane (one batch item, one channel) below 2^31 elements.
 * A batch of 0 or C_out of 0 is valid and plans CONVT_ROUTE_NONE; C_in of 0
 * (or an input axis of size 0 with positive output size) plans
 * CONVT_ROUTE_FILL.
 *
 * On success *out receives a plan and, if info is not NULL, *info is filled.
 * On failure *out is set to NULL (when out is not NULL) and the status says
 * why: CONVT_ERR_INVALID_ARGUMENT or CONVT_ERR_UNSUPPORTED.
 */
convt_status convt_plan(const convt_problem *problem, convt_plan_t *out, convt_plan_info *info);

/*
 * y = convT(x, W) + bias, enqueued on `stream`; no host synchronisation.
 * x, W, y: device pointers with the plan's shapes and element type; bias: a
 * device pointer to C_out elements, required (non-NULL) iff has_bias, NULL
 * otherwise. workspace: device memory of at least info.workspace_bytes bytes
 * (NULL allowed when that is 0), 16-byte aligned; it must not be used by
 * another call until this call's work on `stream` has finished. y must not
 * overlap x, W, bias or the workspace. Same result, byte for byte, as
 * convt_prepare_weights followed by convt_forward_prepared; on the
 * PHASE_GEMM_PACKED route it runs the weight reorder and the input copy as
 * one launch. On the PHASE_GEMM route with a two-byte element type, x must
 * be 4-byte aligned (that kernel reads neighbouring positions in pairs as
 * 32-bit words); a misaligned x is refused with CONVT_ERR_INVALID_ARGUMENT
 * before anything is enqueued. On the PHASE_GEMM_ALLPHASE route x must be
 * 4-byte aligned and W 16-byte aligned (W is read in 16-byte pieces of 8
 * taps), else CONVT_ERR_INVALID_ARGUMENT; that route needs no workspace.
 */
convt_status convt_forward(convt_plan_t plan, const void *x, const void *w, const void *bias,
                           void *y, void *workspace, void *stream);

/*
 * First half of convt_forward: reorder W into the workspace, with taps
 * flipped and grouped by stride phase (the plan's weight layout). Weights are
 * taken in forward orientation and reversed by the library, the behaviour the
 * AWS Neuron page calls flip_filter_taps_in_kernel=True. Does nothing for
 * routes that read W directly. Arguments as in convt_forward.
 */
convt_status convt_prepare_weights(convt_plan_t plan, const void *w, void *workspace, void *stream);

/*
 * Second half of convt_forward: compute y from x, the workspace written by
 * convt_prepare_weights (for the same plan and the same W), W itself (used
 * by the routes that read it directly; may be NULL for the others) and bias.
 * The prepared weights at the start of the workspace are left unchanged; the
 * rest of it is scratch that the call overwrites (the PHASE_GEMM_PACKED
 * route stages a channel-chunked copy of x there). Arguments as in
 * convt_forward.
 */
convt_status convt_forward_prepared(convt_plan_t plan, const void *x, const void *w,
                                    const void *bias, void *y, void *workspace, void *stream);

/*
 * Backward data: the gradient of a loss with respect to x, given its gradient
 * dy with respect to y (the SKaiNET page's Summary names this adjoint for the
 * input, convTranspose2dBackward). y is linear in x, so
 *     dx[b, ci, i] = sum over oc in the group of ci and taps kk with
 *                    o = i*s - p + kk*d inside y:  dy[b, oc, o] * W[ci, oc - g*Cog, kk]
 * per axis, p the low padding; the bias does not enter.
 *
 * dy: [B, C_out, O...] (the plan's out_shape), W as for convt_forward, dx:
 * [B, C_in, I...] (x's shape), all device memory of the plan's element type;
 * dx is overwritten and must not alias dy or W. Products are accumulated in
 * float32 and rounded once to the element type. workspace: device memory of
 * at least info.bwd_workspace_bytes bytes, 16-byte aligned (may be NULL when
 * that is 0); it is scratch, and may be the forward's workspace buffer if
 * large enough, but not in use by a concurrent call. Asynchronous on stream,
 * errors as for convt_forward. route_bwd may not be PHASE_GEMM_PACKED
 * (CONVT_ERR_UNSUPPORTED at planning). Routes (info.route_bwd): NONE (dx empty),
 * FILL (no output channels: dx = 0), PHASE_GEMM (stride phases summed inside
 * one implicit-gather GEMM on MFMA), PHASE_GEMM_ALLPHASE (two-byte types,
 * stride 2 and dilation 1 on the two innermost axes with 16 taps over them,
 * W in the CI_CO_K layout: one MFMA GEMM reads dy and W as stored and sums
 * the four stride phases of each dx box from one halo; no workspace; dy must
 * be 4-byte and W and dx 16-byte aligned, else CONVT_ERR_INVALID_ARGUMENT),
 * GROUPED (two-byte 2-D problems whose output channels per group are a
 * multiple of 8 with at most 16 (tap, 8-channel slice) slots, at most 16
 * input channels per group and dy rows of whole 16-byte chunks: a strided
 * correlation of dy on MFMA, a block per (batch, group, dx row tile) with
 * dy's halo and the group's W in LDS; no workspace; when dy or W is not
 * 16-byte aligned the call runs the DIRECT kernel instead, same result),
 * DIRECT (few channels per group: a thread per dx position over its group's
 * input channels, weights in LDS), NAIVE (one thread per dx element).
 */
convt_status convt_backward_data(convt_plan_t plan, const void *dy, const void *w, void *dx,
                                 void *workspace, void *stream);

/* Free a plan. NULL is accepted and ignored. */
void convt_destroy(convt_plan_t plan);

/* Static text for a status code (never NULL). */
const char *convt_status_string(convt_status status);

/* Static name of a route ("phase_gemm", ...; never NULL). */
const char *convt_route_name(int32_t route);

/*
 * Stride-phase table of one axis of a plan, for inspection. For output residue
 * r (0 <= r < stride of the axis) it reports the output positions s*q + r,
 * q in [0, q_count), and the taps kk whose products land on them, in the
 * order the plan uses (ascending input offset), with each tap's input offset
 * off = (r + p - kk*d) / s (exact; p is the low padding), so that y[s*q + r]
 * gathers x[q + off] * W[kk].
 * `axis` counts spatial axes from 0. taps/offsets receive at most `cap`
 * entries; *n_taps gets the full count. Host only.
 */
convt_status convt_plan_axis_phase(convt_plan_t plan, int32_t axis, int64_t residue,
                                   int64_t *q_count, int64_t *n_taps, int64_t *taps,
                                   int64_t *offsets, int64_t cap);

/* The plan information of an existing plan (what convt_plan returned in
 * *info). Host only. CONVT_ERR_INVALID_ARGUMENT if plan or info is NULL. */
convt_status convt_plan_query(convt_plan_t plan, convt_plan_info *info);

/* Library version, major*10000 + minor*100 + patch. */
int32_t convt_version(void);

/*
 * For callers that cannot allocate device memory (code under stream or graph
 * capture that must not call the allocator, tight serving loops, harnesses
 * that forbid allocation): convt_forward with the workspace taken from a
 * fixed array of CONVT_SCRATCH_MAX_BYTES bytes inside this library, one
 * per GPU, held from the library's first use on that GPU until the process
 * ends. Arguments and result as for convt_forward, without the workspace.
 * Makes no allocation call (no hipMalloc, no hipFree). Plans whose
 * info.workspace_bytes exceed CONVT_SCRATCH_MAX_BYTES are refused with
 * CONVT_ERR_UNSUPPORTED before anything is enqueued; CONVT_ERR_DEVICE if the
 * array's address on the current device cannot be obtained. Every call on
 * one GPU uses the same array: calls whose work overlaps on that GPU (other
 * streams, or another host thread) race on it and must be serialised by the
 * caller; calls in one stream are ordered and safe. Nothing needs to start
 * at zero: each call writes every byte it reads from the array before
 * reading it.
 */
#define CONVT_SCRATCH_MAX_BYTES (32 * 1024 * 1024)
convt_status convt_forward_scratch(convt_plan_t plan, const void *x, const void *w,
                                   const void *bias, void *y, void *stream);

/* CONVT_SCRATCH_MAX_BYTES, for bindings. */
int64_t convt_scratch_max_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVT_H */
