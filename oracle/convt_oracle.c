/*
 * Plain double-precision CPU oracle for the ConvTranspose forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The GPU library never
 * links, loads or calls it, and it shares no code with the GPU library: its
 * shape arithmetic, its loops and its headers are its own.
 *
 * What it computes is the definition of the transposed convolution as a
 * scatter-add, written out with no blocking or reordering:
 *
 *   y[b, oc, o]  = bias[oc]
 *                + sum over ci in the group of oc, input position i, tap kk
 *                  with o = i*s - p + kk*d (per spatial axis) and 0 <= o < O:
 *                    x[b, ci, i] * W[ci, oc - g*Cog, kk]
 *
 * which is the loop "out[b, oc, ih*sH - pH + kh*dH, iw*sW - pW + kw*dW] +=
 * in * w" of the SKaiNET convTranspose2d pull request (page "feat(ops):
 * implement convTranspose2d", Summary), with the 1-D form it mirrors and the
 * 3-D form obtained by adding the depth axis in the same way. Weights are in
 * the layout that page states, [C_in, C_out/groups, k...], in forward (not
 * flipped) orientation; channel ci of group g feeds output channels
 * g*Cog ... g*Cog + Cog - 1, with C_out = Cog * groups (the same page's
 * "groups-aware C_out").
 *
 * The output size per axis is (I - 1)*s - 2*p + d*(k - 1) + op + 1 (same
 * page, Summary; the AWS Neuron conv3d_transpose page's Dimensions list gives
 * the op = 0 form).
 *
 * Padding may differ between the two ends of an axis (the AWS Neuron
 * conv3d_transpose page's padding parameter: a low and a high value per
 * axis). Read here as: the low value p is the p of the scatter above (it
 * shifts every output), and the high value p_hi only trims the end, so that
 * O = (I - 1)*s - (p + p_hi) + d*(k - 1) + op + 1; the symmetric form is
 * p_hi = p. The same reading makes the result the window [p, p + O) of the
 * unpadded (p = p_hi = 0) output.
 *
 * Alongside y it can accumulate scale[b, oc, o] = sum of |x * W| over the same
 * terms, the per-output magnitude used to normalise the GPU error.
 *
 * Every rank is handled as rank 3 with leading unit axes (size 1, k 1,
 * s 1, p 0, d 1, op 0), which leaves the sums unchanged.
 *
 * Parallelism: OpenMP over (b, oc) output planes. Each plane is written by one
 * thread only and its terms are added in a fixed order, so results do not
 * depend on the thread count.
 *
 * Activation (the AWS Neuron conv3d_transpose page's activation_fn, an
 * optional function applied after the convolution; the page names no
 * functions). Read here as one of a fixed set applied to each output after
 * the bias: code 1 ReLU max(v, 0); 2 logistic sigmoid 1/(1 + e^-v); 3 tanh;
 * 4 SiLU v/(1 + e^-v); 5 GELU v/2 (1 + erf(v/sqrt 2)); 0 none
 * (convt_oracle_activation, applied by the caller to the forward result).
 *
 * Backward data (the input gradient, named as the adjoint for the input in
 * the SKaiNET page's Summary, convTranspose2dBackward): y is linear in x, and
 * x[b, ci, i] enters exactly the terms listed above, so for an upstream
 * gradient dy of y's shape
 *
 *   dx[b, ci, i] = sum over oc in the group of ci and taps kk
 *                  with o = i*s - p + kk*d (per axis) and 0 <= o < O:
 *                    dy[b, oc, o] * W[ci, oc - g*Cog, kk]
 *
 * (the same index relation read from the input side; no bias term). It is
 * computed one (b, ci) plane at a time, with its own magnitude sum of
 * |dy * W| over the same terms.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t B, Ci, Co, G, Cig, Cog;
    int64_t I[3], K[3], S[3], P[3], PH[3], D[3], OP[3], O[3];
} oracle_prob;

/* Output size of one axis (p: low padding, ph: high padding); returns < 1
 * when the axis has no outputs. */
static int64_t axis_out(int64_t in, int64_t k, int64_t s, int64_t p, int64_t ph, int64_t d,
                        int64_t op)
{
    return (in - 1) * s - (p + ph) + d * (k - 1) + op + 1;
}

/* Fill an oracle_prob from rank-ndim arguments (padding_end NULL: the high
 * padding equals the low one). Returns 0, or -1 when the arguments do not
 * describe a well-formed transposed convolution. */
static int make_prob(int ndim, const int64_t *x_shape, const int64_t *w_shape,
                     const int64_t *stride, const int64_t *padding, const int64_t *padding_end,
                     const int64_t *dilation, const int64_t *output_padding, int64_t groups,
                     oracle_prob *pb)
{
    if (ndim < 1 || ndim > 3 || groups < 1) return -1;
    pb->B = x_shape[0];
    pb->Ci = x_shape[1];
    pb->Cig = w_shape[0] / groups;
    pb->Cog = w_shape[1];
    pb->G = groups;
    pb->Co = pb->Cog * groups;
    if (pb->B < 0 || pb->Ci < 0 || pb->Cog < 0) return -1;
    if (w_shape[0] != pb->Ci || pb->Ci % groups != 0) return -1;
    int lead = 3 - ndim;
    for (int a = 0; a < 3; ++a) {
        if (a < lead) {
            pb->I[a] = 1; pb->K[a] = 1; pb->S[a] = 1; pb->P[a] = 0; pb->PH[a] = 0; pb->D[a] = 1;
            pb->OP[a] = 0;
        } else {
            int j = a - lead;
            pb->I[a] = x_shape[2 + j];
            pb->K[a] = w_shape[2 + j];
            pb->S[a] = stride[j];
            pb->P[a] = padding[j];
            pb->PH[a] = padding_end ? padding_end[j] : padding[j];
            pb->D[a] = dilation[j];
            pb->OP[a] = output_padding[j];
        }
        if (pb->I[a] < 0 || pb->K[a] < 1 || pb->S[a] < 1 || pb->P[a] < 0 || pb->PH[a] < 0 ||
            pb->D[a] < 1 || pb->OP[a] < 0)
            return -1;
        pb->O[a] = axis_out(pb->I[a], pb->K[a], pb->S[a], pb->P[a], pb->PH[a], pb->D[a], pb->OP[a]);
        if (pb->O[a] < 1) return -1;
    }
    return 0;
}

/* Output spatial sizes (rank ndim). Returns 0 or -1 (as make_prob). */
int convt_oracle_out_shape(int ndim, const int64_t *x_shape, const int64_t *w_shape,
                           const int64_t *stride, const int64_t *padding,
                           const int64_t *padding_end, const int64_t *dilation,
                           const int64_t *output_padding, int64_t groups, int64_t *out_shape)
{
    oracle_prob pb;
    if (make_prob(ndim, x_shape, w_shape, stride, padding, padding_end, dilation, output_padding,
                  groups, &pb))
        return -1;
    out_shape[0] = pb.B;
    out_shape[1] = pb.Co;
    for (int j = 0; j < ndim; ++j) out_shape[2 + j] = pb.O[3 - ndim + j];
    return 0;
}

/* Full forward pass by scatter-add. x: [B, C_in, I...], w: [C_in, Cog, k...],
 * bias: [C_out] or NULL, y: [B, C_out, O...], scale: same shape as y or NULL.
 * nthreads <= 0 leaves the OpenMP default. Returns 0 or -1. */
int convt_oracle_forward(int ndim, const int64_t *x_shape, const int64_t *w_shape,
                         const int64_t *stride, const int64_t *padding, const int64_t *padding_end,
                         const int64_t *dilation, const int64_t *output_padding, int64_t groups,
                         const double *x, const double *w, const double *bias, double *y,
                         double *scale, int nthreads)
{
    oracle_prob pb;
    if (make_prob(ndim, x_shape, w_shape, stride, padding, padding_end, dilation, output_padding,
                  groups, &pb))
        return -1;
    const int64_t isz = pb.I[0] * pb.I[1] * pb.I[2];
    const int64_t ksz = pb.K[0] * pb.K[1] * pb.K[2];
    const int64_t osz = pb.O[0] * pb.O[1] * pb.O[2];
    const int64_t planes = pb.B * pb.Co;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t plane = 0; plane < planes; ++plane) {
        const int64_t b = plane / pb.Co;
        const int64_t oc = plane % pb.Co;
        const int64_t g = oc / pb.Cog;
        const int64_t ocl = oc % pb.Cog;
        double *yp = y + plane * osz;
        double *sp = scale ? scale + plane * osz : NULL;
        const double b0 = bias ? bias[oc] : 0.0;
        for (int64_t o = 0; o < osz; ++o) {
            yp[o] = b0;
            if (sp) sp[o] = 0.0;
        }
        for (int64_t ci = g * pb.Cig; ci < (g + 1) * pb.Cig; ++ci) {
            const double *xp = x + (b * pb.Ci + ci) * isz;
            const double *wp = w + (ci * pb.Cog + ocl) * ksz;
            for (int64_t i0 = 0; i0 < pb.I[0]; ++i0)
            for (int64_t i1 = 0; i1 < pb.I[1]; ++i1)
            for (int64_t i2 = 0; i2 < pb.I[2]; ++i2) {
                const double xv = xp[(i0 * pb.I[1] + i1) * pb.I[2] + i2];
                for (int64_t k0 = 0; k0 < pb.K[0]; ++k0) {
                    const int64_t o0 = i0 * pb.S[0] - pb.P[0] + k0 * pb.D[0];
                    if (o0 < 0 || o0 >= pb.O[0]) continue;
                    for (int64_t k1 = 0; k1 < pb.K[1]; ++k1) {
                        const int64_t o1 = i1 * pb.S[1] - pb.P[1] + k1 * pb.D[1];
                        if (o1 < 0 || o1 >= pb.O[1]) continue;
                        for (int64_t k2 = 0; k2 < pb.K[2]; ++k2) {
                            const int64_t o2 = i2 * pb.S[2] - pb.P[2] + k2 * pb.D[2];
                            if (o2 < 0 || o2 >= pb.O[2]) continue;
                            const double wv = wp[(k0 * pb.K[1] + k1) * pb.K[2] + k2];
                            const int64_t o = (o0 * pb.O[1] + o1) * pb.O[2] + o2;
                            yp[o] += xv * wv;
                            if (sp) sp[o] += fabs(xv * wv);
                        }
                    }
                }
            }
        }
    }
    return 0;
}

/* Selected outputs, each evaluated on its own from the same definition: for
 * output o, the terms are the (i, kk) pairs with o = i*s - p + kk*d, i.e. for
 * each tap kk the input position i = (o + p - kk*d) / s when that division is
 * exact and 0 <= i < I. pts holds npts rows of (b, oc, o...) (2 + ndim
 * entries). yv and sv (sv may be NULL) receive one value per point. Returns 0,
 * or -1 for a malformed problem or an out-of-range point. */
int convt_oracle_points(int ndim, const int64_t *x_shape, const int64_t *w_shape,
                        const int64_t *stride, const int64_t *padding, const int64_t *padding_end,
                        const int64_t *dilation, const int64_t *output_padding, int64_t groups,
                        const double *x, const double *w, const double *bias, int64_t npts,
                        const int64_t *pts, double *yv, double *sv, int nthreads)
{
    oracle_prob pb;
    if (make_prob(ndim, x_shape, w_shape, stride, padding, padding_end, dilation, output_padding,
                  groups, &pb))
        return -1;
    const int lead = 3 - ndim;
    for (int64_t n = 0; n < npts; ++n) {
        const int64_t *pt = pts + n * (2 + ndim);
        if (pt[0] < 0 || pt[0] >= pb.B || pt[1] < 0 || pt[1] >= pb.Co) return -1;
        for (int j = 0; j < ndim; ++j)
            if (pt[2 + j] < 0 || pt[2 + j] >= pb.O[lead + j]) return -1;
    }
    const int64_t isz = pb.I[0] * pb.I[1] * pb.I[2];
    const int64_t ksz = pb.K[0] * pb.K[1] * pb.K[2];
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t n = 0; n < npts; ++n) {
        const int64_t *pt = pts + n * (2 + ndim);
        int64_t o[3] = {0, 0, 0};
        for (int j = 0; j < ndim; ++j) o[lead + j] = pt[2 + j];
        const int64_t b = pt[0], oc = pt[1];
        const int64_t g = oc / pb.Cog, ocl = oc % pb.Cog;
        double acc = bias ? bias[oc] : 0.0, mag = 0.0;
        for (int64_t ci = g * pb.Cig; ci < (g + 1) * pb.Cig; ++ci) {
            const double *xp = x + (b * pb.Ci + ci) * isz;
            const double *wp = w + (ci * pb.Cog + ocl) * ksz;
            for (int64_t k0 = 0; k0 < pb.K[0]; ++k0) {
                const int64_t t0 = o[0] + pb.P[0] - k0 * pb.D[0];
                if (t0 % pb.S[0] != 0) continue;
                const int64_t i0 = t0 / pb.S[0];
                if (i0 < 0 || i0 >= pb.I[0]) continue;
                for (int64_t k1 = 0; k1 < pb.K[1]; ++k1) {
                    const int64_t t1 = o[1] + pb.P[1] - k1 * pb.D[1];
                    if (t1 % pb.S[1] != 0) continue;
                    const int64_t i1 = t1 / pb.S[1];
                    if (i1 < 0 || i1 >= pb.I[1]) continue;
                    for (int64_t k2 = 0; k2 < pb.K[2]; ++k2) {
                        const int64_t t2 = o[2] + pb.P[2] - k2 * pb.D[2];
                        if (t2 % pb.S[2] != 0) continue;
                        const int64_t i2 = t2 / pb.S[2];
                        if (i2 < 0 || i2 >= pb.I[2]) continue;
                        const double xv = xp[(i0 * pb.I[1] + i1) * pb.I[2] + i2];
                        const double wv = wp[(k0 * pb.K[1] + k1) * pb.K[2] + k2];
                        acc += xv * wv;
                        mag += fabs(xv * wv);
                    }
                }
            }
        }
        yv[n] = acc;
        if (sv) sv[n] = mag;
    }
    return 0;
}

/* Threads an OpenMP parallel region of this library would use. */
int convt_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Backward data: dx = d<y, dy>/dx for the problem's shapes. dy: [B, C_out,
 * O...], w: [C_in, Cog, k...], dx: [B, C_in, I...], scale: dx's shape or NULL.
 * Each dx element gathers the (oc, kk) terms whose output o = i*s - p + kk*d
 * lies inside y. Returns 0 or -1. */
int convt_oracle_backward_data(int ndim, const int64_t *x_shape, const int64_t *w_shape,
                               const int64_t *stride, const int64_t *padding,
                               const int64_t *padding_end, const int64_t *dilation,
                               const int64_t *output_padding, int64_t groups, const double *dy,
                               const double *w, double *dx, double *scale, int nthreads)
{
    oracle_prob pb;
    if (make_prob(ndim, x_shape, w_shape, stride, padding, padding_end, dilation, output_padding,
                  groups, &pb))
        return -1;
    const int64_t isz = pb.I[0] * pb.I[1] * pb.I[2];
    const int64_t ksz = pb.K[0] * pb.K[1] * pb.K[2];
    const int64_t osz = pb.O[0] * pb.O[1] * pb.O[2];
    const int64_t planes = pb.B * pb.Ci;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t plane = 0; plane < planes; ++plane) {
        const int64_t b = plane / pb.Ci;
        const int64_t ci = plane % pb.Ci;
        const int64_t g = ci / pb.Cig;
        double *xp = dx + plane * isz;
        double *sp = scale ? scale + plane * isz : NULL;
        for (int64_t i0 = 0; i0 < pb.I[0]; ++i0)
        for (int64_t i1 = 0; i1 < pb.I[1]; ++i1)
        for (int64_t i2 = 0; i2 < pb.I[2]; ++i2) {
            double acc = 0.0, mag = 0.0;
            for (int64_t ocl = 0; ocl < pb.Cog; ++ocl) {
                const double *yp = dy + (b * pb.Co + g * pb.Cog + ocl) * osz;
                const double *wp = w + (ci * pb.Cog + ocl) * ksz;
                for (int64_t k0 = 0; k0 < pb.K[0]; ++k0) {
                    const int64_t o0 = i0 * pb.S[0] - pb.P[0] + k0 * pb.D[0];
                    if (o0 < 0 || o0 >= pb.O[0]) continue;
                    for (int64_t k1 = 0; k1 < pb.K[1]; ++k1) {
                        const int64_t o1 = i1 * pb.S[1] - pb.P[1] + k1 * pb.D[1];
                        if (o1 < 0 || o1 >= pb.O[1]) continue;
                        for (int64_t k2 = 0; k2 < pb.K[2]; ++k2) {
                            const int64_t o2 = i2 * pb.S[2] - pb.P[2] + k2 * pb.D[2];
                            if (o2 < 0 || o2 >= pb.O[2]) continue;
                            const double t = yp[(o0 * pb.O[1] + o1) * pb.O[2] + o2] *
                                             wp[(k0 * pb.K[1] + k1) * pb.K[2] + k2];
                            acc += t;
                            mag += fabs(t);
                        }
                    }
                }
            }
            const int64_t i = (i0 * pb.I[1] + i1) * pb.I[2] + i2;
            xp[i] = acc;
            if (sp) sp[i] = mag;
        }
    }
    return 0;
}

/* Selected dx elements of the backward-data pass, each from the definition
 * above. pts: npts rows of (b, ci, i...). Returns 0, or -1 for a malformed
 * problem or an out-of-range point. */
int convt_oracle_backward_data_points(int ndim, const int64_t *x_shape, const int64_t *w_shape,
                                      const int64_t *stride, const int64_t *padding,
                                      const int64_t *padding_end, const int64_t *dilation,
                                      const int64_t *output_padding, int64_t groups,
                                      const double *dy, const double *w, int64_t npts,
                                      const int64_t *pts, double *dxv, double *sv, int nthreads)
{
    oracle_prob pb;
    if (make_prob(ndim, x_shape, w_shape, stride, padding, padding_end, dilation, output_padding,
                  groups, &pb))
        return -1;
    const int lead = 3 - ndim;
    for (int64_t n = 0; n < npts; ++n) {
        const int64_t *pt = pts + n * (2 + ndim);
        if (pt[0] < 0 || pt[0] >= pb.B || pt[1] < 0 || pt[1] >= pb.Ci) return -1;
        for (int j = 0; j < ndim; ++j)
            if (pt[2 + j] < 0 || pt[2 + j] >= pb.I[lead + j]) return -1;
    }
    const int64_t ksz = pb.K[0] * pb.K[1] * pb.K[2];
    const int64_t osz = pb.O[0] * pb.O[1] * pb.O[2];
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t n = 0; n < npts; ++n) {
        const int64_t *pt = pts + n * (2 + ndim);
        int64_t i[3] = {0, 0, 0};
        for (int j = 0; j < ndim; ++j) i[lead + j] = pt[2 + j];
        const int64_t b = pt[0], ci = pt[1], g = ci / pb.Cig;
        double acc = 0.0, mag = 0.0;
        for (int64_t ocl = 0; ocl < pb.Cog; ++ocl) {
            const double *yp = dy + (b * pb.Co + g * pb.Cog + ocl) * osz;
            const double *wp = w + (ci * pb.Cog + ocl) * ksz;
            for (int64_t k0 = 0; k0 < pb.K[0]; ++k0) {
                const int64_t o0 = i[0] * pb.S[0] - pb.P[0] + k0 * pb.D[0];
                if (o0 < 0 || o0 >= pb.O[0]) continue;
                for (int64_t k1 = 0; k1 < pb.K[1]; ++k1) {
                    const int64_t o1 = i[1] * pb.S[1] - pb.P[1] + k1 * pb.D[1];
                    if (o1 < 0 || o1 >= pb.O[1]) continue;
                    for (int64_t k2 = 0; k2 < pb.K[2]; ++k2) {
                        const int64_t o2 = i[2] * pb.S[2] - pb.P[2] + k2 * pb.D[2];
                        if (o2 < 0 || o2 >= pb.O[2]) continue;
                        const double t = yp[(o0 * pb.O[1] + o1) * pb.O[2] + o2] *
                                         wp[(k0 * pb.K[1] + k1) * pb.K[2] + k2];
                        acc += t;
                        mag += fabs(t);
                    }
                }
            }
        }
        dxv[n] = acc;
        if (sv) sv[n] = mag;
    }
    return 0;
}

/* out[i] = f(in[i]) for activation code act (0..5, see the header); in and
 * out may be the same array. Returns 0, or -1 for an unknown code. */
int convt_oracle_activation(int act, const double *in, double *out, int64_t n)
{
    if (act < 0 || act > 5) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const double v = in[i];
        double r = v;
        switch (act) {
            case 1: r = v > 0.0 ? v : 0.0; break;
            case 2: r = 1.0 / (1.0 + exp(-v)); break;
            case 3: r = tanh(v); break;
            case 4: r = v / (1.0 + exp(-v)); break;
            case 5: r = 0.5 * v * (1.0 + erf(v / sqrt(2.0))); break;
            default: break;
        }
        out[i] = r;
    }
    return 0;
}
