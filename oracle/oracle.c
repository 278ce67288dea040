/*
 * oracle.c -- fp64 CPU oracle for forward N-d convolution and for the fused
 * Conv3d -> min over one spatial axis -> softmax over channels.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the checker, not the product: only the
 * test suite, the smoke check and the bench's CPU-baseline leg load it. It
 * shares no code, header, table or helper with the HIP library.
 *
 * What it computes (the problem statements of the three POPCORNBENCH
 * "Kimi-K2.6" pages: l1_p60 "Conv3d with asymmetric kernel", l2_p24
 * "Conv3d + min + softmax", l1_p76 "Conv1d strided and dilated"; each page's
 * opening turn restates the PyTorch module it replaces):
 *
 *   out_i = floor((L_i + 2 p_i - d_i (k_i - 1) - 1) / s_i) + 1        (per axis)
 *
 *   y[n,co,o] = bias[co]
 *             + sum_{c'<C_g} sum_{t} w[co,c',t] * xz[n, g(co) C_g + c', o s + t d - p]
 *
 * with C_g = C_in / groups, g(co) = co / (C_out / groups), the sums over every
 * kernel tap t (a 1- or 3-vector), and xz equal to x inside [0, L_i) on every
 * axis and 0 outside (zero padding: the pages load zeros for out-of-range
 * input). Products are formed and summed in double precision from the fp32
 * inputs; nothing is rounded back to fp32.
 *
 * Fused op (page l2_p24, opening turns): m = min over the chosen spatial axis of
 * the conv output (bias included before the min), then softmax over the channel
 * axis with the row maximum subtracted before exp (the page's softmax epilogue).
 * Non-finite values follow the PyTorch modules the pages replace: a NaN in the
 * conv output makes its minimum NaN (torch.min propagates it), and a NaN
 * minimum makes its whole softmax row NaN.
 *
 * Parallelism: OpenMP over (n, co) output planes only; the arithmetic order
 * inside one output is the plain nested loop above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_ARG (-1)
#define OR_ERR_EMPTY (-2)

static int64_t floor_div(int64_t a, int64_t b) { /* b > 0 */
    int64_t q = a / b;
    if ((a % b != 0) && (a < 0)) q -= 1;
    return q;
}

/* Output length of one axis; may be <= 0 for inputs shorter than the dilated kernel. */
int64_t oracle_out_len(int64_t L, int64_t k, int64_t s, int64_t d, int64_t p) {
    return floor_div(L + 2 * p - d * (k - 1) - 1, s) + 1;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* nd = 1: x [N,C_in,L], w [C_out,C_g,k]; nd = 2: x [N,C_in,H,W], w [C_out,C_g,kH,kW];
   nd = 3: x [N,C_in,D,H,W], w [C_out,C_g,kD,kH,kW].
 * y (double) is [N, C_out, out...]. bias may be NULL. Returns OR_OK or a negative code. */
int oracle_conv(int nd, const float *x, const int64_t *xs, const float *w, const int64_t *ws,
                const float *bias, const int *stride, const int *dilation, const int *padding,
                int groups, double *y) {
    if (nd < 1 || nd > 3) return OR_ERR_ARG;
    if (!x || !xs || !w || !ws || !stride || !dilation || !padding || !y) return OR_ERR_ARG;
    if (groups < 1) return OR_ERR_ARG;
    /* View every case as 3 spatial axes; a 1-D conv has D = H = 1 and kD = kH = 1,
       a 2-D conv D = 1 and kD = 1. */
    int64_t N = xs[0], Cin = xs[1], Cout = ws[0], Cg = ws[1];
    int64_t L[3], K[3], S[3], Dl[3], P[3], O[3];
    for (int a = 0; a < 3; a++) { L[a] = 1; K[a] = 1; S[a] = 1; Dl[a] = 1; P[a] = 0; }
    for (int a = 0; a < nd; a++) {
        int ax = 3 - nd + a;
        L[ax] = xs[2 + a]; K[ax] = ws[2 + a];
        S[ax] = stride[a]; Dl[ax] = dilation[a]; P[ax] = padding[a];
    }
    if (Cin % groups || Cout % groups || Cg != Cin / groups) return OR_ERR_ARG;
    for (int a = 0; a < 3; a++) {
        if (S[a] < 1 || Dl[a] < 1 || P[a] < 0 || K[a] < 1) return OR_ERR_ARG;
        O[a] = oracle_out_len(L[a], K[a], S[a], Dl[a], P[a]);
        if (O[a] < 1) return OR_ERR_EMPTY;
    }
    const int64_t coutg = Cout / groups;
    const int64_t kvol = K[0] * K[1] * K[2];
    const int64_t xplane = L[0] * L[1] * L[2];
    const int64_t oplane = O[0] * O[1] * O[2];

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t co = 0; co < Cout; co++) {
            const int64_t g = co / coutg;
            double *yp = y + (n * Cout + co) * oplane;
            for (int64_t od = 0; od < O[0]; od++)
            for (int64_t oh = 0; oh < O[1]; oh++)
            for (int64_t ow = 0; ow < O[2]; ow++) {
                double acc = bias ? (double)bias[co] : 0.0;
                for (int64_t cc = 0; cc < Cg; cc++) {
                    const int64_t ci = g * Cg + cc;
                    const float *xc = x + (n * Cin + ci) * xplane;
                    const float *wc = w + (co * Cg + cc) * kvol;
                    for (int64_t td = 0; td < K[0]; td++) {
                        int64_t id = od * S[0] + td * Dl[0] - P[0];
                        if (id < 0 || id >= L[0]) continue;
                        for (int64_t th = 0; th < K[1]; th++) {
                            int64_t ih = oh * S[1] + th * Dl[1] - P[1];
                            if (ih < 0 || ih >= L[1]) continue;
                            for (int64_t tw = 0; tw < K[2]; tw++) {
                                int64_t iw = ow * S[2] + tw * Dl[2] - P[2];
                                if (iw < 0 || iw >= L[2]) continue;
                                acc += (double)wc[(td * K[1] + th) * K[2] + tw] *
                                       (double)xc[(id * L[1] + ih) * L[2] + iw];
                            }
                        }
                    }
                }
                yp[(od * O[1] + oh) * O[2] + ow] = acc;
            }
        }
    }
    return OR_OK;
}

/* Fused oracle: out = softmax over dim 1 of (min over dim `min_dim` of conv3d(x)).
 * min_dim is 2, 3 or 4 (an axis of the 5-D conv output). out (double) has the
 * 4-D shape with that axis removed. The conv is computed in full by oracle_conv
 * (the composed definition), then reduced. */
int oracle_conv3d_min_softmax(const float *x, const int64_t *xs, const float *w, const int64_t *ws,
                              const float *bias, const int *stride, const int *dilation,
                              const int *padding, int groups, int min_dim, double *out) {
    if (min_dim < 2 || min_dim > 4) return OR_ERR_ARG;
    int64_t O[3];
    for (int a = 0; a < 3; a++) {
        if (stride[a] < 1 || dilation[a] < 1 || padding[a] < 0) return OR_ERR_ARG;
        O[a] = oracle_out_len(xs[2 + a], ws[2 + a], stride[a], dilation[a], padding[a]);
        if (O[a] < 1) return OR_ERR_EMPTY;
    }
    const int64_t N = xs[0], C = ws[0];
    const int64_t vol = O[0] * O[1] * O[2];
    double *conv = (double *)malloc(sizeof(double) * (size_t)(N * C * vol));
    if (!conv) return OR_ERR_ARG;
    int rc = oracle_conv(3, x, xs, w, ws, bias, stride, dilation, padding, groups, conv);
    if (rc != OR_OK) { free(conv); return rc; }
    const int r = min_dim - 2;             /* reduced spatial axis */
    const int64_t R = O[r];
    int64_t keep[2], nk = 0;
    for (int a = 0; a < 3; a++) if (a != r) keep[nk++] = O[a];
    const int64_t rest = keep[0] * keep[1];
    int64_t st[3] = {O[1] * O[2], O[2], 1};  /* strides of (od, oh, ow) in one plane */

    /* m[n, c, rest] = min over the reduced axis */
    double *m = (double *)malloc(sizeof(double) * (size_t)(N * C * rest));
    if (!m) { free(conv); return OR_ERR_ARG; }
#pragma omp parallel for collapse(2)
    for (int64_t n = 0; n < N; n++)
        for (int64_t c = 0; c < C; c++) {
            const double *cp = conv + (n * C + c) * vol;
            for (int64_t i0 = 0; i0 < keep[0]; i0++)
                for (int64_t i1 = 0; i1 < keep[1]; i1++) {
                    int64_t base;
                    int64_t s0, s1;
                    if (r == 0) { s0 = st[1]; s1 = st[2]; }
                    else if (r == 1) { s0 = st[0]; s1 = st[2]; }
                    else { s0 = st[0]; s1 = st[1]; }
                    base = i0 * s0 + i1 * s1;
                    /* A NaN anywhere along the axis makes the minimum NaN, as
                       torch.min does (the module the page replaces). */
                    double v = cp[base];
                    for (int64_t j = 1; j < R; j++) {
                        double u = cp[base + j * st[r]];
                        if (u < v || isnan(u)) v = u;
                        if (isnan(v)) break;
                    }
                    m[(n * C + c) * rest + i0 * keep[1] + i1] = v;
                }
        }
    /* softmax over c with the maximum subtracted */
#pragma omp parallel for collapse(2)
    for (int64_t n = 0; n < N; n++)
        for (int64_t i = 0; i < rest; i++) {
            double mx = -INFINITY;
            for (int64_t c = 0; c < C; c++) {
                double v = m[(n * C + c) * rest + i];
                if (v > mx) mx = v;
            }
            double s = 0.0;
            for (int64_t c = 0; c < C; c++) s += exp(m[(n * C + c) * rest + i] - mx);
            for (int64_t c = 0; c < C; c++)
                out[(n * C + c) * rest + i] = exp(m[(n * C + c) * rest + i] - mx) / s;
        }
    free(m);
    free(conv);
    return OR_OK;
}

/* The fused op's last two steps on their own, as the unfused form runs them
 * after a separate conv (page l2_p24, opening turns: torch.min over `dim` of
 * the conv output, then torch.softmax over dim 1).
 *
 * oracle_min_axis: y is a 5-D fp32 tensor [N, C, D, H, W] (ys: 5 entries),
 * dim in {2, 3, 4}; out (fp32) is y's shape with that axis removed and holds
 * the minimum along it. A minimum rounds nothing, so fp32 is exact. A NaN
 * anywhere along the axis makes the result NaN (torch.min propagates it). */
int oracle_min_axis(const float *y, const int64_t *ys, int dim, float *out) {
    if (dim < 2 || dim > 4) return OR_ERR_ARG;
    for (int a = 0; a < 5; a++) if (ys[a] < 1) return OR_ERR_ARG;
    /* y viewed as [outer, R, inner] with R the reduced axis */
    int64_t outer = 1, inner = 1;
    for (int a = 0; a < dim; a++) outer *= ys[a];
    for (int a = dim + 1; a < 5; a++) inner *= ys[a];
    const int64_t R = ys[dim];
#pragma omp parallel for
    for (int64_t o = 0; o < outer; o++)
        for (int64_t i = 0; i < inner; i++) {
            const float *p = y + o * R * inner + i;
            float v = p[0];
            for (int64_t j = 1; j < R && !isnan(v); j++) {
                const float u = p[j * inner];
                if (u < v || isnan(u)) v = u;
            }
            out[o * inner + i] = v;
        }
    return OR_OK;
}

/* oracle_softmax_channels: z [N, C, S] fp32 (zs: 3 entries; S is the product
 * of the trailing axes), out (double) the same shape:
 *   out[n,c,s] = exp(z[n,c,s] - M) / sum_c' exp(z[n,c',s] - M),  M = max_c z[n,c,s]
 * in double precision. A NaN among a position's channels makes all of its
 * outputs NaN, as torch.softmax gives. */
int oracle_softmax_channels(const float *z, const int64_t *zs, double *out) {
    for (int a = 0; a < 3; a++) if (zs[a] < 1) return OR_ERR_ARG;
    const int64_t N = zs[0], C = zs[1], S = zs[2];
#pragma omp parallel for collapse(2)
    for (int64_t n = 0; n < N; n++)
        for (int64_t s = 0; s < S; s++) {
            const float *p = z + n * C * S + s;
            double *q = out + n * C * S + s;
            int has_nan = 0;
            double mx = -INFINITY;
            for (int64_t c = 0; c < C; c++) {
                const double v = p[c * S];
                if (isnan(v)) has_nan = 1;
                else if (v > mx) mx = v;
            }
            if (has_nan) {
                for (int64_t c = 0; c < C; c++) q[c * S] = NAN;
                continue;
            }
            double sum = 0.0;
            for (int64_t c = 0; c < C; c++) sum += exp((double)p[c * S] - mx);
            for (int64_t c = 0; c < C; c++) q[c * S] = exp((double)p[c * S] - mx) / sum;
        }
    return OR_OK;
}
