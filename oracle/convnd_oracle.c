/*
 * convnd_oracle.c -- plain, slow, fp64 reference for the generalised
 * convolution: 1, 2 or 3 spatial dimensions, groups, dilation, separate low
 * and high zero padding per dimension, per-dimension strides; forward,
 * backward-data and backward-filter.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the HIP library.
 * Only the test suite, the package smoke check and the benchmark's CPU
 * baseline leg load it.  It includes nothing from the HIP library and the
 * HIP library includes nothing from it.
 *
 * Every function is the plain definition written out as direct nested loops
 * in double precision, with no blocking, tiling or reordering.
 *
 * Tensors (every problem is written in three spatial dimensions; a 2-D problem
 * has D = T = OD = 1 and a 1-D one also H = R = OH = 1, with pad 0, stride 1
 * and dilation 1 in the unused dimensions):
 *   x  [N][C][D][H][W],  w [K][C/G][T][R][S],  y [N][K][OD][OH][OW]
 * with G groups: output channel k belongs to group g = k / (K/G) and reads
 * only input channels g*(C/G) .. g*(C/G) + C/G - 1 (the grouped convolution of
 * the MXNet deconvolution's num_group).  The definition (cross-correlation,
 * zero padding) is the one of the 2-D oracle, with the filter taps spaced by
 * the dilation (MXNet DeconvDescCreator's dilates, which oneDNN takes minus
 * one) and the low padding placing the first window:
 *   x~(n, c, i, j, l) = x[n][c][i][j][l] inside the volume, 0 outside
 *   y[n,k,od,oh,ow] = sum_{c < C/G, t, r, s} w[k,c,t,r,s] *
 *       x~(n, g*C/G + c, od*sd - pd + t*dd, oh*sh - ph + r*dh, ow*sw - pw + s*dw)
 * The high padding enters only through the output sizes, which the caller
 * passes: OD = floor((D + pd_lo + pd_hi - dd*(T-1) - 1) / sd) + 1, likewise
 * OH and OW (checked by the Python wrapper).
 *
 * Size vector `z` (22 ints), in this order:
 *   N, C, K, G, D, H, W, T, R, S, OD, OH, OW,
 *   pad_d, pad_h, pad_w (low pads), stride_d, stride_h, stride_w,
 *   dil_d, dil_h, dil_w
 *
 * Parallelism: OpenMP over an output slice one thread owns entirely, so no
 * two threads write the same element and results do not depend on the
 * thread count.
 */
#include <stddef.h>
#include <stdint.h>

enum { ZN, ZC, ZK, ZG, ZD, ZH, ZW, ZT, ZR, ZS, ZOD, ZOH, ZOW, ZPD, ZPH, ZPW, ZSD, ZSH, ZSW, ZDD, ZDH, ZDW };

/* Forward: y = sum over the group's channels and the taps of w * x~. */
void oracle_convnd_fwd(const double *x, const double *w, double *y, const int *z) {
    const int N = z[ZN], C = z[ZC], K = z[ZK], G = z[ZG];
    const int D = z[ZD], H = z[ZH], W = z[ZW], T = z[ZT], R = z[ZR], S = z[ZS];
    const int OD = z[ZOD], OH = z[ZOH], OW = z[ZOW];
    const int Cg = C / G, Kg = K / G;
    long long NK = (long long)N * K;
#pragma omp parallel for schedule(static)
    for (long long nk = 0; nk < NK; ++nk) {
        int n = (int)(nk / K), k = (int)(nk % K), g = k / Kg;
        for (int od = 0; od < OD; ++od)
            for (int oh = 0; oh < OH; ++oh)
                for (int ow = 0; ow < OW; ++ow) {
                    double acc = 0.0;
                    for (int c = 0; c < Cg; ++c)
                        for (int t = 0; t < T; ++t) {
                            int i = od * z[ZSD] - z[ZPD] + t * z[ZDD];
                            if (i < 0 || i >= D) continue;
                            for (int r = 0; r < R; ++r) {
                                int j = oh * z[ZSH] - z[ZPH] + r * z[ZDH];
                                if (j < 0 || j >= H) continue;
                                for (int s = 0; s < S; ++s) {
                                    int l = ow * z[ZSW] - z[ZPW] + s * z[ZDW];
                                    if (l < 0 || l >= W) continue;
                                    acc += w[((((size_t)k * Cg + c) * T + t) * R + r) * S + s] *
                                           x[((((size_t)n * C + g * Cg + c) * D + i) * H + j) * W + l];
                                }
                            }
                        }
                    y[((((size_t)n * K + k) * OD + od) * OH + oh) * OW + ow] = acc;
                }
    }
}

/*
 * Backward-data as the literal adjoint of the forward map (scatter form):
 * every forward product w[k,c,t,r,s] * x[n, g*C/G + c, i, j, l] sends
 * dy[n,k,od,oh,ow] * w[k,c,t,r,s] back to dx[n, g*C/G + c, i, j, l].
 * Positions no window reaches receive 0.
 */
void oracle_convnd_bwd_data(const double *dy, const double *w, double *dx, const int *z) {
    const int N = z[ZN], C = z[ZC], K = z[ZK], G = z[ZG];
    const int D = z[ZD], H = z[ZH], W = z[ZW], T = z[ZT], R = z[ZR], S = z[ZS];
    const int OD = z[ZOD], OH = z[ZOH], OW = z[ZOW];
    const int Cg = C / G, Kg = K / G;
    long long NC = (long long)N * C;
#pragma omp parallel for schedule(static)
    for (long long nc = 0; nc < NC; ++nc) {
        int n = (int)(nc / C), ci = (int)(nc % C), g = ci / Cg, c = ci % Cg;
        double *out = dx + (size_t)nc * D * H * W;
        for (size_t e = 0; e < (size_t)D * H * W; ++e) out[e] = 0.0;
        for (int k = g * Kg; k < (g + 1) * Kg; ++k)
            for (int od = 0; od < OD; ++od)
                for (int oh = 0; oh < OH; ++oh)
                    for (int ow = 0; ow < OW; ++ow) {
                        double gr = dy[((((size_t)n * K + k) * OD + od) * OH + oh) * OW + ow];
                        for (int t = 0; t < T; ++t) {
                            int i = od * z[ZSD] - z[ZPD] + t * z[ZDD];
                            if (i < 0 || i >= D) continue;
                            for (int r = 0; r < R; ++r) {
                                int j = oh * z[ZSH] - z[ZPH] + r * z[ZDH];
                                if (j < 0 || j >= H) continue;
                                for (int s = 0; s < S; ++s) {
                                    int l = ow * z[ZSW] - z[ZPW] + s * z[ZDW];
                                    if (l < 0 || l >= W) continue;
                                    out[((size_t)i * H + j) * W + l] +=
                                        w[((((size_t)k * Cg + c) * T + t) * R + r) * S + s] * gr;
                                }
                            }
                        }
                    }
    }
}

/* Backward-filter: dw[k,c,t,r,s] = sum over n and the output positions of dy * x~. */
void oracle_convnd_bwd_filter(const double *x, const double *dy, double *dw, const int *z) {
    const int N = z[ZN], C = z[ZC], K = z[ZK], G = z[ZG];
    const int D = z[ZD], H = z[ZH], W = z[ZW], T = z[ZT], R = z[ZR], S = z[ZS];
    const int OD = z[ZOD], OH = z[ZOH], OW = z[ZOW];
    const int Cg = C / G, Kg = K / G;
    long long KC = (long long)K * Cg;
#pragma omp parallel for schedule(static)
    for (long long kc = 0; kc < KC; ++kc) {
        int k = (int)(kc / Cg), c = (int)(kc % Cg), g = k / Kg;
        for (int t = 0; t < T; ++t)
            for (int r = 0; r < R; ++r)
                for (int s = 0; s < S; ++s) {
                    double acc = 0.0;
                    for (int n = 0; n < N; ++n)
                        for (int od = 0; od < OD; ++od) {
                            int i = od * z[ZSD] - z[ZPD] + t * z[ZDD];
                            if (i < 0 || i >= D) continue;
                            for (int oh = 0; oh < OH; ++oh) {
                                int j = oh * z[ZSH] - z[ZPH] + r * z[ZDH];
                                if (j < 0 || j >= H) continue;
                                for (int ow = 0; ow < OW; ++ow) {
                                    int l = ow * z[ZSW] - z[ZPW] + s * z[ZDW];
                                    if (l < 0 || l >= W) continue;
                                    acc += dy[((((size_t)n * K + k) * OD + od) * OH + oh) * OW + ow] *
                                           x[((((size_t)n * C + g * Cg + c) * D + i) * H + j) * W + l];
                                }
                            }
                        }
                    dw[((((size_t)k * Cg + c) * T + t) * R + r) * S + s] = acc;
                }
    }
}
