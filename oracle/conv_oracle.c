/*
 * conv_oracle.c -- plain, slow, fp64 reference for 2-D convolution on NCHW
 * tensors with a KCRS filter: forward, backward-data, backward-filter, and
 * transposed-convolution (deconvolution) forward and its two backward passes.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the HIP library.
 * Only the test suite, the package smoke check and the benchmark's CPU
 * baseline leg load it.  It includes nothing from the HIP library and the
 * HIP library includes nothing from it.
 *
 * Every function is the plain definition written out as direct nested loops,
 * in double precision, with no blocking, tiling or reordering.
 *
 * The definition, as the pages give it:
 *   - The convolution descriptor is cross-correlation (the filter is not
 *     flipped), dilation 1 in both dimensions, one zero-padding amount per
 *     spatial dimension (pad_h, pad_w) and one stride per dimension
 *     [SystemDS "LibMatrixCuDNNConvolutionAlgorithm.java",
 *      allocateConvolutionDescriptor].
 *   - Input x is packed N x C x H x W ("nchw"), output y is packed
 *     N x K x P x Q ("nkpq"), filter is packed K x C x R x S with S fastest
 *     [same page, private constructor, allocateTensorDescriptor,
 *      allocateFilterDescriptor].
 *   - P and Q are passed in by the caller next to the other sizes
 *     [same page, the three factory methods' parameter lists]; the oracle
 *     takes them as given and only requires the caller to pass the value
 *     floor((H + 2 pad_h - R) / stride_h) + 1 (and likewise Q), which the
 *     Python wrapper checks.
 *   - The three passes are forward (x, W -> y), backward-filter (x, dy -> dW)
 *     and backward-data (W, dy -> dx) [same page, the three factory methods],
 *     each overwriting its output (alpha = 1, beta = 0)
 *     [FilterDescriptor.SetFilter4dDescriptor examples, Conv2D and
 *      Conv2DKernelsGradient].
 *   - Deconvolution forward is convolution backward-data with the weight
 *     tensor read as (deconv_in_channels, deconv_out_channels, h, w), i.e. as
 *     a KCRS filter with K = deconv_in and C = deconv_out, with no flip
 *     [MXNet "mkldnn_deconvolution.cc", MKLDNNDeconvFwd::Execute comment].
 *
 * Zero padding: x~(n,c,i,j) = x[n,c,i,j] when 0 <= i < H and 0 <= j < W,
 * and 0 otherwise.
 *
 * Parallelism: OpenMP over an output slice that one thread owns entirely, so
 * no two threads write the same element and results do not depend on the
 * thread count.
 */
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads the OpenMP runtime will use for a parallel region. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Forward: y[n,k,p,q] = sum_{c,r,s} W[k,c,r,s] * x~(n, c, p*sh - ph + r, q*sw - pw + s). */
void oracle_conv2d_fwd(const double *x, const double *w, double *y,
                       int N, int C, int H, int W, int K, int R, int S,
                       int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q) {
    long long NK = (long long)N * K;
#pragma omp parallel for schedule(static)
    for (long long nk = 0; nk < NK; ++nk) {
        int n = (int)(nk / K), k = (int)(nk % K);
        for (int p = 0; p < P; ++p) {
            for (int q = 0; q < Q; ++q) {
                double acc = 0.0;
                for (int c = 0; c < C; ++c) {
                    for (int r = 0; r < R; ++r) {
                        int i = p * stride_h - pad_h + r;
                        if (i < 0 || i >= H) continue;
                        for (int s = 0; s < S; ++s) {
                            int j = q * stride_w - pad_w + s;
                            if (j < 0 || j >= W) continue;
                            acc += w[(((size_t)k * C + c) * R + r) * S + s] *
                                   x[(((size_t)n * C + c) * H + i) * W + j];
                        }
                    }
                }
                y[(((size_t)n * K + k) * P + p) * Q + q] = acc;
            }
        }
    }
}

/*
 * Backward-data, written as the literal adjoint of the forward map (scatter
 * form): every forward product W[k,c,r,s] * x[n,c,i,j] that contributes to
 * y[n,k,p,q] sends dy[n,k,p,q] * W[k,c,r,s] back to dx[n,c,i,j].  Positions
 * of x that no filter window reaches receive 0.
 */
void oracle_conv2d_bwd_data(const double *dy, const double *w, double *dx,
                            int N, int C, int H, int W, int K, int R, int S,
                            int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q) {
    long long NC = (long long)N * C;
#pragma omp parallel for schedule(static)
    for (long long nc = 0; nc < NC; ++nc) {
        int n = (int)(nc / C), c = (int)(nc % C);
        double *out = dx + (size_t)nc * H * W;
        for (size_t e = 0; e < (size_t)H * W; ++e) out[e] = 0.0;
        for (int k = 0; k < K; ++k) {
            for (int p = 0; p < P; ++p) {
                for (int q = 0; q < Q; ++q) {
                    double g = dy[(((size_t)n * K + k) * P + p) * Q + q];
                    for (int r = 0; r < R; ++r) {
                        int i = p * stride_h - pad_h + r;
                        if (i < 0 || i >= H) continue;
                        for (int s = 0; s < S; ++s) {
                            int j = q * stride_w - pad_w + s;
                            if (j < 0 || j >= W) continue;
                            out[(size_t)i * W + j] += w[(((size_t)k * C + c) * R + r) * S + s] * g;
                        }
                    }
                }
            }
        }
    }
}

/* Backward-filter: dW[k,c,r,s] = sum_{n,p,q} dy[n,k,p,q] * x~(n, c, p*sh - ph + r, q*sw - pw + s). */
void oracle_conv2d_bwd_filter(const double *x, const double *dy, double *dw,
                              int N, int C, int H, int W, int K, int R, int S,
                              int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q) {
    long long KC = (long long)K * C;
#pragma omp parallel for schedule(static)
    for (long long kc = 0; kc < KC; ++kc) {
        int k = (int)(kc / C), c = (int)(kc % C);
        for (int r = 0; r < R; ++r) {
            for (int s = 0; s < S; ++s) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    for (int p = 0; p < P; ++p) {
                        int i = p * stride_h - pad_h + r;
                        if (i < 0 || i >= H) continue;
                        for (int q = 0; q < Q; ++q) {
                            int j = q * stride_w - pad_w + s;
                            if (j < 0 || j >= W) continue;
                            acc += dy[(((size_t)n * K + k) * P + p) * Q + q] *
                                   x[(((size_t)n * C + c) * H + i) * W + j];
                        }
                    }
                }
                dw[(((size_t)k * C + c) * R + r) * S + s] = acc;
            }
        }
    }
}

/*
 * Deconvolution (transposed convolution) forward:
 *   out = conv2d_bwd_data(dy := x_in, W := w) with K := C_in, C := C_out,
 *   H := H_out, W := W_out, P := H_in, Q := W_in; w is [C_in][C_out][R][S]
 *   and is used as it is (no flip, no copy).
 */
void oracle_deconv2d_fwd(const double *x_in, const double *w, double *out,
                         int N, int C_in, int H_in, int W_in, int C_out, int R, int S,
                         int pad_h, int pad_w, int stride_h, int stride_w, int H_out, int W_out) {
    oracle_conv2d_bwd_data(x_in, w, out, N, C_out, H_out, W_out, C_in, R, S,
                           pad_h, pad_w, stride_h, stride_w, H_in, W_in);
}

/*
 * Deconvolution backward-data: the adjoint of deconvolution forward in its
 * input, applied to the output gradient dout [N][C_out][H_out][W_out].  The
 * adjoint of "convolution backward-data" is convolution forward, so
 *   din = conv2d_fwd(x := dout, W := w) with C := C_out, H := H_out,
 *   W := W_out, K := C_in, P := H_in, Q := W_in, giving [N][C_in][H_in][W_in]
 * [MXNet "mkldnn_deconvolution.cc", MKLDNNDeconvFwd::Execute comment:
 *  deconvolution backward data = convolution forward; MKLDNNDeconvBwd::
 *  ScheduleBwdData takes the output gradient and the weights].
 */
void oracle_deconv2d_bwd_data(const double *dout, const double *w, double *din,
                              int N, int C_in, int H_in, int W_in, int C_out, int R, int S,
                              int pad_h, int pad_w, int stride_h, int stride_w, int H_out, int W_out) {
    oracle_conv2d_fwd(dout, w, din, N, C_out, H_out, W_out, C_in, R, S,
                      pad_h, pad_w, stride_h, stride_w, H_in, W_in);
}

/*
 * Deconvolution backward-weights: the adjoint of deconvolution forward in w,
 * applied to dout.  With the same role swap this is convolution
 * backward-filter with x := dout (C_out channels at H_out x W_out) and
 * dy := x_in (C_in channels at H_in x W_in), whose [K][C][R][S] result is
 * [C_in][C_out][R][S], the deconvolution weight layout
 * [MXNet "mkldnn_deconvolution.cc", MKLDNNDeconvBwd::ScheduleBwdWeights:
 *  output gradient and input data in, weight gradient out].
 */
void oracle_deconv2d_bwd_filter(const double *x_in, const double *dout, double *dw,
                                int N, int C_in, int H_in, int W_in, int C_out, int R, int S,
                                int pad_h, int pad_w, int stride_h, int stride_w, int H_out, int W_out) {
    oracle_conv2d_bwd_filter(dout, x_in, dw, N, C_out, H_out, W_out, C_in, R, S,
                             pad_h, pad_w, stride_h, stride_w, H_in, W_in);
}

/*
 * Point evaluators: the same definitions evaluated at a list of flat output
 * indices only, for sampled comparisons at sizes where the full oracle would
 * take too long.  Backward-data is evaluated in gather form: dx[n,c,i,j]
 * collects W[k,c,r,s] * dy[n,k,p,q] over every (k,r,s) and every output
 * position (p,q) whose window puts tap (r,s) on (i,j), i.e.
 * p*sh - ph + r == i and q*sw - pw + s == j.
 */
void oracle_conv2d_fwd_points(const double *x, const double *w, const int64_t *idx, int count,
                              double *out,
                              int N, int C, int H, int W, int K, int R, int S,
                              int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q) {
    (void)N;
#pragma omp parallel for schedule(static)
    for (int e = 0; e < count; ++e) {
        int64_t t = idx[e];
        int q = (int)(t % Q); t /= Q;
        int p = (int)(t % P); t /= P;
        int k = (int)(t % K); t /= K;
        int n = (int)t;
        double acc = 0.0;
        for (int c = 0; c < C; ++c)
            for (int r = 0; r < R; ++r) {
                int i = p * stride_h - pad_h + r;
                if (i < 0 || i >= H) continue;
                for (int s = 0; s < S; ++s) {
                    int j = q * stride_w - pad_w + s;
                    if (j < 0 || j >= W) continue;
                    acc += w[(((size_t)k * C + c) * R + r) * S + s] *
                           x[(((size_t)n * C + c) * H + i) * W + j];
                }
            }
        out[e] = acc;
    }
}

void oracle_conv2d_bwd_data_points(const double *dy, const double *w, const int64_t *idx, int count,
                                   double *out,
                                   int N, int C, int H, int W, int K, int R, int S,
                                   int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q) {
    (void)N;
#pragma omp parallel for schedule(static)
    for (int e = 0; e < count; ++e) {
        int64_t t = idx[e];
        int j = (int)(t % W); t /= W;
        int i = (int)(t % H); t /= H;
        int c = (int)(t % C); t /= C;
        int n = (int)t;
        double acc = 0.0;
        for (int k = 0; k < K; ++k)
            for (int p = 0; p < P; ++p) {
                int r = i + pad_h - p * stride_h;
                if (r < 0 || r >= R) continue;
                for (int q = 0; q < Q; ++q) {
                    int s = j + pad_w - q * stride_w;
                    if (s < 0 || s >= S) continue;
                    acc += w[(((size_t)k * C + c) * R + r) * S + s] *
                           dy[(((size_t)n * K + k) * P + p) * Q + q];
                }
            }
        out[e] = acc;
    }
}

void oracle_conv2d_bwd_filter_points(const double *x, const double *dy, const int64_t *idx, int count,
                                     double *out,
                                     int N, int C, int H, int W, int K, int R, int S,
                                     int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q) {
#pragma omp parallel for schedule(static)
    for (int e = 0; e < count; ++e) {
        int64_t t = idx[e];
        int s = (int)(t % S); t /= S;
        int r = (int)(t % R); t /= R;
        int c = (int)(t % C); t /= C;
        int k = (int)t;
        double acc = 0.0;
        for (int n = 0; n < N; ++n)
            for (int p = 0; p < P; ++p) {
                int i = p * stride_h - pad_h + r;
                if (i < 0 || i >= H) continue;
                for (int q = 0; q < Q; ++q) {
                    int j = q * stride_w - pad_w + s;
                    if (j < 0 || j >= W) continue;
                    acc += dy[(((size_t)n * K + k) * P + p) * Q + q] *
                           x[(((size_t)n * C + c) * H + i) * W + j];
                }
            }
        out[e] = acc;
    }
}
