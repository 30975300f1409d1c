// abi.cpp -- the C entry points declared in include/miconv.h: argument
// validation (before anything is enqueued), plan choice, launch.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include "../../include/miconv.h"
#include "launch.h"
#include "plan.h"

using namespace miconv;

namespace {

bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

Problem make_problem(int pass, int dtype, int N, int C, int H, int W, int K, int R, int S, int ph, int pw,
                     int sh, int sw, int P, int Q) {
    Problem p;
    p.pass = pass;
    p.dtype = dtype;
    p.N = N; p.C = C; p.H = H; p.W = W; p.K = K; p.R = R; p.S = S;
    p.ph = ph; p.pw = pw; p.sh = sh; p.sw = sw; p.P = P; p.Q = Q;
    return p;
}

// Maps the public pass id and its 13 sizes to the convolution problem (the
// deconvolution passes read their sizes in deconv2d_fwd's order and swap them
// into the convolution view: K = C_in, C = C_out).
int problem_from_pass(int pass, int dtype, int a0, int a1, int a2, int a3, int a4, int R, int S, int ph,
                      int pw, int sh, int sw, int a11, int a12, Problem *out) {
    switch (pass) {
        case MICONV_FWD:
            *out = make_problem(FWD, dtype, a0, a1, a2, a3, a4, R, S, ph, pw, sh, sw, a11, a12);
            return MICONV_OK;
        case MICONV_BWD_DATA:
            *out = make_problem(BWD_DATA, dtype, a0, a1, a2, a3, a4, R, S, ph, pw, sh, sw, a11, a12);
            return MICONV_OK;
        case MICONV_BWD_FILTER:
            *out = make_problem(BWD_FILTER, dtype, a0, a1, a2, a3, a4, R, S, ph, pw, sh, sw, a11, a12);
            return MICONV_OK;
        case MICONV_DECONV_FWD:
        case MICONV_DECONV_BWD_DATA:
        case MICONV_DECONV_BWD_FILTER: {
            // (N, C_in, H_in, W_in, C_out, ..., H_out, W_out) -> conv (N, C_out, H_out, W_out, K = C_in, P = H_in, Q = W_in);
            // deconvolution forward = convolution backward-data, its backward-data =
            // convolution forward, its backward-weights = convolution backward-filter
            const int cp = pass == MICONV_DECONV_FWD ? BWD_DATA : (pass == MICONV_DECONV_BWD_DATA ? FWD : BWD_FILTER);
            *out = make_problem(cp, dtype, a0, a4, a11, a12, a1, R, S, ph, pw, sh, sw, a2, a3);
            return MICONV_OK;
        }
        default:
            return MICONV_ERR_PASS;
    }
}

}  // namespace

// Common body of the compute entry points.  in0/in1/out follow the
// pass's reading: forward (x, w, y), backward-data (dy, w, dx),
// backward-filter (x, dy, dW).
int miconv::run_problem(const Problem &p, const void *in0, const void *in1, float *out, void *ws, size_t ws_bytes,
                        void *stream, const Epi *epi) {
    int st = validate_problem(p);
    if (st != MICONV_OK) return st;
    if (!in0 || !in1 || !out) return MICONV_ERR_NULL;
    if (!ws && ws_bytes > 0) return MICONV_ERR_NULL;
    if (misaligned(in0) || misaligned(in1) || misaligned(out) || (ws && misaligned(ws)))
        return MICONV_ERR_ALIGN;
    const size_t es = p.dtype == MICONV_BF16 ? 2 : 4;
    const size_t nchw = (size_t)p.N * p.C * p.H * p.W, nkpq = (size_t)p.N * p.K * p.P * p.Q;
    const size_t kcrs = (size_t)p.K * p.C * p.R * p.S;
    const size_t oes = epi && epi->out_bf16 ? 2 : 4;   // output element bytes
    size_t b0, b1, bo;
    if (p.pass == FWD) {
        b0 = nchw * es; b1 = kcrs * es; bo = nkpq * oes;
    } else if (p.pass == BWD_DATA) {
        b0 = nkpq * es; b1 = kcrs * es; bo = nchw * oes;
    } else {
        b0 = nchw * es; b1 = nkpq * es; bo = kcrs * oes;
    }
    Plan pl;
    make_plan(p, ws ? ws_bytes : 0, &pl);
    if (overlaps(out, bo, in0, b0) || overlaps(out, bo, in1, b1) || overlaps(out, bo, ws, pl.ws_used))
        return MICONV_ERR_ALIAS;
    if (epi && epi->bias) {
        // one bias value per output channel: K for the forward, C for backward-data
        const size_t nb = (size_t)(p.pass == FWD ? p.K : p.C) * 4;
        if (((uintptr_t)epi->bias & 3u) != 0) return MICONV_ERR_ALIGN;
        if (overlaps(out, bo, epi->bias, nb)) return MICONV_ERR_ALIAS;
    }
    return launch_plan(pl, p, in0, in1, out, ws, (hipStream_t)stream, epi);
}

namespace {

int run(const Problem &p, const void *in0, const void *in1, float *out, void *ws, size_t ws_bytes,
        void *stream, const Epi *epi = nullptr) {
    return run_problem(p, in0, in1, out, ws, ws_bytes, stream, epi);
}

// A call with an output epilogue: the plain kernels when it is the identity
// (alpha 1, beta 0, no bias, no ReLU, fp32 out: bitwise the plain result).
int run_epi(const Problem &p, const void *in0, const void *in1, void *out, void *ws, size_t ws_bytes,
            void *stream, const float *bias, float alpha, float beta, int relu, int out_dtype) {
    if (out_dtype != MICONV_F32 && out_dtype != MICONV_BF16) return MICONV_ERR_DTYPE;
    if (alpha == 1.0f && beta == 0.0f && !bias && !relu && out_dtype == MICONV_F32)
        return run(p, in0, in1, (float *)out, ws, ws_bytes, stream);
    Epi e;
    e.bias = bias;
    e.alpha = alpha;
    e.beta = beta;
    e.relu = relu ? 1 : 0;
    e.out_bf16 = out_dtype == MICONV_BF16 ? 1 : 0;
    return run(p, in0, in1, (float *)out, ws, ws_bytes, stream, &e);
}

Problem deconv_problem(int pass, int dtype, int N, int C_in, int H_in, int W_in, int C_out, int R, int S,
                       int pad_h, int pad_w, int stride_h, int stride_w, int H_out, int W_out) {
    Problem p;
    problem_from_pass(pass, dtype, N, C_in, H_in, W_in, C_out, R, S, pad_h, pad_w, stride_h, stride_w, H_out,
                      W_out, &p);
    return p;
}

}  // namespace

extern "C" {

int miconv_abi_version(void) { return 3; }

const char *miconv_status_string(int status) {
    switch (status) {
        case MICONV_OK: return "ok";
        case MICONV_ERR_NULL: return "null pointer argument";
        case MICONV_ERR_BAD_DIM: return "invalid size, padding or stride";
        case MICONV_ERR_OUT_SIZE: return "output size does not match floor((in + 2*pad - filter)/stride) + 1";
        case MICONV_ERR_DTYPE: return "unsupported dtype (expected MICONV_F32 or MICONV_BF16)";
        case MICONV_ERR_ALIAS: return "output overlaps an input or the workspace";
        case MICONV_ERR_ALIGN: return "pointer not 16-byte aligned";
        case MICONV_ERR_WORKSPACE: return "workspace error";
        case MICONV_ERR_HIP: return "HIP launch or runtime error";
        case MICONV_ERR_PASS: return "unknown pass";
        case MICONV_ERR_TOO_LARGE: return "tensor too large (2 GiB or more)";
        default: return "unknown status";
    }
}

int miconv_workspace_size(int pass, int dtype, int N, int C, int H, int W, int K, int R, int S, int pad_h,
                          int pad_w, int stride_h, int stride_w, int P, int Q, size_t workspace_limit,
                          size_t *bytes_out) {
    if (!bytes_out) return MICONV_ERR_NULL;
    Problem p;
    int st = problem_from_pass(pass, dtype, N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w, P, Q, &p);
    if (st != MICONV_OK) return st;
    st = validate_problem(p);
    if (st != MICONV_OK) return st;
    Plan pl;
    make_plan(p, workspace_limit, &pl);
    *bytes_out = pl.ws_used;
    return MICONV_OK;
}

int miconv_plan_describe(int pass, int dtype, int N, int C, int H, int W, int K, int R, int S, int pad_h,
                         int pad_w, int stride_h, int stride_w, int P, int Q, size_t workspace_bytes, char *buf,
                         size_t buflen) {
    if (!buf || buflen == 0) return MICONV_ERR_NULL;
    buf[0] = 0;
    Problem p;
    int st = problem_from_pass(pass, dtype, N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w, P, Q, &p);
    if (st != MICONV_OK) return st;
    st = validate_problem(p);
    if (st != MICONV_OK) return st;
    Plan pl;
    make_plan(p, workspace_bytes, &pl);
    describe_plan(pl, buf, buflen);
    return MICONV_OK;
}

int conv2d_fwd(int N, int C, int H, int W, int K, int R, int S, int pad_h, int pad_w, int stride_h, int stride_w,
               int P, int Q, int dtype, const void *x, const void *w, float *y, void *workspace,
               size_t workspace_bytes, void *stream) {
    Problem p = make_problem(FWD, dtype, N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w, P, Q);
    return run(p, x, w, y, workspace, workspace_bytes, stream);
}

int conv2d_fwd_ex(int N, int C, int H, int W, int K, int R, int S, int pad_h, int pad_w, int stride_h,
                  int stride_w, int P, int Q, int dtype, const void *x, const void *w, const float *bias, float alpha,
                  float beta, int relu, int out_dtype, void *y, void *workspace, size_t workspace_bytes,
                  void *stream) {
    Problem p = make_problem(FWD, dtype, N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w, P, Q);
    return run_epi(p, x, w, y, workspace, workspace_bytes, stream, bias, alpha, beta, relu, out_dtype);
}

int conv2d_bwd_data(int N, int C, int H, int W, int K, int R, int S, int pad_h, int pad_w, int stride_h,
                    int stride_w, int P, int Q, int dtype, const void *dy, const void *w, float *dx,
                    void *workspace, size_t workspace_bytes, void *stream) {
    Problem p = make_problem(BWD_DATA, dtype, N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w, P, Q);
    return run(p, dy, w, dx, workspace, workspace_bytes, stream);
}

int conv2d_bwd_filter(int N, int C, int H, int W, int K, int R, int S, int pad_h, int pad_w, int stride_h,
                      int stride_w, int P, int Q, int dtype, const void *x, const void *dy, float *dw,
                      void *workspace, size_t workspace_bytes, void *stream) {
    Problem p = make_problem(BWD_FILTER, dtype, N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w, P, Q);
    return run(p, x, dy, dw, workspace, workspace_bytes, stream);
}

int deconv2d_fwd(int N, int C_in, int H_in, int W_in, int C_out, int R, int S, int pad_h, int pad_w,
                 int stride_h, int stride_w, int H_out, int W_out, int dtype, const void *x, const void *w,
                 float *y, void *workspace, size_t workspace_bytes, void *stream) {
    Problem p;
    problem_from_pass(MICONV_DECONV_FWD, dtype, N, C_in, H_in, W_in, C_out, R, S, pad_h, pad_w, stride_h,
                      stride_w, H_out, W_out, &p);
    return run(p, x, w, y, workspace, workspace_bytes, stream);
}

// dy [N][C_out][H_out][W_out] is the forward convolution's x; dx is its y
int deconv2d_bwd_data(int N, int C_in, int H_in, int W_in, int C_out, int R, int S, int pad_h, int pad_w,
                      int stride_h, int stride_w, int H_out, int W_out, int dtype, const void *dy, const void *w,
                      float *dx, void *workspace, size_t workspace_bytes, void *stream) {
    Problem p;
    problem_from_pass(MICONV_DECONV_BWD_DATA, dtype, N, C_in, H_in, W_in, C_out, R, S, pad_h, pad_w, stride_h,
                      stride_w, H_out, W_out, &p);
    return run(p, dy, w, dx, workspace, workspace_bytes, stream);
}

// backward-filter with x := dy (C_out channels) and dy := x (C_in channels)
int deconv2d_bwd_filter(int N, int C_in, int H_in, int W_in, int C_out, int R, int S, int pad_h, int pad_w,
                        int stride_h, int stride_w, int H_out, int W_out, int dtype, const void *x, const void *dy,
                        float *dw, void *workspace, size_t workspace_bytes, void *stream) {
    Problem p;
    problem_from_pass(MICONV_DECONV_BWD_FILTER, dtype, N, C_in, H_in, W_in, C_out, R, S, pad_h, pad_w, stride_h,
                      stride_w, H_out, W_out, &p);
    return run(p, dy, x, dw, workspace, workspace_bytes, stream);
}

int conv2d_bwd_data_ex(int N, int C, int H, int W, int K, int R, int S, int pad_h, int pad_w, int stride_h,
                       int stride_w, int P, int Q, int dtype, const void *dy, const void *w, float alpha, float beta,
                       int out_dtype, void *dx, void *workspace, size_t workspace_bytes, void *stream) {
    Problem p = make_problem(BWD_DATA, dtype, N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w, P, Q);
    return run_epi(p, dy, w, dx, workspace, workspace_bytes, stream, nullptr, alpha, beta, 0, out_dtype);
}

int conv2d_bwd_filter_ex(int N, int C, int H, int W, int K, int R, int S, int pad_h, int pad_w, int stride_h,
                         int stride_w, int P, int Q, int dtype, const void *x, const void *dy, float alpha,
                         float beta, int out_dtype, void *dw, void *workspace, size_t workspace_bytes,
                         void *stream) {
    Problem p = make_problem(BWD_FILTER, dtype, N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w, P, Q);
    return run_epi(p, x, dy, dw, workspace, workspace_bytes, stream, nullptr, alpha, beta, 0, out_dtype);
}

int deconv2d_fwd_ex(int N, int C_in, int H_in, int W_in, int C_out, int R, int S, int pad_h, int pad_w,
                    int stride_h, int stride_w, int H_out, int W_out, int dtype, const void *x, const void *w,
                    const float *bias, float alpha, float beta, int relu, int out_dtype, void *y, void *workspace,
                    size_t workspace_bytes, void *stream) {
    Problem p = deconv_problem(MICONV_DECONV_FWD, dtype, N, C_in, H_in, W_in, C_out, R, S, pad_h, pad_w,
                               stride_h, stride_w, H_out, W_out);
    return run_epi(p, x, w, y, workspace, workspace_bytes, stream, bias, alpha, beta, relu, out_dtype);
}

int deconv2d_bwd_data_ex(int N, int C_in, int H_in, int W_in, int C_out, int R, int S, int pad_h, int pad_w,
                         int stride_h, int stride_w, int H_out, int W_out, int dtype, const void *dy, const void *w,
                         float alpha, float beta, int out_dtype, void *dx, void *workspace, size_t workspace_bytes,
                         void *stream) {
    Problem p = deconv_problem(MICONV_DECONV_BWD_DATA, dtype, N, C_in, H_in, W_in, C_out, R, S, pad_h, pad_w,
                               stride_h, stride_w, H_out, W_out);
    return run_epi(p, dy, w, dx, workspace, workspace_bytes, stream, nullptr, alpha, beta, 0, out_dtype);
}

int deconv2d_bwd_filter_ex(int N, int C_in, int H_in, int W_in, int C_out, int R, int S, int pad_h, int pad_w,
                           int stride_h, int stride_w, int H_out, int W_out, int dtype, const void *x,
                           const void *dy, float alpha, float beta, int out_dtype, void *dw, void *workspace,
                           size_t workspace_bytes, void *stream) {
    Problem p = deconv_problem(MICONV_DECONV_BWD_FILTER, dtype, N, C_in, H_in, W_in, C_out, R, S, pad_h, pad_w,
                               stride_h, stride_w, H_out, W_out);
    return run_epi(p, dy, x, dw, workspace, workspace_bytes, stream, nullptr, alpha, beta, 0, out_dtype);
}

int conv2d_bwd_bias(int N, int K, int P, int Q, int dtype, const void *dy, float alpha, float beta, float *db,
                    void *stream) {
    if (!dy || !db) return MICONV_ERR_NULL;
    if (N <= 0 || K <= 0 || P <= 0 || Q <= 0) return MICONV_ERR_BAD_DIM;
    if (dtype != MICONV_F32 && dtype != MICONV_BF16) return MICONV_ERR_DTYPE;
    const size_t es = dtype == MICONV_BF16 ? 2 : 4;
    const size_t n = (size_t)N * K * P * Q;
    if ((size_t)P * Q >= (1u << 31) || n >= (1u << 31) || n * es >= (1ull << 31)) return MICONV_ERR_TOO_LARGE;
    if (misaligned(dy) || ((uintptr_t)db & 3u) != 0) return MICONV_ERR_ALIGN;
    if (overlaps(db, (size_t)K * 4, dy, n * es)) return MICONV_ERR_ALIAS;
    return launch_bias_grad(dtype, N, K, P * Q, dy, alpha, beta, db, (hipStream_t)stream);
}

}  // extern "C"
