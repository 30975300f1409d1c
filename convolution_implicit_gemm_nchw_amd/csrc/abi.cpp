// abi.cpp -- the C entry points declared in include/miconv.h: argument
// validation (before anything is enqueued), plan choice, launch.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include "../../include/miconv.h"
#include "launch.h"
#include "nd.h"
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

namespace {

// Pointer checks of a call that runs plan `pl` (the problem is already
// validated): non-null, 16-byte aligned, the output disjoint from the inputs,
// the workspace part the plan touches and the bias.
int check_buffers(const Problem &p, const Plan &pl, const void *in0, const void *in1, const void *out,
                  const void *ws, size_t ws_bytes, const Epi *epi) {
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
    if (overlaps(out, bo, in0, b0) || overlaps(out, bo, in1, b1) || overlaps(out, bo, ws, pl.ws_used))
        return MICONV_ERR_ALIAS;
    if (epi && epi->bias) {
        // one bias value per output channel: K for the forward, C for backward-data
        const size_t nb = (size_t)(p.pass == FWD ? p.K : p.C) * 4;
        if (((uintptr_t)epi->bias & 3u) != 0) return MICONV_ERR_ALIGN;
        if (overlaps(out, bo, epi->bias, nb)) return MICONV_ERR_ALIAS;
    }
    return MICONV_OK;
}

}  // namespace

// Common body of the compute entry points.  in0/in1/out follow the
// pass's reading: forward (x, w, y), backward-data (dy, w, dx),
// backward-filter (x, dy, dW).  The plan comes from the plan cache (a tuned
// plan for these sizes when it fits the budget, else the default choice).
int miconv::run_problem(const Problem &p, const void *in0, const void *in1, float *out, void *ws, size_t ws_bytes,
                        void *stream, const Epi *epi) {
    int st = validate_problem(p);
    if (st != MICONV_OK) return st;
    if (!ws && ws_bytes > 0) return MICONV_ERR_NULL;
    Plan pl;
    cached_plan(p, ws ? ws_bytes : 0, &pl);
    st = check_buffers(p, pl, in0, in1, out, ws, ws_bytes, epi);
    if (st != MICONV_OK) return st;
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
        case MICONV_ERR_INDEX: return "plan candidate index out of range";
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
    cached_plan(p, workspace_limit, &pl);
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
    cached_plan(p, workspace_bytes, &pl);
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

int miconv_plan_candidates(int pass, int dtype, int N, int C, int H, int W, int K, int R, int S, int pad_h,
                           int pad_w, int stride_h, int stride_w, int P, int Q, size_t workspace_limit, int *count,
                           size_t *max_workspace_bytes) {
    if (!count) return MICONV_ERR_NULL;
    Problem p;
    int st = problem_from_pass(pass, dtype, N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w, P, Q, &p);
    if (st == MICONV_OK) st = validate_problem(p);
    if (st != MICONV_OK) return st;
    Plan c[kMaxCandidates];
    *count = enumerate_plans(p, workspace_limit, c, kMaxCandidates);
    if (max_workspace_bytes) {
        *max_workspace_bytes = 0;
        for (int i = 0; i < *count; ++i)
            if (c[i].ws_used > *max_workspace_bytes) *max_workspace_bytes = c[i].ws_used;
    }
    return MICONV_OK;
}

int miconv_plan_select(int pass, int dtype, int N, int C, int H, int W, int K, int R, int S, int pad_h, int pad_w,
                       int stride_h, int stride_w, int P, int Q, size_t workspace_limit, int index) {
    Problem p;
    int st = problem_from_pass(pass, dtype, N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w, P, Q, &p);
    if (st == MICONV_OK) st = validate_problem(p);
    if (st != MICONV_OK) return st;
    if (index < 0) {
        drop_tuned_plan(p);
        return MICONV_OK;
    }
    Plan c[kMaxCandidates];
    const int n = enumerate_plans(p, workspace_limit, c, kMaxCandidates);
    if (index >= n) return MICONV_ERR_INDEX;
    set_tuned_plan(p, c[index]);
    return MICONV_OK;
}

int miconv_plan_cache_clear(void) {
    clear_plan_cache();
    return MICONV_OK;
}

int miconv_plan_cache_entries(int *tuned, int *total) {
    if (!tuned || !total) return MICONV_ERR_NULL;
    plan_cache_counts(tuned, total);
    return MICONV_OK;
}

int miconv_find_plan(int pass, int dtype, int N, int C, int H, int W, int K, int R, int S, int pad_h, int pad_w,
                     int stride_h, int stride_w, int P, int Q, const void *in0, const void *in1, void *out,
                     void *workspace, size_t workspace_bytes, void *stream, int requested, int *returned,
                     miconv_perf_t *perf) {
    if (!returned || (requested > 0 && !perf)) return MICONV_ERR_NULL;
    *returned = 0;
    Problem p;
    int st = problem_from_pass(pass, dtype, N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w, P, Q, &p);
    if (st == MICONV_OK) st = validate_problem(p);
    if (st != MICONV_OK) return st;
    if (!workspace && workspace_bytes > 0) return MICONV_ERR_NULL;
    // the deconvolution backward-weights call reads its activations the other way round
    if (pass == MICONV_DECONV_BWD_FILTER) {
        const void *t = in0;
        in0 = in1;
        in1 = t;
    }
    const size_t budget = workspace ? workspace_bytes : 0;
    Plan c[kMaxCandidates];
    const int n = enumerate_plans(p, budget, c, kMaxCandidates);
    for (int i = 0; i < n; ++i) {
        st = check_buffers(p, c[i], in0, in1, out, workspace, workspace_bytes, nullptr);
        if (st != MICONV_OK) return st;
    }
    hipStream_t s = (hipStream_t)stream;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        return MICONV_ERR_HIP;
    }
    // every candidate once untimed, then rounds of kReps back-to-back launches
    // per candidate; a candidate's time is its best round's mean
    constexpr int kRounds = 3, kReps = 3;
    float best[kMaxCandidates];
    int status[kMaxCandidates];
    for (int i = 0; i < n; ++i) {
        best[i] = -1.0f;
        status[i] = launch_plan(c[i], p, in0, in1, (float *)out, workspace, s, nullptr);
    }
    int hip_fail = hipStreamSynchronize(s) != hipSuccess;
    for (int r = 0; r < kRounds && !hip_fail; ++r)
        for (int i = 0; i < n && !hip_fail; ++i) {
            if (status[i] != MICONV_OK) continue;
            hip_fail |= hipEventRecord(e0, s) != hipSuccess;
            for (int k = 0; k < kReps && status[i] == MICONV_OK; ++k)
                status[i] = launch_plan(c[i], p, in0, in1, (float *)out, workspace, s, nullptr);
            hip_fail |= hipEventRecord(e1, s) != hipSuccess;
            hip_fail |= hipEventSynchronize(e1) != hipSuccess;
            float ms = 0.0f;
            if (!hip_fail && status[i] == MICONV_OK && hipEventElapsedTime(&ms, e0, e1) == hipSuccess) {
                ms /= kReps;
                if (best[i] < 0.0f || ms < best[i]) best[i] = ms;
            }
        }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (hip_fail) return MICONV_ERR_HIP;
    // order: successful candidates by time, then the failed ones
    int order[kMaxCandidates];
    for (int i = 0; i < n; ++i) order[i] = i;
    for (int i = 1; i < n; ++i)
        for (int j = i; j > 0; --j) {
            const int a = order[j - 1], b = order[j];
            const bool a_ok = status[a] == MICONV_OK && best[a] >= 0.0f, b_ok = status[b] == MICONV_OK && best[b] >= 0.0f;
            if ((b_ok && !a_ok) || (a_ok && b_ok && best[b] < best[a])) {
                order[j - 1] = b;
                order[j] = a;
            }
        }
    const int first = order[0];
    if (n > 0 && status[first] == MICONV_OK && best[first] >= 0.0f) set_tuned_plan(p, c[first]);
    const int m = requested < n ? requested : n;
    for (int i = 0; i < m; ++i) {
        const int k = order[i];
        perf[i].index = k;
        perf[i].status = status[k] == MICONV_OK && best[k] < 0.0f ? MICONV_ERR_HIP : status[k];
        perf[i].time_ms = best[k];
        perf[i].workspace_bytes = c[k].ws_used;
        describe_plan(c[k], perf[i].plan, sizeof perf[i].plan);
    }
    *returned = m;
    return MICONV_OK;
}

}  // extern "C"

namespace {

int nd_problem(int pass, const miconv_nd_desc_t *d, int dtype, NdProblem *p) {
    if (!d) return MICONV_ERR_NULL;
    int st = nd_from_desc(pass, dtype, d->ndim, d->N, d->C, d->K, d->groups, d->in, d->filter, d->out, d->pad_lo,
                          d->pad_hi, d->stride, d->dilation, p);
    return st == MICONV_OK ? validate_nd(*p) : st;
}

// Body of the generalised entry points: the 2-D kernels for plain 2-D / 1-D
// problems, else the generic kernel.  in0/in1/out as in run_problem.
int run_nd(int pass, const miconv_nd_desc_t *d, int dtype, const void *in0, const void *in1, float *out, void *ws,
           size_t ws_bytes, void *stream) {
    NdProblem p;
    int st = nd_problem(pass, d, dtype, &p);
    if (st != MICONV_OK) return st;
    Problem q;
    if (nd_as_2d(p, &q)) return run_problem(q, in0, in1, out, ws, ws_bytes, stream);
    if (!in0 || !in1 || !out) return MICONV_ERR_NULL;
    if (!ws && ws_bytes > 0) return MICONV_ERR_NULL;
    if (misaligned(in0) || misaligned(in1) || misaligned(out) || (ws && misaligned(ws))) return MICONV_ERR_ALIGN;
    NdPlan pl;
    make_nd_plan(p, ws ? ws_bytes : 0, &pl);
    const size_t es = dtype == MICONV_BF16 ? 2 : 4;
    const size_t vin = (size_t)p.in[0] * p.in[1] * p.in[2], vout = (size_t)p.out[0] * p.out[1] * p.out[2];
    const size_t nx = (size_t)p.N * p.C * vin, ny = (size_t)p.N * p.K * vout;
    const size_t nw = (size_t)p.K * (p.C / p.G) * p.f[0] * p.f[1] * p.f[2];
    size_t b0, b1, bo;
    if (pass == FWD) {
        b0 = nx * es; b1 = nw * es; bo = ny * 4;
    } else if (pass == BWD_DATA) {
        b0 = ny * es; b1 = nw * es; bo = nx * 4;
    } else {
        b0 = nx * es; b1 = ny * es; bo = nw * 4;
    }
    if (overlaps(out, bo, in0, b0) || overlaps(out, bo, in1, b1) || overlaps(out, bo, ws, pl.ws_used))
        return MICONV_ERR_ALIAS;
    return launch_nd(p, pl, in0, in1, out, ws, (hipStream_t)stream);
}

}  // namespace

extern "C" {

int miconv_nd_padding(miconv_nd_desc_t *d, int mode) {
    if (!d) return MICONV_ERR_NULL;
    if (d->ndim < 1 || d->ndim > 3 || (mode != MICONV_PAD_VALID && mode != MICONV_PAD_SAME)) return MICONV_ERR_BAD_DIM;
    for (int i = 0; i < d->ndim; ++i) {
        if (d->in[i] <= 0 || d->filter[i] <= 0 || d->stride[i] <= 0 || d->dilation[i] <= 0) return MICONV_ERR_BAD_DIM;
        nd_padding(mode, d->in[i], d->filter[i], d->stride[i], d->dilation[i], &d->pad_lo[i], &d->pad_hi[i],
                   &d->out[i]);
        if (d->out[i] < 1) return MICONV_ERR_BAD_DIM;
    }
    return MICONV_OK;
}

int convnd_fwd(const miconv_nd_desc_t *d, int dtype, const void *x, const void *w, float *y, void *workspace,
               size_t workspace_bytes, void *stream) {
    return run_nd(FWD, d, dtype, x, w, y, workspace, workspace_bytes, stream);
}

int convnd_bwd_data(const miconv_nd_desc_t *d, int dtype, const void *dy, const void *w, float *dx,
                    void *workspace, size_t workspace_bytes, void *stream) {
    return run_nd(BWD_DATA, d, dtype, dy, w, dx, workspace, workspace_bytes, stream);
}

int convnd_bwd_filter(const miconv_nd_desc_t *d, int dtype, const void *x, const void *dy, float *dw,
                      void *workspace, size_t workspace_bytes, void *stream) {
    return run_nd(BWD_FILTER, d, dtype, x, dy, dw, workspace, workspace_bytes, stream);
}

int convnd_workspace_size(int pass, const miconv_nd_desc_t *d, int dtype, size_t workspace_limit,
                          size_t *bytes_out) {
    if (!bytes_out) return MICONV_ERR_NULL;
    if (pass < MICONV_FWD || pass > MICONV_BWD_FILTER) return MICONV_ERR_PASS;
    NdProblem p;
    int st = nd_problem(pass, d, dtype, &p);
    if (st != MICONV_OK) return st;
    Problem q;
    if (nd_as_2d(p, &q)) {
        Plan pl;
        cached_plan(q, workspace_limit, &pl);
        *bytes_out = pl.ws_used;
        return MICONV_OK;
    }
    NdPlan pl;
    make_nd_plan(p, workspace_limit, &pl);
    *bytes_out = pl.ws_used;
    return MICONV_OK;
}

int convnd_describe(int pass, const miconv_nd_desc_t *d, int dtype, size_t workspace_bytes, char *buf,
                    size_t buflen) {
    if (!buf || buflen == 0) return MICONV_ERR_NULL;
    buf[0] = 0;
    if (pass < MICONV_FWD || pass > MICONV_BWD_FILTER) return MICONV_ERR_PASS;
    NdProblem p;
    int st = nd_problem(pass, d, dtype, &p);
    if (st != MICONV_OK) return st;
    Problem q;
    if (nd_as_2d(p, &q)) {
        Plan pl;
        cached_plan(q, workspace_bytes, &pl);
        describe_plan(pl, buf, buflen);
        return MICONV_OK;
    }
    NdPlan pl;
    make_nd_plan(p, workspace_bytes, &pl);
    describe_nd_plan(p, pl, buf, buflen);
    return MICONV_OK;
}

}  // extern "C"

