/*
 * miconv.h -- C ABI of the MI355X (gfx950) implicit-GEMM convolution library.
 *
 * Operation (all entry points): 2-D cross-correlation convolution with
 * dilation 1, symmetric zero padding (pad_h, pad_w) and strides
 * (stride_h, stride_w), on packed NCHW activations and a packed KCRS filter
 * (S fastest).  This is the convolution descriptor, tensor descriptors and
 * filter descriptor of SystemDS "LibMatrixCuDNNConvolutionAlgorithm.java"
 * (allocateConvolutionDescriptor: cross-correlation, dilation (1,1);
 * allocateTensorDescriptor: NCHW; allocateFilterDescriptor: K, C, R, S).
 *
 *   P = floor((H + 2*pad_h - R) / stride_h) + 1,  Q = floor((W + 2*pad_w - S) / stride_w) + 1
 *   x~(n,c,i,j) = x[n,c,i,j] inside the image, 0 outside (padding)
 *
 *   forward          y[n,k,p,q]  = sum_{c,r,s} W[k,c,r,s] * x~(n, c, p*sh - ph + r, q*sw - pw + s)
 *   backward-data    dx[n,c,i,j] = sum_{k,r,s,p,q : p*sh-ph+r = i, q*sw-pw+s = j} W[k,c,r,s] * dy[n,k,p,q]
 *   backward-filter  dW[k,c,r,s] = sum_{n,p,q} dy[n,k,p,q] * x~(n, c, p*sh - ph + r, q*sw - pw + s)
 *
 * The three passes are the three factory methods of the same SystemDS page
 * (forward: x, W -> y; backward-filter: x, dy -> dW; backward-data: W, dy -> dx),
 * with the size arguments (N, C, H, W, K, R, S, pad_h, pad_w, stride_h,
 * stride_w, P, Q) and a workspace limit that the page caps at 1e9 bytes
 * (MAX_WORKSPACE_LIMIT_BYTES).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * dtype      MICONV_F32 or MICONV_BF16 names the element type of ALL inputs
 *            (x, W, dy).  Accumulation is fp32 and every output is fp32
 *            (the *_ex entry points can write bf16 instead).
 *            (The MXNet "mkldnn_deconvolution.cc" page, SupportMKLDNNDeconv,
 *            admits exactly these two input types.)
 * Layout     packed row-major: x [N][C][H][W], y / dy [N][K][P][Q],
 *            W / dW [K][C][R][S]; no stride arguments.
 * Writes     outputs are overwritten (alpha = 1, beta = 0, except in
 *            the *_ex entry points, which take alpha and beta; as the
 *            FilterDescriptor.SetFilter4dDescriptor examples page calls
 *            ConvolutionForward / ConvolutionBackwardFilter /
 *            ConvolutionBackwardData), including every dx position that no
 *            filter window reaches, which is written as 0.
 * Memory     every pointer is device memory of the current HIP device, owned
 *            by the caller; the library allocates no device memory.  Base
 *            pointers must be 16-byte aligned.  Each tensor must be smaller
 *            than 2 GiB.  Outputs must not overlap any input or the workspace.
 * Workspace  `workspace` / `workspace_bytes` is caller-provided scratch.  The
 *            library uses at most min(workspace_bytes, 1e9) bytes of it and
 *            picks the fastest plan that fits; any budget, including 0, is
 *            valid.  `workspace` may be NULL only when workspace_bytes is 0.
 *            miconv_workspace_size() reports what the preferred plan needs.
 * Stream     `stream` is a hipStream_t (NULL = the null stream).  Work is
 *            enqueued on it and the call returns without synchronising.
 * Errors     every argument is validated before anything is enqueued; an
 *            invalid call returns a non-zero status and touches no memory.
 *            A failed kernel launch returns MICONV_ERR_HIP.  Nothing aborts or
 *            throws across this boundary.
 * Plans     each call runs a plan (kernel family, tiling, split count) from a
 *            process-wide plan cache: the plan installed for its sizes by
 *            miconv_find_plan / miconv_plan_select when that plan's workspace
 *            fits min(workspace_bytes, 1e9), else the default choice for that
 *            budget.
 * Determinism for a fixed plan the results are bitwise reproducible (no
 *            atomics; split-K partial sums are reduced in a fixed order): so
 *            for fixed (pass, dtype, sizes, min(workspace_bytes, 1e9)) and no
 *            plan installed in between.  Different plans agree within the
 *            tolerance of the arithmetic, not bitwise.
 * Threads    calls are re-entrant and may come from several host threads.
 *            The library's mutable state is a per-process cache of plans and
 *            occupancy queries (guarded by a mutex; it changes no result) and
 *            the per-device scratch array of conv2d_bwd_filter_noalloc.
 */
#ifndef MICONV_H
#define MICONV_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input element types (outputs are always fp32). */
#define MICONV_F32 0
#define MICONV_BF16 1

/* Passes, for miconv_workspace_size. */
#define MICONV_FWD 0
#define MICONV_BWD_DATA 1
#define MICONV_BWD_FILTER 2
#define MICONV_DECONV_FWD 3
#define MICONV_DECONV_BWD_DATA 4
#define MICONV_DECONV_BWD_FILTER 5

/* Status codes. */
#define MICONV_OK 0
#define MICONV_ERR_NULL 1        /* a required pointer is NULL (or workspace NULL with bytes > 0) */
#define MICONV_ERR_BAD_DIM 2     /* a size <= 0, pad < 0, stride < 1, or filter larger than padded input */
#define MICONV_ERR_OUT_SIZE 3    /* P/Q (deconv: H_in/W_in) differ from the floor formula */
#define MICONV_ERR_DTYPE 4       /* dtype is neither MICONV_F32 nor MICONV_BF16 */
#define MICONV_ERR_ALIAS 5       /* the output overlaps an input or the workspace */
#define MICONV_ERR_ALIGN 6       /* a base pointer is not 16-byte aligned */
#define MICONV_ERR_WORKSPACE 7   /* reserved: no budget is ever rejected (plans adapt) */
#define MICONV_ERR_HIP 8         /* a HIP call or kernel launch failed */
#define MICONV_ERR_PASS 9        /* unknown pass id */
#define MICONV_ERR_TOO_LARGE 10  /* a tensor is 2 GiB or larger */
#define MICONV_ERR_INDEX 11      /* plan candidate index out of range */

/* The workspace cap of SystemDS MAX_WORKSPACE_LIMIT_BYTES (1e9 bytes). */
#define MICONV_MAX_WORKSPACE_BYTES 1000000000ull

/*
 * Bytes of workspace the preferred plan for this problem uses, given that at
 * most `workspace_limit` bytes are available (the library never uses more
 * than min(workspace_limit, 1e9)).  For the three MICONV_DECONV_* passes the
 * 13 sizes are read in deconv2d_fwd's order (N, C_in, H_in, W_in, C_out, R, S,
 * pad_h, pad_w, stride_h, stride_w, H_out, W_out).  Pure host computation.
 */
int miconv_workspace_size(int pass, int dtype, int N, int C, int H, int W, int K, int R, int S,
                          int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
                          size_t workspace_limit, size_t *bytes_out);

/*
 * Forward: y = conv(x, W).  x [N][C][H][W] (dtype), w [K][C][R][S] (dtype),
 * y [N][K][P][Q] fp32 (overwritten).  SystemDS page,
 * cudnnGetConvolutionForwardAlgorithm.
 */
int conv2d_fwd(int N, int C, int H, int W, int K, int R, int S,
               int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
               int dtype, const void *x, const void *w, float *y,
               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Forward with a fused epilogue:
 *   y[n,k,p,q] = act(alpha * conv(x, W)[n,k,p,q] + beta * y_prev[n,k,p,q] + bias[k])
 * where y_prev is y's content before the call and act is max(0, .) when
 * relu != 0 (a NaN becomes 0), the identity otherwise.  bias is fp32 [K] in
 * device memory, or NULL for none (4-byte aligned, must not overlap y).
 * y_prev is read only when beta != 0, so with beta == 0 y may hold anything.
 * out_dtype (MICONV_F32 or MICONV_BF16, else MICONV_ERR_DTYPE) is the element
 * type of y (and of y_prev): with MICONV_BF16 the fp32 result is rounded to
 * nearest even once, at the store, which halves the bytes written.
 * Sources: the alpha / beta output scaling of the cuDNN convolution calls on
 * the SystemDS page and the FilterDescriptor.SetFilter4dDescriptor examples
 * page; the per-output-channel bias tensor (1 x K x 1 x 1) and the ReLU
 * activation descriptor of that page's ConvolutionalLayer; the optional bias
 * of the MXNet deconvolution (DeconvDescCreator, MKLDNNDeconvFwd::Execute).
 * The epilogue is applied to the fp32 accumulators before the one store of
 * each output, so it adds no pass over y (one extra read of y when
 * beta != 0).  alpha == 1, beta == 0, no bias and no relu run the plain
 * forward's kernels.  Other arguments, validation and errors as conv2d_fwd.
 */
int conv2d_fwd_ex(int N, int C, int H, int W, int K, int R, int S,
                  int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
                  int dtype, const void *x, const void *w, const float *bias,
                  float alpha, float beta, int relu, int out_dtype, void *y,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward-data: dx = adjoint of the forward map in x, applied to dy.
 * dy [N][K][P][Q] (dtype), w [K][C][R][S] (dtype), dx [N][C][H][W] fp32
 * (overwritten, zeros where no window reaches).  SystemDS page,
 * cudnnGetConvolutionBackwardDataAlgorithm.
 */
int conv2d_bwd_data(int N, int C, int H, int W, int K, int R, int S,
                    int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
                    int dtype, const void *dy, const void *w, float *dx,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward-filter: dW = adjoint of the forward map in W, applied to dy.
 * x [N][C][H][W] (dtype), dy [N][K][P][Q] (dtype), dw [K][C][R][S] fp32
 * (overwritten).  SystemDS page, cudnnGetConvolutionBackwardFilterAlgorithm.
 */
int conv2d_bwd_filter(int N, int C, int H, int W, int K, int R, int S,
                      int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
                      int dtype, const void *x, const void *dy, float *dw,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Deconvolution (transposed convolution) forward.  x [N][C_in][H_in][W_in]
 * (dtype), w [C_in][C_out][R][S] (dtype), y [N][C_out][H_out][W_out] fp32
 * (overwritten).  Computed as conv2d_bwd_data with K := C_in, C := C_out,
 * H := H_out, W := W_out, P := H_in, Q := W_in, dy := x, and the weight used
 * as it is (no flip): MXNet "mkldnn_deconvolution.cc",
 * MKLDNNDeconvFwd::Execute (deconvolution forward = convolution backward
 * data; weights (deconv_in, deconv_out, h, w)).  H_out/W_out must satisfy
 * floor((H_out + 2*pad_h - R)/stride_h) + 1 == H_in (likewise W), else
 * MICONV_ERR_OUT_SIZE.
 */
int deconv2d_fwd(int N, int C_in, int H_in, int W_in, int C_out, int R, int S,
                 int pad_h, int pad_w, int stride_h, int stride_w, int H_out, int W_out,
                 int dtype, const void *x, const void *w, float *y,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Deconvolution backward-data: the adjoint of deconv2d_fwd in its input,
 * applied to the output gradient.  dy [N][C_out][H_out][W_out] (dtype),
 * w [C_in][C_out][R][S] (dtype), dx [N][C_in][H_in][W_in] fp32
 * (overwritten).  Computed as conv2d_fwd with C := C_out, H := H_out,
 * W := W_out, K := C_in, P := H_in, Q := W_in, x := dy and the weight used
 * as it is: MXNet "mkldnn_deconvolution.cc", MKLDNNDeconvFwd::Execute
 * (deconvolution backward data = convolution forward) and
 * MKLDNNDeconvBwd::ScheduleBwdData (output gradient, weights -> input
 * gradient).  Sizes, validation and errors as deconv2d_fwd.
 */
int deconv2d_bwd_data(int N, int C_in, int H_in, int W_in, int C_out, int R, int S,
                      int pad_h, int pad_w, int stride_h, int stride_w, int H_out, int W_out,
                      int dtype, const void *dy, const void *w, float *dx,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Deconvolution backward-weights: the adjoint of deconv2d_fwd in w, applied
 * to the output gradient.  x [N][C_in][H_in][W_in] (dtype, the deconvolution's
 * input), dy [N][C_out][H_out][W_out] (dtype), dw [C_in][C_out][R][S] fp32
 * (overwritten).  Computed as conv2d_bwd_filter with the same role swap
 * (x := dy with C_out channels, dy := x with C_in channels); its KCRS result
 * is the deconvolution weight layout.  MXNet "mkldnn_deconvolution.cc",
 * MKLDNNDeconvBwd::ScheduleBwdWeights (output gradient, input data -> weight
 * gradient).  Split-K partial sums use the workspace as for
 * conv2d_bwd_filter.  Sizes, validation and errors as deconv2d_fwd.
 */
int deconv2d_bwd_filter(int N, int C_in, int H_in, int W_in, int C_out, int R, int S,
                        int pad_h, int pad_w, int stride_h, int stride_w, int H_out, int W_out,
                        int dtype, const void *x, const void *dy, float *dw,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Output epilogue of the *_ex backward entry points (and of deconv2d_fwd_ex):
 *   out = act(alpha * result + beta * out_prev + bias[channel])
 * where result is what the plain entry point would write, out_prev is out's
 * content before the call (read only when beta != 0, so with beta == 0 out may
 * hold anything) and out_dtype (MICONV_F32 or MICONV_BF16, else
 * MICONV_ERR_DTYPE) is the element type of out and out_prev; with MICONV_BF16
 * the fp32 value is rounded to nearest even once, at the store.  bias and act
 * exist only in deconv2d_fwd_ex.  Every output element is written exactly once
 * (dx positions no window reaches get alpha * 0 + beta * out_prev + bias).
 * beta = 0 overwrites (MXNet OpReqType kWriteTo), beta = 1 accumulates
 * (kAddTo), as MKLDNNDeconvBwd::ScheduleBwdData / ScheduleBwdWeights honour the
 * request on the MXNet "mkldnn_deconvolution.cc" page; alpha / beta are the
 * output scaling of the cuDNN ConvolutionBackwardData / ConvolutionBackwardFilter
 * calls on the FilterDescriptor.SetFilter4dDescriptor examples page.
 * Backward-filter applies the epilogue in the last stage (the split-K reduce,
 * or the kernel itself with one split), so partial sums stay fp32.
 * alpha == 1, beta == 0 and fp32 output run the plain entry point's kernels.
 * Other arguments, layouts, validation and errors as the plain entry point.
 */
int conv2d_bwd_data_ex(int N, int C, int H, int W, int K, int R, int S,
                       int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
                       int dtype, const void *dy, const void *w, float alpha, float beta,
                       int out_dtype, void *dx, void *workspace, size_t workspace_bytes, void *stream);

int conv2d_bwd_filter_ex(int N, int C, int H, int W, int K, int R, int S,
                         int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
                         int dtype, const void *x, const void *dy, float alpha, float beta,
                         int out_dtype, void *dw, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Deconvolution forward with the epilogue above, including the optional fp32
 * bias [C_out] (NULL for none; 4-byte aligned, must not overlap y) of the
 * MXNet deconvolution (MKLDNNDeconvFwd::Execute, bias argument) and
 * act = max(0, .) when relu != 0.
 */
int deconv2d_fwd_ex(int N, int C_in, int H_in, int W_in, int C_out, int R, int S,
                    int pad_h, int pad_w, int stride_h, int stride_w, int H_out, int W_out,
                    int dtype, const void *x, const void *w, const float *bias, float alpha, float beta,
                    int relu, int out_dtype, void *y, void *workspace, size_t workspace_bytes, void *stream);

/* Deconvolution backward-data / backward-weights with the epilogue above (no bias). */
int deconv2d_bwd_data_ex(int N, int C_in, int H_in, int W_in, int C_out, int R, int S,
                         int pad_h, int pad_w, int stride_h, int stride_w, int H_out, int W_out,
                         int dtype, const void *dy, const void *w, float alpha, float beta,
                         int out_dtype, void *dx, void *workspace, size_t workspace_bytes, void *stream);

int deconv2d_bwd_filter_ex(int N, int C_in, int H_in, int W_in, int C_out, int R, int S,
                           int pad_h, int pad_w, int stride_h, int stride_w, int H_out, int W_out,
                           int dtype, const void *x, const void *dy, float alpha, float beta,
                           int out_dtype, void *dw, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bias gradient: db[k] = alpha * sum_{n,p,q} dy[n,k,p,q] + beta * db_prev[k]
 * (db_prev read only when beta != 0).  dy [N][K][P][Q] (dtype), db [K] fp32.
 * For a convolution with a bias on its K outputs, dy is the output gradient;
 * for a deconvolution with a bias, call it with (N, C_out, H_out, W_out) and
 * the deconvolution's output gradient (MXNet MKLDNNDeconvBwd::ScheduleBwdWeights,
 * diff_bias).  Summed in fp64 in a fixed order, rounded to fp32 once: bitwise
 * repeatable.  Errors: MICONV_ERR_NULL, MICONV_ERR_BAD_DIM (a size <= 0),
 * MICONV_ERR_DTYPE, MICONV_ERR_TOO_LARGE, MICONV_ERR_ALIGN (dy not 16-byte or
 * db not 4-byte aligned), MICONV_ERR_ALIAS (db overlaps dy), MICONV_ERR_HIP.
 */
int conv2d_bwd_bias(int N, int K, int P, int Q, int dtype, const void *dy, float alpha, float beta,
                    float *db, void *stream);

/* Capacity of the static scratch array of conv2d_bwd_filter_noalloc (128 MiB per device). */
#define MICONV_NOALLOC_SCRATCH_BYTES (128ull << 20)

/*
 * Backward-filter for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same operation, arguments, layouts, validation and errors as
 * conv2d_bwd_filter, with no workspace argument: the split-K partial sums live
 * in a static device array of MICONV_NOALLOC_SCRATCH_BYTES that the library
 * holds on each device it runs on until the process ends.  The plan is made
 * under that capacity, so the result is bitwise that of conv2d_bwd_filter with
 * workspace_bytes = MICONV_NOALLOC_SCRATCH_BYTES; a plan that would need more
 * (none does: the split count adapts) returns MICONV_ERR_WORKSPACE.  The call
 * makes no hipMalloc / hipFree and no allocating library call.  All calls on
 * one device share that device's array: calls that overlap in time on one
 * device (on different streams or host threads) race and must be serialised
 * by the caller.  Nothing in the array needs to start at zero.
 */
int conv2d_bwd_filter_noalloc(int N, int C, int H, int W, int K, int R, int S,
                              int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
                              int dtype, const void *x, const void *dy, float *dw, void *stream);

/*
 * Plan search (autotuning) and the plan cache.  For the (pass, dtype, sizes)
 * of miconv_workspace_size's reading, the library enumerates up to 16
 * distinct candidate plans that fit min(workspace_limit, 1e9) bytes: its
 * default choice first, then the other kernel families that apply, other tile
 * heights, shorter patch tiles, other backward-filter split counts and MFMA
 * forms.  Every candidate computes the same operation (the GPU tests compare
 * each one with the reference).  This is the algorithm search of the cuDNN
 * FindConvolution*Algorithm calls on the FilterDescriptor.SetFilter4dDescriptor
 * examples page (ConvolutionalLayer), the choice under a workspace limit of
 * the SystemDS page's algorithm factories, and the keyed primitive cache of
 * MXNet's MKLDNNDeconvFwd::GetCached / MKLDNNDeconvBwd::GetCached.
 */
typedef struct miconv_perf {
    int index;              /* candidate index (miconv_plan_select's numbering) */
    int status;             /* MICONV_OK, or what launching this candidate returned */
    float time_ms;          /* best of 3 rounds of the mean of 3 back-to-back calls; < 0 if failed */
    size_t workspace_bytes; /* workspace the candidate uses */
    char plan[256];         /* miconv_plan_describe's text for the candidate */
} miconv_perf_t;

/*
 * Number of candidate plans (>= 1) in *count and, when max_workspace_bytes is
 * not NULL, the largest workspace any of them uses.  Pure host computation.
 */
int miconv_plan_candidates(int pass, int dtype, int N, int C, int H, int W, int K, int R, int S,
                           int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
                           size_t workspace_limit, int *count, size_t *max_workspace_bytes);

/*
 * Installs candidate `index` (0 .. count-1) of the enumeration under
 * workspace_limit as the plan for these sizes (index < 0 removes the installed
 * plan, restoring the default choice).  MICONV_ERR_INDEX if index >= count.
 * Pure host computation; affects later calls of this process on every device.
 */
int miconv_plan_select(int pass, int dtype, int N, int C, int H, int W, int K, int R, int S,
                       int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
                       size_t workspace_limit, int index);

/*
 * Times every candidate that fits min(workspace_bytes, 1e9) on the caller's
 * buffers (in0, in1, out in the reading of the pass's compute entry point:
 * forward x, w, y; backward-data dy, w, dx; backward-filter x, dy, dw;
 * deconvolution passes as deconv2d_fwd / deconv2d_bwd_data /
 * deconv2d_bwd_filter), on `stream`, and installs the fastest as the plan for
 * these sizes.  Writes min(requested, count) results, fastest first, to perf
 * and their number to *returned.  Blocks until the timing runs finish.  The
 * content of out afterwards is the result of one of the candidates; the
 * inputs are not modified.  Validation and errors as the compute entry
 * points, checked for every candidate before anything is launched.
 */
int miconv_find_plan(int pass, int dtype, int N, int C, int H, int W, int K, int R, int S,
                     int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
                     const void *in0, const void *in1, void *out, void *workspace, size_t workspace_bytes,
                     void *stream, int requested, int *returned, miconv_perf_t *perf);

/* Empties the plan cache (installed plans included). */
int miconv_plan_cache_clear(void);

/* Installed (tuned) plans and all cached plans, in *tuned and *total. */
int miconv_plan_cache_entries(int *tuned, int *total);

/*
 * Generalised convolution: 1, 2 or 3 spatial dimensions, groups, dilation and
 * separate low / high zero padding per dimension (MXNet
 * "mkldnn_deconvolution.cc": SupportMKLDNNDeconv admits 1 to 3 spatial
 * dimensions, num_group groups, DeconvDescCreator's dilates; the C# page's
 * padding modes, Tensor.GetPaddingParams / PaddingType).  Tensors, packed,
 * with the spatial sizes of the descriptor (outermost first):
 *   x [N][C][in...],  w [K][C/groups][filter...],  y / dy [N][K][out...]
 * Output channel k is in group g = k / (K/groups) and reads input channels
 * g*(C/groups) .. g*(C/groups) + C/groups - 1:
 *   y[n,k,o] = sum_{c < C/groups, taps f} w[k,c,f] * x~(n, g*C/groups + c, o*stride - pad_lo + f*dilation)
 * per spatial dimension; backward-data and backward-filter are its adjoints
 * in x and w.  out must equal floor((in + pad_lo + pad_hi - dilation*(filter-1) - 1)/stride) + 1
 * (else MICONV_ERR_OUT_SIZE); C and K must divide by groups (else
 * MICONV_ERR_BAD_DIM).  A deconvolution is convnd_bwd_data with the
 * convolution view of its sizes (the 2-D role swap above).  Problems that are
 * plain 2-D (or 1-D) convolutions -- one group, dilation 1, equal low and high
 * padding -- run the specialised 2-D kernels and plans (the plan cache
 * included); the rest run one generic MFMA implicit-GEMM kernel per pass.
 * dtype, alignment, aliasing, workspace, stream, errors and determinism as
 * for the 2-D entry points; outputs fp32, overwritten.
 */
typedef struct miconv_nd_desc {
    int ndim;                 /* 1, 2 or 3 */
    int N, C, K, groups;
    int in[3];                /* input sizes, outermost first (W; H, W; or D, H, W) */
    int filter[3];            /* filter sizes, same order */
    int out[3];               /* output sizes, same order */
    int pad_lo[3], pad_hi[3]; /* zero padding before / after each dimension */
    int stride[3], dilation[3];
} miconv_nd_desc_t;

#define MICONV_PAD_VALID 0
#define MICONV_PAD_SAME 1

/*
 * Fills d->pad_lo, d->pad_hi and d->out from d->in, d->filter, d->stride and
 * d->dilation for a padding mode: MICONV_PAD_VALID pads nothing;
 * MICONV_PAD_SAME gives out = ceil(in / stride) with total padding
 * max((out - 1)*stride + dilation*(filter - 1) + 1 - in, 0), the smaller half
 * low (the page names the modes without defining them; this is the common
 * reading).  MICONV_ERR_BAD_DIM for an unknown mode, ndim or non-positive size.
 */
int miconv_nd_padding(miconv_nd_desc_t *d, int mode);

int convnd_fwd(const miconv_nd_desc_t *d, int dtype, const void *x, const void *w, float *y,
               void *workspace, size_t workspace_bytes, void *stream);
int convnd_bwd_data(const miconv_nd_desc_t *d, int dtype, const void *dy, const void *w, float *dx,
                    void *workspace, size_t workspace_bytes, void *stream);
int convnd_bwd_filter(const miconv_nd_desc_t *d, int dtype, const void *x, const void *dy, float *dw,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Workspace the plan for (pass, d, dtype) uses under workspace_limit (pass: MICONV_FWD,
 * MICONV_BWD_DATA or MICONV_BWD_FILTER).  Pure host computation. */
int convnd_workspace_size(int pass, const miconv_nd_desc_t *d, int dtype, size_t workspace_limit,
                          size_t *bytes_out);

/* One-line description of the plan (2-D kernels' format, or algo=generic). */
int convnd_describe(int pass, const miconv_nd_desc_t *d, int dtype, size_t workspace_bytes, char *buf,
                    size_t buflen);

/* Static text for a status code (never NULL). */
const char *miconv_status_string(int status);

/*
 * Writes a one-line description of the plan a call with these arguments
 * would run (kernel tile, split count, workspace use) into buf (always
 * NUL-terminated when buflen > 0).  Same argument reading as
 * miconv_workspace_size.  Pure host computation.
 */
int miconv_plan_describe(int pass, int dtype, int N, int C, int H, int W, int K, int R, int S,
                         int pad_h, int pad_w, int stride_h, int stride_w, int P, int Q,
                         size_t workspace_bytes, char *buf, size_t buflen);

/* Library ABI version (increments on any signature change). */
int miconv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MICONV_H */
