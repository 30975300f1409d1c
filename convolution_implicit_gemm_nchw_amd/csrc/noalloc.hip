// noalloc.hip -- backward-filter whose scratch memory is a static device array,
// for callers that cannot allocate device memory.
//
// conv2d_bwd_filter keeps its split-K partial sums in a caller-provided
// workspace.  conv2d_bwd_filter_noalloc runs the same plan with that workspace
// replaced by `scratch`, a file-scope __device__ array of
// MICONV_NOALLOC_SCRATCH_BYTES: the plan is made under that capacity, exactly
// as conv2d_bwd_filter plans with workspace_bytes = MICONV_NOALLOC_SCRATCH_BYTES,
// so the two calls give bitwise the same dW.
//
// The array's name is a host-side stand-in in host code, not a device address.
// Its address on a device comes from hipGetSymbolAddress, queried once per
// device (with that device current) on the first call there and kept; only
// that address is ever passed to kernels.  Each device holds its own copy of
// the array until the process ends.
//
// Every call on one device shares that device's array.  Stage 1 writes every
// element of the partial sums that stage 2 reads, so nothing needs clearing
// between calls; calls that overlap in time on one device (different streams,
// or different host threads) race on the array and must be serialised by the
// caller.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/miconv.h"
#include "launch.h"
#include "plan.h"

namespace miconv {
namespace {

constexpr size_t kScratchBytes = (size_t)MICONV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device, once queried

// Address of this device's `scratch`, or null with *err set.
void *scratch_on_current_device(int *err) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = MICONV_ERR_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            *err = MICONV_ERR_HIP;
            return nullptr;
        }
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

}  // namespace
}  // namespace miconv

using namespace miconv;

extern "C" int conv2d_bwd_filter_noalloc(int N, int C, int H, int W, int K, int R, int S, int pad_h, int pad_w,
                                         int stride_h, int stride_w, int P, int Q, int dtype, const void *x,
                                         const void *dy, float *dw, void *stream) {
    Problem p;
    p.pass = BWD_FILTER;
    p.dtype = dtype;
    p.N = N; p.C = C; p.H = H; p.W = W; p.K = K; p.R = R; p.S = S;
    p.ph = pad_h; p.pw = pad_w; p.sh = stride_h; p.sw = stride_w; p.P = P; p.Q = Q;
    int st = validate_problem(p);
    if (st != MICONV_OK) return st;
    // the plan never needs more than its budget; checked anyway before anything is enqueued
    Plan pl;
    make_plan(p, kScratchBytes, &pl);
    if (pl.ws_used > kScratchBytes) return MICONV_ERR_WORKSPACE;
    int err = MICONV_OK;
    void *ptr = scratch_on_current_device(&err);
    if (!ptr) return err;
    return run_problem(p, x, dy, dw, ptr, kScratchBytes, stream);
}
