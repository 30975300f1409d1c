// bwd_bias.hip -- gradient of a per-channel bias: db[k] = alpha * sum over n, p, q
// of dy[n, k, p, q] + beta * db[k] (db read only when beta != 0), fp32 output.
//
// For a convolution with a bias on its K output channels, dy is the output
// gradient [N][K][P][Q]; for a deconvolution with a bias on its C_out output
// channels, it is the deconvolution's output gradient [N][C_out][H_out][W_out].
//
// One work-group of 1024 threads per channel k.  The channel's N*P*Q values
// (N contiguous runs of P*Q) are read with consecutive lanes on consecutive
// elements, four elements per load when P*Q is a multiple of 4 (16-byte fp32 or
// 8-byte bf16 loads); every thread sums its elements in fp64 in increasing
// order, then the 1024 partial sums are added in a fixed tree order.  The
// result depends on neither timing nor the launch, so calls are bitwise
// repeatable, and the fp64 accumulation leaves only the final rounding to fp32.
#include "device.h"
#include "launch.h"

namespace miconv {

namespace {
constexpr int kThreads = 1024;
}

template <int ES, bool V4>
__global__ __launch_bounds__(kThreads) void bias_grad_kernel(const void *__restrict__ dy, float *__restrict__ db,
                                                             int N, int K, int PQ, float alpha, float beta) {
    __shared__ double red[kThreads];
    const int k = blockIdx.x, tid = threadIdx.x;
    double s = 0.0;
    if constexpr (V4) {
        const int pq4 = PQ / 4, total = N * pq4;
        for (int e = tid; e < total; e += kThreads) {
            const int n = e / pq4, u = e - n * pq4;
            const size_t off = ((size_t)n * K + k) * PQ + 4 * u;
            if constexpr (ES == 4) {
                const float4 v = *(const float4 *)((const float *)dy + off);
                s += (double)v.x + (double)v.y + (double)v.z + (double)v.w;
            } else {
                const u32x2 h = *(const u32x2 *)((const uint16_t *)dy + off);
                s += (double)bf16_to_f32(h[0] & 0xffffu) + (double)bf16_to_f32(h[0] >> 16) +
                     (double)bf16_to_f32(h[1] & 0xffffu) + (double)bf16_to_f32(h[1] >> 16);
            }
        }
    } else {
        const int total = N * PQ;
        for (int e = tid; e < total; e += kThreads) {
            const int n = e / PQ, u = e - n * PQ;
            const size_t off = ((size_t)n * K + k) * PQ + u;
            if constexpr (ES == 4)
                s += (double)((const float *)dy)[off];
            else
                s += (double)bf16_to_f32(((const uint16_t *)dy)[off]);
        }
    }
    red[tid] = s;
    __syncthreads();
    for (int h = kThreads / 2; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    if (tid == 0) {
        float v = alpha * (float)red[0];
        if (beta != 0.0f) v += beta * db[k];
        db[k] = v;
    }
}

int launch_bias_grad(int dtype, int N, int K, int PQ, const void *dy, float alpha, float beta, float *db,
                     hipStream_t st) {
    const bool v4 = PQ % 4 == 0;
    const void *kern = dtype ? (v4 ? (const void *)bias_grad_kernel<2, true> : (const void *)bias_grad_kernel<2, false>)
                             : (v4 ? (const void *)bias_grad_kernel<4, true> : (const void *)bias_grad_kernel<4, false>);
    void *args[] = {(void *)&dy, (void *)&db, (void *)&N, (void *)&K, (void *)&PQ, (void *)&alpha, (void *)&beta};
    const hipError_t e = hipLaunchKernel(kern, dim3((unsigned)K), dim3(kThreads), args, 0, st);
    return e == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
}

}  // namespace miconv
