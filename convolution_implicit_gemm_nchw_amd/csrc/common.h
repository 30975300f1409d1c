// common.h -- index helpers shared by host planning code and device kernels.
//
// Division of a non-negative 31-bit integer by a fixed divisor
// with one multiply-high and one shift.
//
// For d >= 2 let l = ceil(log2 d), m = ceil(2^(31+l) / d) and s = l - 1.  Then
// for every 0 <= n < 2^31:  floor(n / d) == floor(n * m / 2^32) >> s.
// (m < 2^32 because d > 2^(l-1); the error n*(m - 2^(31+l)/d) / 2^(31+l) is
// below 2^-l <= 1/d, which cannot carry floor(n/d) over an integer.)
// d == 1 is flagged with m == 0 and returns n.
#pragma once
#include <stdint.h>

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC_RTC__) || defined(MICONV_DEVICE_CODE)
#define MICONV_HD __host__ __device__
#else
#define MICONV_HD
#endif

struct FDiv {
    uint32_t d, m, s;
};

MICONV_HD inline FDiv make_fdiv(uint32_t d) {
    FDiv f;
    f.d = d;
    if (d <= 1) {
        f.m = 0;
        f.s = 0;
        return f;
    }
    uint32_t l = 0;
    while ((1ull << l) < (uint64_t)d) ++l;
    uint64_t num = 1ull << (31 + l);
    f.m = (uint32_t)((num + d - 1) / d);
    f.s = l - 1;
    return f;
}

MICONV_HD inline uint32_t fdiv_host(uint32_t n, const FDiv &f) {
    return f.m == 0 ? n : (uint32_t)(((uint64_t)n * f.m) >> 32) >> f.s;
}

// Fused forward epilogue: y = act(alpha * acc + beta * y_prev + bias[k]),
// act = max(0, .) when relu; y_prev is read only when beta != 0.
struct Epi {
    const float *bias;    // [K] or null
    float alpha, beta;
    int relu;
    int out_bf16;         // y is bf16 (round to nearest even) instead of fp32
};

// Stride-phase geometry of backward-data along one spatial dimension.
// For phase f (0 <= f < stride): the input rows i = i0 + stride*a (0 <= a < na)
// are exactly those with (i + pad) mod stride == f; they receive the taps
// r = f + stride*u (0 <= u < nu) and nothing else, each from output row
// p = base + a - u (used only when 0 <= p < P).  No zero-inserted tap is
// ever visited.
struct PhaseDim {
    int i0, na, nu, base;
};

MICONV_HD inline PhaseDim phase_dim(int f, int stride, int pad, int in, int filt) {
    PhaseDim d;
    d.i0 = ((f - pad) % stride + stride) % stride;
    d.na = d.i0 < in ? (in - d.i0 + stride - 1) / stride : 0;
    d.nu = f < filt ? (filt - f + stride - 1) / stride : 0;
    d.base = (d.i0 + pad - f) / stride;
    return d;
}
