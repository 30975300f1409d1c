// convnd.hip -- the generalised convolution on MFMA: 1 to 3 spatial dimensions,
// groups, dilation, separate low / high zero padding, every stride; forward,
// backward-data and backward-filter, fp32 or bf16 inputs, fp32 accumulation
// and output.
//
// One implicit GEMM per group (the GEMM shapes are listed in nd.h).  A
// work-group owns a 64 x 64 output tile of one group (and, for
// backward-filter, one split of the reduction); four waves of 32 x 32
// (v_mfma_f32_32x32x16_bf16, or v_mfma_f32_32x32x2_f32 for fp32 inputs).
// Each reduction step stages 64 bytes of reduction per tile row of both
// operands in LDS ([row][64 B], 80-byte pitch); a thread gathers one 16-byte
// piece (8 bf16 or 4 fp32 consecutive reduction indices of one row or column),
// decoding the first index with multiply-high divisions and stepping to the
// next with carries.  Out-of-volume taps, taps whose backward-data output row
// does not divide by the stride, and indices past the end read 0 through
// the buffer loads' range check.  The next step's pieces are loaded into
// registers while the current step's MFMAs run.  Backward-filter writes fp32
// partial sums per split, summed in split order by nd_reduce.
#include "device.h"
#include "launch.h"
#include "nd.h"

namespace miconv {

struct NdArgs {
    const void *a0, *a1;   // forward: x, w;  backward-data: dy, w;  backward-filter: x, dy
    float *out;            // y, dx, dW, or the split-K partial sums
    uint32_t a0_bytes, a1_bytes;
    int N, C, K, G, Cg, Kg;
    int D, H, W, T, R, S, OD, OH, OW;
    int pd, ph, pw, sd, sh, sw, dd, dh, dw;
    int rows, cols, red;   // per-group GEMM
    int m_tiles, n_tiles, splits, chunk;
    FDiv fd_S, fd_RS, fd_TRS, fd_OW, fd_OH, fd_ODHW, fd_W, fd_H, fd_DHW, fd_sd, fd_sh, fd_sw;
};

namespace {
constexpr int kBM = 64, kBN = 64, kBKB = 64, kPitch = kBKB + 16;
}

// Reduction index kr -> (channel-like index, t, r, s) with channel = kr / (T*R*S).
struct Tap {
    int c, t, r, s;
};
DEVI Tap decode_tap(const NdArgs &a, int kr) {
    Tap q;
    const int RS = a.R * a.S;
    q.c = (int)fdiv((uint32_t)kr, a.fd_TRS);
    int rem = kr - q.c * a.T * RS;
    q.t = (int)fdiv((uint32_t)rem, a.fd_RS);
    rem -= q.t * RS;
    q.r = (int)fdiv((uint32_t)rem, a.fd_S);
    q.s = rem - q.r * a.S;
    return q;
}
DEVI void next_tap(const NdArgs &a, Tap &q) {
    if (++q.s == a.S) {
        q.s = 0;
        if (++q.r == a.R) {
            q.r = 0;
            if (++q.t == a.T) {
                q.t = 0;
                ++q.c;
            }
        }
    }
}

// Output-space position (n, od, oh, ow) of a flat index over N x OD x OH x OW.
struct Pos {
    int n, d, h, w;
};
DEVI Pos decode_pos(int e, FDiv fd_vol, FDiv fd_hw_w, FDiv fd_h, int vol, int Hs, int Ws) {
    Pos p;
    p.n = (int)fdiv((uint32_t)e, fd_vol);
    int rem = e - p.n * vol;
    const int hw = (int)fdiv((uint32_t)rem, fd_hw_w);   // rem / W -> (d*H + h)
    p.w = rem - hw * Ws;
    p.d = (int)fdiv((uint32_t)hw, fd_h);
    p.h = hw - p.d * Hs;
    return p;
}
DEVI void next_pos(Pos &p, int Ds, int Hs, int Ws) {
    if (++p.w == Ws) {
        p.w = 0;
        if (++p.h == Hs) {
            p.h = 0;
            if (++p.d == Ds) {
                p.d = 0;
                ++p.n;
            }
        }
    }
}

template <int ES>
DEVI uint32_t elem_off(uint32_t e) {
    return e * ES;   // element index -> byte offset (tensors are below 2 GiB)
}

// One 16-byte piece (VEC consecutive reduction indices kr0 ..) of row `row` of
// the A operand and of column `col` of the B operand, for group g.
template <int PASS, int ES>
struct NdGather {
    static constexpr int VEC = 16 / ES;

    static DEVI u32x4 load_a(const NdArgs &a, rsrc_t ra, int g, int row, int kr0, int kend) {
        uint32_t e[VEC];
        const bool rok = row < a.rows;
        if constexpr (PASS == FWD) {
            // w [K][Cg*T*R*S]: the row's reduction is contiguous
            const uint32_t base = (uint32_t)((g * a.Kg + row) * a.red);
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                e[j] = ld_elem<ES>(ra, rok && kr0 + j < kend ? elem_off<ES>(base + kr0 + j) : kOOB);
        } else if constexpr (PASS == BWD_DATA) {
            // w [K][Cg][T*R*S] at (k = g*Kg + kr / TRS, c = row, trs = kr % TRS)
            const int TRS = a.T * a.R * a.S;
            int k = (int)fdiv((uint32_t)kr0, a.fd_TRS), trs = kr0 - k * TRS;
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const bool ok = rok && kr0 + j < kend;
                e[j] = ld_elem<ES>(ra, ok ? elem_off<ES>((uint32_t)(((g * a.Kg + k) * a.Cg + row) * TRS + trs)) : kOOB);
                if (++trs == TRS) {
                    trs = 0;
                    ++k;
                }
            }
        } else {
            // dy [N][K][OD*OH*OW] at (n, g*Kg + row, o) with kr = n*ODHW + o
            const int vol = a.OD * a.OH * a.OW;
            int n = (int)fdiv((uint32_t)kr0, a.fd_ODHW), o = kr0 - n * vol;
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const bool ok = rok && kr0 + j < kend;
                e[j] = ld_elem<ES>(ra, ok ? elem_off<ES>((uint32_t)((n * a.K + g * a.Kg + row) * vol + o)) : kOOB);
                if (++o == vol) {
                    o = 0;
                    ++n;
                }
            }
        }
        return pack<ES>(e);
    }

    static DEVI u32x4 load_b(const NdArgs &a, rsrc_t rb, int g, int col, int kr0, int kend) {
        uint32_t e[VEC];
        const bool cok = col < a.cols;
        if constexpr (PASS == FWD) {
            // x~ at (n, g*Cg + c, od*sd - pd + t*dd, ...) for col = (n, od, oh, ow), kr = (c, t, r, s)
            const Pos p = decode_pos(cok ? col : 0, a.fd_ODHW, a.fd_OW, a.fd_OH, a.OD * a.OH * a.OW, a.OH, a.OW);
            const int i0 = p.d * a.sd - a.pd, j0 = p.h * a.sh - a.ph, l0 = p.w * a.sw - a.pw;
            Tap q = decode_tap(a, kr0);
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int i = i0 + q.t * a.dd, jj = j0 + q.r * a.dh, l = l0 + q.s * a.dw;
                const bool ok = cok && kr0 + j < kend && (unsigned)i < (unsigned)a.D && (unsigned)jj < (unsigned)a.H &&
                                (unsigned)l < (unsigned)a.W;
                e[j] = ld_elem<ES>(
                    rb, ok ? elem_off<ES>((uint32_t)((((p.n * a.C + g * a.Cg + q.c) * a.D + i) * a.H + jj) * a.W + l))
                           : kOOB);
                next_tap(a, q);
            }
        } else if constexpr (PASS == BWD_DATA) {
            // dy at (n, g*Kg + k, (i + pd - t*dd)/sd, ...) for col = (n, i, j, l), kr = (k, t, r, s),
            // only where every division is exact and in range
            const Pos p = decode_pos(cok ? col : 0, a.fd_DHW, a.fd_W, a.fd_H, a.D * a.H * a.W, a.H, a.W);
            const int i0 = p.d + a.pd, j0 = p.h + a.ph, l0 = p.w + a.pw;
            Tap q = decode_tap(a, kr0);
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int ni = i0 - q.t * a.dd, nj = j0 - q.r * a.dh, nl = l0 - q.s * a.dw;
                const int od = (int)fdiv((uint32_t)max(ni, 0), a.fd_sd), oh = (int)fdiv((uint32_t)max(nj, 0), a.fd_sh),
                          ow = (int)fdiv((uint32_t)max(nl, 0), a.fd_sw);
                const bool ok = cok && kr0 + j < kend && ni >= 0 && nj >= 0 && nl >= 0 && od * a.sd == ni &&
                                oh * a.sh == nj && ow * a.sw == nl && od < a.OD && oh < a.OH && ow < a.OW;
                e[j] = ld_elem<ES>(
                    rb, ok ? elem_off<ES>((uint32_t)((((p.n * a.K + g * a.Kg + q.c) * a.OD + od) * a.OH + oh) * a.OW + ow))
                           : kOOB);
                next_tap(a, q);
            }
        } else {
            // x~ at (n, g*Cg + c, od*sd - pd + t*dd, ...) for col = (c, t, r, s), kr = (n, od, oh, ow)
            const Tap q = decode_tap(a, cok ? col : 0);
            Pos p = decode_pos(kr0, a.fd_ODHW, a.fd_OW, a.fd_OH, a.OD * a.OH * a.OW, a.OH, a.OW);
            const int ti = q.t * a.dd - a.pd, tj = q.r * a.dh - a.ph, tl = q.s * a.dw - a.pw;
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int i = p.d * a.sd + ti, jj = p.h * a.sh + tj, l = p.w * a.sw + tl;
                const bool ok = cok && kr0 + j < kend && (unsigned)i < (unsigned)a.D && (unsigned)jj < (unsigned)a.H &&
                                (unsigned)l < (unsigned)a.W;
                e[j] = ld_elem<ES>(
                    rb, ok ? elem_off<ES>((uint32_t)((((p.n * a.C + g * a.Cg + q.c) * a.D + i) * a.H + jj) * a.W + l))
                           : kOOB);
                next_pos(p, a.OD, a.OH, a.OW);
            }
        }
        return pack<ES>(e);
    }
};

template <int DT, int PASS>
__global__ __launch_bounds__(256) void convnd_kernel(NdArgs a) {
    constexpr int ES = DT ? 2 : 4, BK = kBKB / ES, VEC = 16 / ES;
    constexpr int STAGE = (kBM + kBN) * kPitch;
    __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];
    using Gth = NdGather<PASS, ES>;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tiles = a.m_tiles * a.n_tiles;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int zg = logical / tiles, tt = logical - zg * tiles;
    const int z = zg / a.G, g = zg - z * a.G;
    const int m0 = (tt % a.m_tiles) * kBM, n0 = (tt / a.m_tiles) * kBN;
    const int kbeg = z * a.chunk, kend = min(a.red, kbeg + a.chunk);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    const rsrc_t r0 = make_rsrc(a.a0, a.a0_bytes), r1 = make_rsrc(a.a1, a.a1_bytes);
    // operand A is the filter (forward, backward-data: a1) or dy (backward-filter: a1);
    // operand B is gathered from x (forward, backward-filter: a0) or dy (backward-data: a0)
    const int row = m0 + (tid & 63), col = n0 + (tid & 63), q = tid >> 6;

    f32x16 acc[1][1];
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[0][0][v] = 0.0f;

    u32x4 ra, rb;
    auto load = [&](int step) __attribute__((always_inline)) {
        const int kr0 = kbeg + step * BK + q * VEC;
        ra = Gth::load_a(a, r1, g, row, kr0, kend);
        rb = Gth::load_b(a, r0, g, col, kr0, kend);
    };
    auto store = [&](char *st) __attribute__((always_inline)) {
        *(u32x4 *)(st + (tid & 63) * kPitch + q * 16) = ra;
        *(u32x4 *)(st + kBM * kPitch + (tid & 63) * kPitch + q * 16) = rb;
    };
    if (nk > 0) {
        load(0);
        store(lds);
    }
    __syncthreads();
    const int wm = wave & 1, wn = wave >> 1;
    for (int kt = 0; kt < nk; ++kt) {
        char *cur = lds + (kt & 1) * STAGE;
        const bool more = kt + 1 < nk;
        if (more) load(kt + 1);
        mma_stage<DT, 1, 1, kBKB / 32, kPitch>(cur + wm * 32 * kPitch, cur + kBM * kPitch + wn * 32 * kPitch, acc,
                                               lane);
        if (more) store(lds + ((kt + 1) & 1) * STAGE);
        __syncthreads();
    }

    // epilogue: lane holds column n0 + wn*32 + (lane & 31) and rows m0 + wm*32 + acc_row(v, lane >> 5)
    const int lr = lane & 31, lh = lane >> 5;
    const int oc = n0 + wn * 32 + lr;
    if (oc >= a.cols) return;
    size_t base;
    int rstride;   // output elements between consecutive rows
    if constexpr (PASS == FWD) {
        const int vol = a.OD * a.OH * a.OW;
        const int n = (int)fdiv((uint32_t)oc, a.fd_ODHW), o = oc - n * vol;
        base = ((size_t)n * a.K + (size_t)g * a.Kg) * vol + o;
        rstride = vol;
    } else if constexpr (PASS == BWD_DATA) {
        const int vol = a.D * a.H * a.W;
        const int n = (int)fdiv((uint32_t)oc, a.fd_DHW), o = oc - n * vol;
        base = ((size_t)n * a.C + (size_t)g * a.Cg) * vol + o;
        rstride = vol;
    } else if (a.splits == 1) {   // dW [K][Cg*T*R*S]
        base = (size_t)g * a.Kg * a.cols + oc;
        rstride = a.cols;
    } else {                      // partial sums [split][K][Cg*T*R*S]
        base = ((size_t)z * a.K + (size_t)g * a.Kg) * a.cols + oc;
        rstride = a.cols;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 32 + acc_row(v, lh);
        if (m < a.rows) a.out[base + (size_t)m * rstride] = acc[0][0][v];
    }
}

// dW[e] = sum over splits z = 0, 1, ..., splits-1 of part[z][e], in that order.
__global__ __launch_bounds__(256) void nd_reduce(const float *__restrict__ part, float *__restrict__ dw,
                                                 long long total, int splits) {
    for (long long e = blockIdx.x * 256LL + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
        float s = part[e];
        for (int z = 1; z < splits; ++z) s += part[(long long)z * total + e];
        dw[e] = s;
    }
}

template <int DT>
static hipError_t nd_go(int pass, const NdArgs &a, int grid, hipStream_t st) {
    if (pass == FWD) hipLaunchKernelGGL((convnd_kernel<DT, FWD>), dim3(grid), dim3(256), 0, st, a);
    else if (pass == BWD_DATA) hipLaunchKernelGGL((convnd_kernel<DT, BWD_DATA>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((convnd_kernel<DT, BWD_FILTER>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

int launch_nd(const NdProblem &p, const NdPlan &pl, const void *in0, const void *in1, float *out, void *ws,
              hipStream_t st) {
    NdArgs a = {};
    const size_t es = p.dtype ? 2 : 4;
    const size_t vin = (size_t)p.in[0] * p.in[1] * p.in[2], vout = (size_t)p.out[0] * p.out[1] * p.out[2];
    const size_t taps = (size_t)p.f[0] * p.f[1] * p.f[2];
    const size_t nx = (size_t)p.N * p.C * vin, ny = (size_t)p.N * p.K * vout, nw = (size_t)p.K * (p.C / p.G) * taps;
    a.N = p.N; a.C = p.C; a.K = p.K; a.G = p.G; a.Cg = p.C / p.G; a.Kg = p.K / p.G;
    a.D = p.in[0]; a.H = p.in[1]; a.W = p.in[2];
    a.T = p.f[0]; a.R = p.f[1]; a.S = p.f[2];
    a.OD = p.out[0]; a.OH = p.out[1]; a.OW = p.out[2];
    a.pd = p.lo[0]; a.ph = p.lo[1]; a.pw = p.lo[2];
    a.sd = p.st[0]; a.sh = p.st[1]; a.sw = p.st[2];
    a.dd = p.dil[0]; a.dh = p.dil[1]; a.dw = p.dil[2];
    a.rows = (int)pl.rows; a.cols = (int)pl.cols; a.red = (int)pl.red;
    a.m_tiles = pl.m_tiles; a.n_tiles = pl.n_tiles; a.splits = pl.splits; a.chunk = (int)pl.chunk;
    a.fd_S = make_fdiv((uint32_t)a.S);
    a.fd_RS = make_fdiv((uint32_t)(a.R * a.S));
    a.fd_sd = make_fdiv((uint32_t)a.sd);
    a.fd_sh = make_fdiv((uint32_t)a.sh);
    a.fd_sw = make_fdiv((uint32_t)a.sw);
    a.fd_TRS = make_fdiv((uint32_t)taps);
    a.fd_OW = make_fdiv((uint32_t)a.OW);
    a.fd_OH = make_fdiv((uint32_t)a.OH);
    a.fd_ODHW = make_fdiv((uint32_t)vout);
    a.fd_W = make_fdiv((uint32_t)a.W);
    a.fd_H = make_fdiv((uint32_t)a.H);
    a.fd_DHW = make_fdiv((uint32_t)vin);
    a.a0 = in0;
    a.a1 = in1;
    if (p.pass == FWD) {
        a.a0_bytes = (uint32_t)(nx * es); a.a1_bytes = (uint32_t)(nw * es);
    } else if (p.pass == BWD_DATA) {
        a.a0_bytes = (uint32_t)(ny * es); a.a1_bytes = (uint32_t)(nw * es);
    } else {
        a.a0_bytes = (uint32_t)(nx * es); a.a1_bytes = (uint32_t)(ny * es);
    }
    float *part = pl.splits > 1 ? (float *)ws : out;
    a.out = part;
    const long long grid = (long long)pl.m_tiles * pl.n_tiles * p.G * pl.splits;
    if (grid <= 0 || grid > 0x7fffffffLL) return MICONV_ERR_TOO_LARGE;
    hipError_t e = p.dtype ? nd_go<1>(p.pass, a, (int)grid, st) : nd_go<0>(p.pass, a, (int)grid, st);
    if (e != hipSuccess) return MICONV_ERR_HIP;
    if (pl.splits > 1) {
        const long long total = (long long)p.K * pl.cols;
        long long blocks = (total + 255) / 256;
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL(nd_reduce, dim3((unsigned)blocks), dim3(256), 0, st, part, out, total, pl.splits);
        if (hipGetLastError() != hipSuccess) return MICONV_ERR_HIP;
    }
    return MICONV_OK;
}

}  // namespace miconv
