// ndplan.cpp -- validation and plan of the generalised convolution.  Pure host
// code; compiled into the library and, on its own, into a CPU test.
#include "nd.h"

#include <stdio.h>

#include "../../include/miconv.h"

namespace miconv {

static const long long kMaxBytes = (1LL << 31) - 1;
static const size_t kNdWsCap = (size_t)MICONV_MAX_WORKSPACE_BYTES;

static long long cdiv_ll(long long a, long long b) { return (a + b - 1) / b; }

int nd_out_dim(int in, int f, int lo, int hi, int st, int dil) {
    const long long num = (long long)in + lo + hi - (long long)dil * (f - 1) - 1;
    if (num < 0 || st < 1) return 0;
    return (int)(num / st) + 1;
}

int nd_from_desc(int pass, int dtype, int ndim, int N, int C, int K, int G, const int *in, const int *f,
                 const int *out, const int *lo, const int *hi, const int *st, const int *dil, NdProblem *p) {
    if (ndim < 1 || ndim > 3) return MICONV_ERR_BAD_DIM;
    NdProblem q = {};
    q.pass = pass;
    q.dtype = dtype;
    q.N = N; q.C = C; q.K = K; q.G = G;
    for (int d = 0; d < 3; ++d) {
        const int s = d - (3 - ndim);   // index into the caller's arrays, < 0 for a lifted dimension
        q.in[d] = s < 0 ? 1 : in[s];
        q.f[d] = s < 0 ? 1 : f[s];
        q.out[d] = s < 0 ? 1 : out[s];
        q.lo[d] = s < 0 ? 0 : lo[s];
        q.hi[d] = s < 0 ? 0 : hi[s];
        q.st[d] = s < 0 ? 1 : st[s];
        q.dil[d] = s < 0 ? 1 : dil[s];
    }
    *p = q;
    return MICONV_OK;
}

int validate_nd(const NdProblem &p) {
    if (p.dtype != MICONV_F32 && p.dtype != MICONV_BF16) return MICONV_ERR_DTYPE;
    if (p.N <= 0 || p.C <= 0 || p.K <= 0 || p.G <= 0) return MICONV_ERR_BAD_DIM;
    if (p.C % p.G != 0 || p.K % p.G != 0) return MICONV_ERR_BAD_DIM;
    for (int d = 0; d < 3; ++d) {
        if (p.in[d] <= 0 || p.f[d] <= 0 || p.lo[d] < 0 || p.hi[d] < 0 || p.st[d] < 1 || p.dil[d] < 1)
            return MICONV_ERR_BAD_DIM;
        if (p.in[d] > (1 << 20) || p.f[d] > (1 << 20) || p.lo[d] > (1 << 20) || p.hi[d] > (1 << 20) ||
            p.st[d] > (1 << 20) || p.dil[d] > (1 << 20))
            return MICONV_ERR_TOO_LARGE;
        const int o = nd_out_dim(p.in[d], p.f[d], p.lo[d], p.hi[d], p.st[d], p.dil[d]);
        if (o < 1) return MICONV_ERR_BAD_DIM;
        if (p.out[d] != o) return MICONV_ERR_OUT_SIZE;
    }
    const long long vin = (long long)p.in[0] * p.in[1] * p.in[2], vout = (long long)p.out[0] * p.out[1] * p.out[2];
    const long long taps = (long long)p.f[0] * p.f[1] * p.f[2];
    const long long nx = p.N * (long long)p.C * vin, ny = p.N * (long long)p.K * vout;
    const long long nw = (long long)p.K * (p.C / p.G) * taps;
    // every tensor in fp32 below 2 GiB (outputs are fp32; inputs may be) and every GEMM extent
    // and element index inside 31 bits
    if (4 * nx > kMaxBytes || 4 * ny > kMaxBytes || 4 * nw > kMaxBytes) return MICONV_ERR_TOO_LARGE;
    return MICONV_OK;
}

bool nd_as_2d(const NdProblem &p, Problem *q) {
    if (p.G != 1 || p.in[0] != 1 || p.f[0] != 1 || p.out[0] != 1 || p.lo[0] != 0 || p.hi[0] != 0) return false;
    for (int d = 1; d < 3; ++d)
        if (p.dil[d] != 1 || p.lo[d] != p.hi[d]) return false;
    Problem r;
    r.pass = p.pass;
    r.dtype = p.dtype;
    r.N = p.N; r.C = p.C; r.K = p.K;
    r.H = p.in[1]; r.W = p.in[2]; r.R = p.f[1]; r.S = p.f[2];
    r.ph = p.lo[1]; r.pw = p.lo[2]; r.sh = p.st[1]; r.sw = p.st[2];
    r.P = p.out[1]; r.Q = p.out[2];
    *q = r;
    return true;
}

void make_nd_plan(const NdProblem &p, size_t ws_limit, NdPlan *out) {
    NdPlan pl = {};
    const size_t budget = ws_limit < kNdWsCap ? ws_limit : kNdWsCap;
    const long long Cg = p.C / p.G, Kg = p.K / p.G;
    const long long taps = (long long)p.f[0] * p.f[1] * p.f[2];
    const long long vin = (long long)p.in[0] * p.in[1] * p.in[2], vout = (long long)p.out[0] * p.out[1] * p.out[2];
    pl.bm = 64;
    pl.bn = 64;
    pl.bk = p.dtype == MICONV_BF16 ? 32 : 16;   // 64 bytes of reduction per tile row
    if (p.pass == FWD) {
        pl.rows = Kg; pl.cols = p.N * vout; pl.red = Cg * taps;
    } else if (p.pass == BWD_DATA) {
        pl.rows = Cg; pl.cols = p.N * vin; pl.red = Kg * taps;
    } else {
        pl.rows = Kg; pl.cols = Cg * taps; pl.red = p.N * vout;
    }
    pl.m_tiles = (int)cdiv_ll(pl.rows, pl.bm);
    pl.n_tiles = (int)cdiv_ll(pl.cols, pl.bn);
    pl.splits = 1;
    pl.chunk = cdiv_ll(pl.red, pl.bk) * pl.bk;
    if (p.pass == BWD_FILTER) {
        // about two work-groups per CU, at least 8 reduction steps per split, within the budget
        const long long tiles = (long long)p.G * pl.m_tiles * pl.n_tiles;
        long long want = cdiv_ll(512, tiles);
        const long long maxs = pl.red / (8LL * pl.bk);
        if (want > maxs) want = maxs;
        if (want < 1) want = 1;
        const size_t per = (size_t)p.K * (size_t)pl.cols * 4;
        if (want > 1) {
            const long long fit = (long long)(budget / ((per + 255) & ~(size_t)255));
            if (fit < 2) want = 1;
            else if (want > fit) want = fit;
        }
        pl.chunk = cdiv_ll(cdiv_ll(pl.red, want), pl.bk) * pl.bk;
        pl.splits = (int)cdiv_ll(pl.red, pl.chunk);
        if (pl.splits > 1) {
            pl.part_bytes = per * pl.splits;
            pl.ws_used = (pl.part_bytes + 255) & ~(size_t)255;
        }
    }
    *out = pl;
}

void nd_padding(int mode, int in, int f, int st, int dil, int *lo, int *hi, int *out) {
    if (mode == MICONV_PAD_SAME) {
        const int o = (in + st - 1) / st;
        long long tot = (long long)(o - 1) * st + (long long)dil * (f - 1) + 1 - in;
        if (tot < 0) tot = 0;
        *lo = (int)(tot / 2);
        *hi = (int)(tot - tot / 2);
        *out = o;
    } else {
        *lo = *hi = 0;
        *out = nd_out_dim(in, f, 0, 0, st, dil);
    }
}

void describe_nd_plan(const NdProblem &p, const NdPlan &pl, char *buf, size_t buflen) {
    static const char *names[] = {"fwd", "bwd_data", "bwd_filter"};
    if (!buf || buflen == 0) return;
    snprintf(buf, buflen,
             "pass=%s dtype=%s algo=generic groups=%d gemm=%lldx%lldx%lld tile=%dx%dx%d grid=%dx%dx%dx%d "
             "splits=%d chunk=%lld ws=%zu",
             names[p.pass], p.dtype ? "bf16" : "f32", p.G, pl.rows, pl.cols, pl.red, pl.bm, pl.bn, pl.bk, p.G,
             pl.m_tiles, pl.n_tiles, pl.splits, pl.splits, pl.chunk, pl.ws_used);
}

}  // namespace miconv
