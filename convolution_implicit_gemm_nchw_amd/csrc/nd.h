// nd.h -- the generalised convolution (1 to 3 spatial dimensions, groups,
// dilation, separate low / high zero padding): problem, validation, plan.
// Host only (no HIP calls).
//
// Every problem is held in three spatial dimensions (D, H, W), a 2-D problem
// with D = T = OD = 1 and a 1-D one also with H = R = OH = 1 (pad 0, stride 1,
// dilation 1 in the unused dimensions).  Tensors, packed:
//   x [N][C][D][H][W],  w [K][C/G][T][R][S],  y [N][K][OD][OH][OW]
// Output channel k is in group g = k / (K/G) and reads input channels
// g*(C/G) .. g*(C/G) + C/G - 1.  Per group, each pass is an implicit GEMM:
//   forward          rows = K/G (k),  cols = N*OD*OH*OW,   reduction = (C/G)*T*R*S (c, t, r, s)
//   backward-data    rows = C/G (c),  cols = N*D*H*W,      reduction = (K/G)*T*R*S (k, t, r, s),
//                    a tap contributing only where (i + pad - t*dil) divides by the stride
//   backward-filter  rows = K/G (k),  cols = (C/G)*T*R*S,  reduction = N*OD*OH*OW (split-K)
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "plan.h"

namespace miconv {

struct NdProblem {
    int pass, dtype;
    int N, C, K, G;
    int in[3], f[3], out[3];    // D H W / T R S / OD OH OW
    int lo[3], hi[3], st[3], dil[3];
};

struct NdPlan {
    int bm, bn, bk;             // tile rows, cols, reduction elements per step
    long long rows, cols, red;  // per-group GEMM
    int m_tiles, n_tiles;
    int splits;                 // backward-filter split-K count (1 = direct write)
    long long chunk;            // reduction elements per split (multiple of bk)
    size_t part_bytes;          // split-K partial sums [splits][K][cols] fp32
    size_t ws_used;
};

// Builds the 3-D problem from the public descriptor's first ndim entries
// (outermost dimension first); MICONV_OK or MICONV_ERR_BAD_DIM for ndim.
int nd_from_desc(int pass, int dtype, int ndim, int N, int C, int K, int G, const int *in, const int *f,
                 const int *out, const int *lo, const int *hi, const int *st, const int *dil, NdProblem *p);

// 0 if valid, else a MICONV_ERR_* status (sizes, groups, output-size rule, 2 GiB limits).
int validate_nd(const NdProblem &p);

// floor((in + lo + hi - dil*(f-1) - 1) / st) + 1, or 0 when the dilated filter exceeds the
// padded input.
int nd_out_dim(int in, int f, int lo, int hi, int st, int dil);

// The plan of the generic kernel under min(ws_limit, 1e9) bytes of workspace.
void make_nd_plan(const NdProblem &p, size_t ws_limit, NdPlan *out);

// True (and the 2-D problem) when the problem is a plain 2-D convolution the
// specialised kernels run: one group, dilation 1, equal low and high padding,
// a depth of 1 (a 1-D problem runs as 2-D with H = R = 1).
bool nd_as_2d(const NdProblem &p, Problem *q);

// (lo, hi) padding and output sizes of a padding mode for each dimension:
// valid = no padding; same = output ceil(in / stride) with total padding
// max((out - 1)*stride + dil*(f - 1) + 1 - in, 0), the smaller half low.
void nd_padding(int mode, int in, int f, int st, int dil, int *lo, int *hi, int *out);

void describe_nd_plan(const NdProblem &p, const NdPlan &pl, char *buf, size_t buflen);

}  // namespace miconv
