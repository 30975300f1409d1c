// launch.h -- kernel argument block and the host entry into the HIP kernels.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/miconv.h"
#include "common.h"
#include "plan.h"

namespace miconv {

// Arguments of every implicit-GEMM kernel (passed by value).
struct KArgs {
    const void *a0;       // forward: x;  backward-data: dy;  backward-filter: x
    const void *a1;       // forward / backward-data: filter (tap-major copy when wt); backward-filter: dy
    float *out;           // y, dx, dW, or the split-K partial sums
    uint32_t a0_bytes, a1_bytes;
    int N, C, H, W, K, R, S, ph, pw, sh, sw, P, Q;
    int wt;               // a1 is the tap-major filter copy
    int m_tiles, n_tiles, nz;
    int chunk;            // backward-filter: pixels per split
    int direct;           // backward-filter: write dW (one split) instead of partial sums
    int use_map;          // backward-data: z indexes live_map (phases with taps only)
    int live_map[16];     // backward-data: phase fh*sw + fw of each z
    FDiv fd_PQ, fd_Q, fd_C, fd_S, fd_K;
    Epi epi;              // forward: the fused epilogue (EPI template); backward passes: the
    int has_epi;          // output epilogue alpha / beta / bf16 when has_epi
};

// Arguments of the stride-1 LDS-patch kernel (passed by value).
struct PatchArgs {
    const void *X;        // gathered activations [N][Cr][Hi][Wi] (bf16)
    const void *Wt;       // tap-major filter [M][R*S][Cr] (bf16)
    float *O;             // output [N][M][Ho][Wo] (fp32)
    uint32_t x_bytes, w_bytes;
    int N, Cr, Hi, Wi, M, R, S, ph, pw, Ho, Wo;
    int TR, row_tiles, m_tiles;
    int PWc, PR, G;       // patch width / rows; column groups per input row
    int PWs;              // patch row stride in positions (>= PWc)
    Epi epi;              // the fused epilogue (EPI kernels); bias over the M output rows
    // Output placement.  A tile's pixel (row a, column b of the Ho x Wo grid) goes to
    // output row ph_i0[phase] + osh*a, column ph_j0[phase] + osw*b of an OH x OW plane
    // (OHW = OH*OW elements).  Plain runs: one phase, osh = osw = 1, OW = Wo.
    // Backward-data by stride phases (compile-time-tap kernel only): nph phases, each a
    // stride-1 correlation with its own filter fragments (wt_phase bytes apart) whose
    // patch reads start ph_boff[phase] bytes into the shared patch layout.
    int nph, osh, osw, OW, OHW;
    uint32_t wt_phase;
    int ph_i0[4], ph_j0[4], ph_boff[4];
};

// Arguments of the stride-1 backward-filter patch kernel.
struct BFArgs {
    const void *X, *DY;   // x [N][C][H][W], dy [N][K][P][Q] (bf16)
    float *out;           // partial sums [splits][K][R*S][C], or dW [K][C][R][S] when direct
    uint32_t x_bytes, dy_bytes;
    int N, C, H, W, K, R, S, ph, pw, P, Q;
    int TR, row_bands, m_tiles, c_tiles, splits, bands_per_split;
    int PWc, PR, G;
    int PWs;              // patch row stride in positions
    int direct;
    FDiv fd_Q;
    FDiv fd_rb;           // division by row_bands
    FDiv fd_PQ;           // division by P*Q (stream form)
    Epi epi;              // output epilogue of a direct (one-split) write, when has_epi
    int has_epi;
};

// Arguments of the few-input-channel backward-data kernel.
struct TCArgs {
    const void *DY, *Wt;  // dy [N][K][P][Q], filter [K][C][R][S] (fp32 or bf16)
    float *DX;            // dx [N][C][H][W] fp32
    uint32_t dy_bytes, w_bytes;
    int N, C, H, W, K, R, S, ph, pw, sh, sw, P, Q;
    int DH, DW;           // dy window rows / columns one tile reads
    int DWs;              // LDS row stride of the window (>= DW, = 1 mod 32)
    FDiv fd_DW, fd_DHW;   // division by DW and by DH * DW
    int dyw_bytes;        // LDS bytes of the staged dy window
    Epi epi;              // output epilogue, when has_epi
    int has_epi;
    int PB, nbands, phq;  // MFMA form: dx row pairs per work-group, work-groups per image, ph / 2
};

// Few-channel fp32 forward and backward-filter on 16x16x4 MFMAs (plan.tc_rows > 0).
struct TFArgs {
    const void *X, *DY;   // x [N][C][H][W], dy [N][K][P][Q] (fp32; backward-filter)
    const void *Wt;       // filter [K][C][R][S] (fp32; forward)
    float *out;           // forward: y [N][K][P][Q]; backward-filter: dW [K][C][R][S] (direct) or
                          // partials [split][K][R*S][C]
    uint32_t x_bytes, dy_bytes;
    int C, H, W, K, R, S, ph, pw, sh, P, Q;
    int CRS, RS;          // filter values per k, taps
    int rows, rpw;        // output rows N*P; rows per work-group
    int direct;           // one split: apply the epilogue and write dW
    Epi epi;
    int has_epi;
};
int launch_tinyc_bwdf(const Plan &pl, const Problem &p, const void *x, const void *dy, float *dw, void *ws,
                      hipStream_t st, const Epi *epi);
int launch_tinyc_fwd(const Plan &pl, const Problem &p, const void *x, const void *w, float *y, hipStream_t st,
                     const Epi *epi);

// Stride-1 bf16 backward-filter of a 3x3 filter on 16x16x32 MFMAs (plan.k16).
int launch_bwdf16(const Plan &pl, const Problem &p, const void *x, const void *dy, float *dw, void *ws,
                  hipStream_t st, const Epi *epi);

int launch_bwdf_patch(const Plan &pl, const Problem &p, const void *x, const void *dy, float *dw, void *ws,
                      hipStream_t st, const Epi *epi);

// Backward-data for C <= 4 and strides of 1 or 2 (vector ALUs, fp32).
int launch_tinyc(const Plan &pl, const Problem &p, const void *dy, const void *w, float *dx, hipStream_t st, const Epi *epi);

// Deterministic second stage of split-K: dW[k][c][t] = sum_{z = 0 .. splits-1} part[z][k][t][c],
// through the output epilogue when epi is not null.
int launch_splitk_reduce(const float *part, float *dw, int K, int C, int T, int splits, hipStream_t st,
                         const Epi *epi = nullptr);

// db[k] = alpha * sum_{n,pq} dy[n][k][pq] + beta * db[k] (fixed-order fp64 sums).
int launch_bias_grad(int dtype, int N, int K, int PQ, const void *dy, float alpha, float beta, float *db,
                     hipStream_t st);

// Work-groups of `func` the current device holds at once (cached occupancy query).
hipError_t resident_slots(const void *func, int threads, size_t lds, int *slots);

// 1x1 bf16 pointwise path (forward or backward-data, pad 0, stride 1 or 2).
int launch_pointwise(const Plan &pl, const Problem &p, const void *in0, const void *in1, float *out, void *ws,
                     hipStream_t st, const Epi *epi);

// The generalised convolution (nd.h) on the generic MFMA kernel.
struct NdProblem;
struct NdPlan;
int launch_nd(const NdProblem &p, const NdPlan &pl, const void *in0, const void *in1, float *out, void *ws,
              hipStream_t st);

// Stride-1 patch path (forward, or backward-data as a forward over dy).
int launch_patch(const Plan &pl, const Problem &p, const void *in0, const void *in1, float *out, void *ws,
                 hipStream_t st, const Epi *epi);

// Validates the problem and its pointers, plans under min(ws_bytes, 1e9) and
// enqueues the kernels on `stream` (the body of every compute entry point).
int run_problem(const Problem &p, const void *in0, const void *in1, float *out, void *ws, size_t ws_bytes,
                void *stream, const Epi *epi = nullptr);

// Enqueues the plan's kernels on `st`.  Arguments are already validated.  `epi`
// (may be null): forward, the fused epilogue; backward passes, the output
// epilogue alpha / beta / bf16 output (bias and ReLU unused).
int launch_plan(const Plan &pl, const Problem &p, const void *in0, const void *in1, float *out,
                void *ws, hipStream_t st, const Epi *epi = nullptr);

}  // namespace miconv
