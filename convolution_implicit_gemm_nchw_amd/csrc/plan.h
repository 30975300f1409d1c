// plan.h -- host-side problem validation and plan selection (no HIP calls).
//
// Every pass is an implicit GEMM (rows x cols x reduction) over the NCHW /
// KCRS tensors, with the reduction index ordered tap-major (filter tap outer,
// channel inner) so that one vector of consecutive reduction indices shares a
// single padding predicate:
//   forward          rows = K, cols = N*P*Q,                 reduction = (R*S) x C
//   backward-data    per stride phase (ph_h, ph_w):
//                    rows = C, cols = N*|I_phase|*|J_phase|, reduction = (phase taps) x K
//   backward-filter  rows = K, cols = (R*S) x C,              reduction = N*P*Q (split-K)
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace miconv {

enum Pass { FWD = 0, BWD_DATA = 1, BWD_FILTER = 2 };

struct Problem {
    int pass;   // FWD / BWD_DATA / BWD_FILTER (deconvolution arrives as BWD_DATA)
    int dtype;  // 0 fp32, 1 bf16
    int N, C, H, W, K, R, S, ph, pw, sh, sw, P, Q;
};

enum Algo { ALGO_IGEMM = 0, ALGO_PATCH = 1, ALGO_TINYC = 2, ALGO_POINTWISE = 3 };

struct Plan {
    int pass, dtype;
    int algo;             // ALGO_IGEMM (gathered tiles), ALGO_PATCH (stride-1 LDS patch),
                          // ALGO_TINYC (C <= 4: backward-data, fp32 backward-filter) or
                          // ALGO_POINTWISE (1x1 bf16, pad 0, stride 1 or 2: GEMM per image)
    int tr, vw;           // patch: output rows per tile, columns per global load
    int pws;              // patch: row stride in positions
    int bm, bn, wm;       // work-group tile rows x cols, waves along rows
    int bk_bytes;         // bytes of one LDS tile row (reduction slice)
    int vec;              // elements per 16-byte vector (4 fp32, 8 bf16)
    int cvec;             // reduction channel count is a multiple of vec
    int pqvec;            // backward-filter: P*Q is a multiple of vec
    int wt;               // filter operand is the tap-major transformed copy
    size_t wt_offset, wt_bytes;    // transformed filter inside the workspace
    int splits;           // backward-filter split-K count (1 = direct write)
    int chunk;            // backward-filter: pixels per split (multiple of the reduction tile);
                          // patch form: bands per split
    int pair;             // backward-filter patch: the pair form (bands taken two at a time by wave pairs)
    int k16;              // patch kernels on v_mfma_f32_16x16x32_bf16 (else 32x32x16)
    int stream;           // backward-filter 16x16x32 kernel: stream form (whole images, 32 pixels
                          // per step across image boundaries)
    int phases;           // patch backward-data by stride phases: their count (sh*sw), else 0
    int tail;             // patch forward / backward-data, 128 filter rows, 3x3: six 32-pixel blocks and a
                          // 16-pixel tail block on v_mfma_f32_16x16x32_bf16 (tiles of 193..208 pixels)
    int tc_pairs;         // tinyc backward-data, MFMA form (fp32, stride 2, 7 filter rows): pairs of dx
                          // rows per work-group; 0 = the vector-ALU form
    int tc_rows;          // tinyc backward-filter (MFMA form, fp32): output rows per work-group
    int s2d;              // patch forward at stride 2 by space-to-depth: x regrouped into its four
                          // stride phases as channels (z), a stride-1 correlation of z
    int zh, zw;           // space-to-depth: rows and row pitch (columns, zero-padded) of z
    size_t z_offset, z_bytes;   // z inside the workspace
    size_t part_offset, part_bytes;  // backward-filter partial sums inside the workspace
    size_t ws_used;       // total workspace bytes this plan touches
    int m_tiles, n_tiles, nz;        // tile grid; nz = stride phases or splits
    long long rows, cols, red;       // GEMM sizes (largest phase for backward-data)
};

// Floor output size; returns < 1 if the filter does not fit in the padded input.
inline int out_dim(int in, int pad, int f, int stride) {
    long long num = (long long)in + 2LL * pad - f;
    if (num < 0) return 0;
    return (int)(num / stride) + 1;
}

// 0 if the sizes are a valid convolution, else a MICONV_ERR_* status.
int validate_problem(const Problem &p);

// Bytes of each tensor of the problem (inputs in dtype, outputs fp32).
void tensor_bytes(const Problem &p, size_t *x_bytes, size_t *w_bytes, size_t *y_bytes);

// LDS bytes of the 16x16x32 backward-filter kernel: two patch buffers of PR x PWs
// positions (two 32-byte sub-patch halves each) and two staged dy slots of bm rows
// of 80 bytes.
inline size_t bwdf16_lds_bytes(int bm, int PR, int PWs) { return 2 * (size_t)PR * PWs * 64 + 2 * (size_t)bm * 80; }
// The few-channel fp32 backward-filter (MFMA form): QT pixels per lane group (rows of
// at most 4 * QT output pixels); LDS row pitch (floats) of a staged input row, which
// covers the 2 * (4 * QT - 1) + S columns a row's taps read for S <= 10; LDS bytes of
// one stage (4 channels x 7 rows) and of the kernel (two stages).
constexpr int kTcQT = 28, kTcXWP = 232;
constexpr int kTcFwdSteps = 37;   // forward: reduction steps of 4 filter values (C*R*S <= 148)
constexpr int kTcStage = 4 * 7 * kTcXWP * 4;
constexpr size_t kTcBwdfLds = 2 * (size_t)kTcStage;
// LDS of the MFMA form of the few-channel backward-data kernel: the filter as
// [R][C*S][kTcKP] and the column sums G as [2][C*S][kTcJP] (fp32).
constexpr int kTcKP = 68, kTcJP = 132;
inline size_t tinyc_mfma_lds_bytes(int R, int C, int S) {
    return ((size_t)R * C * S * kTcKP + 2 * (size_t)C * S * kTcJP) * 4;
}
// The same kernel's stream form (whole-image bands): three staged dy slots.
inline size_t bwdf16s_lds_bytes(int bm, int PR, int PWs) { return 2 * (size_t)PR * PWs * 64 + 3 * (size_t)bm * 80; }

// Restrictions that steer make_plan to an alternative plan (the candidates the
// autotuner times); the defaults give the standard choice.  Every combination
// yields a plan the kernels support.
struct PlanHints {
    int families = 0xF;   // bit (1 << algo) per allowed family; the generic implicit GEMM is the fallback
    int bm = 0;           // generic implicit GEMM tile rows: 32, 64 or 128 (backward-filter: 64 or 128);
                          // 0 = chosen from the GEMM's row count
    int max_tr = 0;       // patch forward / backward-data: at most this many output rows per tile
    int split_shift = 0;  // backward-filter: target split count times 2^split_shift
    int one_split = 0;    // backward-filter: a single split (direct write, no partial sums)
    int no_k16 = 0;       // backward-filter patch: the 32x32x16 kernel for 3x3 filters too
    int no_stream = 0;    // backward-filter 16x16x32 kernel: bands of at most 224 pixels, not the stream form
    int no_tail = 0;      // patch forward / backward-data: seven 32-pixel blocks, not the 16-pixel tail form
    int no_tc_mma = 0;    // C <= 4: backward-data in the vector-ALU form, backward-filter not in the
                          // few-channel MFMA kernel
};

// Chooses the plan; never needs more than min(ws_limit, 1e9) bytes.
void make_plan(const Problem &p, size_t ws_limit, Plan *out, const PlanHints &h = PlanHints());

// True when two plans launch the same kernels with the same tiling.
bool same_plan(const Plan &a, const Plan &b);

// Distinct candidate plans for the problem under min(ws_limit, 1e9) bytes (at
// most max; make_plan's default first); returns how many were written.
int enumerate_plans(const Problem &p, size_t ws_limit, Plan *out, int max);
constexpr int kMaxCandidates = 16;

// Process-wide plan cache (thread-safe).  The plan for (problem, budget) is
// the tuned plan installed for the problem's sizes when it fits the budget,
// else make_plan's choice (kept in the cache under the budget).
void cached_plan(const Problem &p, size_t ws_limit, Plan *out);
void set_tuned_plan(const Problem &p, const Plan &pl);
void drop_tuned_plan(const Problem &p);
void clear_plan_cache();
void plan_cache_counts(int *tuned, int *total);

// One-line plan description (for logging and tests).
void describe_plan(const Plan &pl, char *buf, size_t buflen);


}  // namespace miconv
