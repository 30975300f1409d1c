// plan.cpp -- validation and plan selection for the implicit-GEMM kernels.
// Pure host code; compiled into the library and, on its own, into a CPU test.
#include "plan.h"

#include <stdio.h>
#include <string.h>

#include <mutex>
#include <unordered_map>

#include "../../include/miconv.h"

namespace miconv {

static const long long kMaxTensorBytes = (1LL << 31) - 1;  // tensors must be < 2 GiB
static const size_t kWsCap = (size_t)MICONV_MAX_WORKSPACE_BYTES;
static const int kCUs = 256;

int validate_problem(const Problem &p) {
    if (p.dtype != MICONV_F32 && p.dtype != MICONV_BF16) return MICONV_ERR_DTYPE;
    if (p.N <= 0 || p.C <= 0 || p.H <= 0 || p.W <= 0 || p.K <= 0 || p.R <= 0 || p.S <= 0)
        return MICONV_ERR_BAD_DIM;
    if (p.ph < 0 || p.pw < 0 || p.sh < 1 || p.sw < 1) return MICONV_ERR_BAD_DIM;
    // keep every index computation comfortably inside 32-bit arithmetic
    if (p.H > (1 << 20) || p.W > (1 << 20) || p.R > (1 << 20) || p.S > (1 << 20) ||
        p.ph > (1 << 20) || p.pw > (1 << 20) || p.sh > (1 << 20) || p.sw > (1 << 20))
        return MICONV_ERR_TOO_LARGE;
    int P = out_dim(p.H, p.ph, p.R, p.sh), Q = out_dim(p.W, p.pw, p.S, p.sw);
    if (P < 1 || Q < 1) return MICONV_ERR_BAD_DIM;
    if (p.P != P || p.Q != Q) return MICONV_ERR_OUT_SIZE;
    size_t xb, wb, yb;
    tensor_bytes(p, &xb, &wb, &yb);
    if ((long long)xb > kMaxTensorBytes || (long long)wb > kMaxTensorBytes ||
        (long long)yb > kMaxTensorBytes)
        return MICONV_ERR_TOO_LARGE;
    // fp32 copies of the other-side tensors (dx / dW outputs are fp32 too)
    long long nchw = (long long)p.N * p.C * p.H * p.W, nkpq = (long long)p.N * p.K * P * Q;
    long long kcrs = (long long)p.K * p.C * p.R * p.S;
    if (4 * nchw > kMaxTensorBytes || 4 * nkpq > kMaxTensorBytes || 4 * kcrs > kMaxTensorBytes)
        return MICONV_ERR_TOO_LARGE;
    return MICONV_OK;
}

void tensor_bytes(const Problem &p, size_t *x_bytes, size_t *w_bytes, size_t *y_bytes) {
    size_t es = p.dtype == MICONV_BF16 ? 2 : 4;
    size_t nchw = (size_t)p.N * p.C * p.H * p.W, nkpq = (size_t)p.N * p.K * p.P * p.Q;
    size_t kcrs = (size_t)p.K * p.C * p.R * p.S;
    *w_bytes = kcrs * es;
    if (p.pass == FWD) {
        *x_bytes = nchw * es;   // x
        *y_bytes = nkpq * 4;    // y
    } else if (p.pass == BWD_DATA) {
        *x_bytes = nkpq * es;   // dy
        *y_bytes = nchw * 4;    // dx
    } else {
        *x_bytes = nchw * es;   // x (dy is nkpq * es, checked by the caller)
        *y_bytes = kcrs * 4;    // dW
    }
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

static long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

static bool allowed(const PlanHints &h, int algo) { return (h.families >> algo) & 1; }

// Stride-1 bf16 forward / backward-data with whole output rows per tile: one
// LDS patch of input rows per 32-channel chunk serves every filter tap.
static void choose_patch(const Problem &p, size_t budget, Plan *pl, const PlanHints &h) {
    if (!allowed(h, ALGO_PATCH)) return;
    if (p.dtype != MICONV_BF16 || p.sh != 1 || p.sw != 1) return;
    const bool fwd = p.pass == FWD;
    const int Cr = fwd ? p.C : p.K, M = fwd ? p.K : p.C;
    const int Hi = fwd ? p.H : p.P, Wi = fwd ? p.W : p.Q, Ho = fwd ? p.P : p.H, Wo = fwd ? p.Q : p.W;
    if (Cr % 32 != 0 || Wi % 2 != 0) return;
    if (p.ph > p.R - 1 || p.pw > p.S - 1) return;
    int bm, cap;
    // 64 filter rows: bands of up to 256 pixels (two waves along the rows, four
    // 32-pixel blocks each); more rows: 128-row tiles of up to 224 pixels
    if (M <= 64) { bm = 64; cap = 256; }
    else { bm = 128; cap = 224; }
    int tr = cap / Wo;
    if (tr < 1) return;
    if (tr > Ho) tr = Ho;
    if (h.max_tr > 0 && tr > h.max_tr) tr = h.max_tr;
    int vw = Wi % 8 == 0 ? 8 : (Wi % 4 == 0 ? 4 : 2);
    // the 128-row form of the runtime-tap kernel (not 3x3) has registers for
    // fill items of at most 4 column groups; fewer rows per tile keep its fill
    // item count (4 per patch row and column group) within 512
    if (bm == 128 && !(p.R == 3 && p.S == 3)) {
        if (vw == 8) vw = 4;
        while (tr > 1 && 4LL * (tr + p.R - 1) * (Wi / vw) > 512) --tr;
    }
    const long long pr = tr + p.R - 1, pwc = Wo + p.S - 1;
    // 80-byte positions repeat their LDS banks every 16 positions: a row stride
    // congruent to Wo (mod 16) keeps the 16 pixels a half-wave reads (which may
    // wrap to the next row) on 16 distinct bank groups.  Two work-groups per CU
    // if that fits, else the plain stride.
    long long pws = pwc + ((Wo - pwc) % 16 + 16) % 16;
    if (2 * pr * pws * 80 * 2 > 160 * 1024) pws = pwc;
    const long long lds = 2 * pr * pws * 80;   // two patch buffers
    if (lds > 160 * 1024) return;
    if (4 * pr * (Wi / vw) > 512) return;
    // filter copy in MFMA fragment order, rows padded to whole BM tiles
    const size_t wbytes = (size_t)((M + bm - 1) / bm) * bm * Cr * p.R * p.S * 2;
    if (align256(wbytes) > budget) return;
    pl->algo = ALGO_PATCH;
    pl->bm = bm;
    pl->bn = tr * Wo;
    pl->wm = bm == 64 ? 2 : 4;
    pl->tr = tr;
    pl->vw = vw;
    pl->pws = (int)pws;
    // A 128-row tile of 193..208 pixels (a 14 x 14 image, say) fills its seventh 32-pixel
    // block with at most 16 pixels: that block runs as one 16-pixel block on 16x16x32
    // MFMAs, half the MFMA work of a 32-pixel block (3x3, fill loads of 2 columns, the
    // register budget of that kernel).
    pl->tail = bm == 128 && p.R == 3 && p.S == 3 && vw == 2 && tr * Wo > 192 && tr * Wo <= 208 && !h.no_tail;
    pl->m_tiles = (M + bm - 1) / bm;
    pl->n_tiles = ((Ho + tr - 1) / tr) * p.N;
    pl->nz = 1;
    pl->wt = 1;
    pl->wt_offset = 0;
    pl->wt_bytes = wbytes;
}

// Geometry shared by every stride phase of a backward-data problem along one
// dimension, when the phases are uniform: taps per phase nu, outputs per phase na,
// and the range [pmin, pmax] of the phases' paddings nu - 1 - base (each phase is a
// stride-1 correlation of dy with its nu taps, reversed, and that padding).
struct PhaseSpan {
    bool ok;
    int nu, na, pmin, pmax;
};
static PhaseSpan phase_span(int stride, int pad, int in, int filt) {
    PhaseSpan s = {true, 0, 0, 1 << 30, -(1 << 30)};
    for (int f = 0; f < stride; ++f) {
        const PhaseDim d = phase_dim(f, stride, pad, in, filt);
        if (f == 0) {
            s.nu = d.nu;
            s.na = d.na;
        }
        const int padf = d.nu - 1 - d.base;
        if (d.nu != s.nu || d.na != s.na || d.nu < 1 || padf < 0 || padf > d.nu - 1) s.ok = false;
        if (padf < s.pmin) s.pmin = padf;
        if (padf > s.pmax) s.pmax = padf;
    }
    return s;
}

// bf16 backward-data with strides of 2 whose stride phases are uniform 2 x 2-tap
// correlations (a 4x4 filter at stride 2, as in a transposed convolution): all the
// phases in one launch of the compile-time-tap patch kernel, each phase a stride-1
// correlation of dy written to every second dx row and column; no zero-inserted tap
// is visited.
static void choose_patch_phases(const Problem &p, size_t budget, Plan *pl, const PlanHints &h) {
    if (!allowed(h, ALGO_PATCH)) return;
    if (p.pass != BWD_DATA || p.dtype != MICONV_BF16 || p.sh != 2 || p.sw != 2) return;
    const PhaseSpan sh = phase_span(p.sh, p.ph, p.H, p.R), sw = phase_span(p.sw, p.pw, p.W, p.S);
    if (!sh.ok || !sw.ok || sh.nu != 2 || sw.nu != 2) return;
    if (p.K % 32 != 0 || p.Q % 2 != 0) return;
    const int M = p.C, Wi = p.Q, Ho = sh.na, Wo = sw.na;
    // the 64-row form computes 256 pixels per tile, the 128-row form 224 (with fill items
    // of 2 columns, for its registers): take the feasible one that computes fewer padding
    // rows and pixels (the phase images are small, so a ragged last row band can waste
    // most of a tile)
    int bm = 0, tr = 0, vw = 0;
    long long pws = 0;
    double best = 0.0;
    for (int b : {128, 64}) {
        const int cap = b == 64 ? 256 : 224;
        int t = cap / Wo;
        if (t < 1) continue;
        if (t > Ho) t = Ho;
        if (h.max_tr > 0 && t > h.max_tr) t = h.max_tr;
        const int v = b == 128 ? 2 : (Wi % 8 == 0 ? 8 : (Wi % 4 == 0 ? 4 : 2));
        const long long pr = t + sh.nu - 1 + (sh.pmax - sh.pmin), pwc = Wo + sw.nu - 1 + (sw.pmax - sw.pmin);
        long long s = pwc + ((Wo - pwc) % 16 + 16) % 16;
        if (2 * pr * s * 80 * 2 > 160 * 1024) s = pwc;
        if (2 * pr * s * 80 > 160 * 1024) continue;
        if (4 * pr * (Wi / v) > 512) continue;
        if (sw.pmax + Wi > s) continue;   // every dy column lands inside its patch row
        const double useful = (double)Ho * Wo * M;
        const double computed = (double)((Ho + t - 1) / t) * cap * ((M + b - 1) / b) * b;
        if (useful / computed > best) {
            best = useful / computed;
            bm = b;
            tr = t;
            vw = v;
            pws = s;
        }
    }
    if (bm == 0) return;
    const int nph = p.sh * p.sw, taps = sh.nu * sw.nu;
    const size_t per = (size_t)((M + bm - 1) / bm) * bm * p.K * taps * 2;   // fragment bytes per phase
    if (((per * nph + 255) & ~(size_t)255) > budget) return;
    pl->algo = ALGO_PATCH;
    pl->phases = nph;
    pl->bm = bm;
    pl->bn = tr * Wo;
    pl->wm = bm == 64 ? 2 : 4;
    pl->tr = tr;
    pl->vw = vw;
    pl->pws = (int)pws;
    pl->m_tiles = (M + bm - 1) / bm;
    pl->n_tiles = ((Ho + tr - 1) / tr) * p.N * nph;
    pl->nz = 1;
    pl->wt = 1;
    pl->wt_offset = 0;
    pl->wt_bytes = per * nph;
}

// Rows of the space-to-depth image z for a stride-2 dimension (input size `in`, padding
// `pad`, even filter size f, output size `out`): the taps of phase a (r - pad = 2u + a) have
// u = u0(a) .. u0(a) + f/2 - 1, and z row i of phase a is input row 2(i + u0(a)) + a.
static int s2d_u0(int a, int pad) {
    const int r0 = ((a + pad) % 2 + 2) % 2;   // smallest tap of the phase
    return (r0 - pad - a) / 2;                // exact: r0 - pad - a is even
}

// bf16 forward at stride 2 x 2 with a 4x4 filter (the deconvolution workload's input
// gradient): x regrouped as z[n][(2a + b)*C + c][i][j] = x[n][c][2(i + u0(a)) + a][2(j + u0(b)) + b]
// (zero outside x), then a stride-1 correlation of z with the 2 x 2 sub-filters, pad 0,
// on the 64-row patch kernel.  Rows of z: P + 1; columns: Q + 1, padded with zeros to a
// multiple of 8 (16-byte fill loads).
static void choose_patch_s2d(const Problem &p, size_t budget, Plan *pl, const PlanHints &h) {
    if (!allowed(h, ALGO_PATCH)) return;
    if (p.pass != FWD || p.dtype != MICONV_BF16 || p.sh != 2 || p.sw != 2 || p.R != 4 || p.S != 4) return;
    if (p.C % 8 != 0) return;
    const int Cz = 4 * p.C, Rz = p.R / 2, Sz = p.S / 2;
    const int zh = p.P + Rz - 1, zwc = p.Q + Sz - 1, zw = (zwc + 7) / 8 * 8;
    const int bm = 64, cap = 256;
    int tr = cap / p.Q;
    if (tr < 1) return;
    if (tr > p.P) tr = p.P;
    // few tiles (a small problem): shorter tiles, so that at least one per CU runs
    const long long mt = (p.K + bm - 1) / bm;
    while (tr > 1 && mt * p.N * ((p.P + tr - 1) / tr) < kCUs) tr = (tr + 1) / 2;
    if (h.max_tr > 0 && tr > h.max_tr) tr = h.max_tr;
    int vw = 8;
    while (tr > 1 && 4LL * (tr + Rz - 1) * (zw / vw) > 512) --tr;
    if (4LL * (tr + Rz - 1) * (zw / vw) > 512) return;
    const long long pr = tr + Rz - 1, pwc = p.Q + Sz - 1;
    long long pws = pwc + ((p.Q - pwc) % 16 + 16) % 16;   // banks, as in choose_patch
    if (pws < zw) pws = zw + ((p.Q - zw) % 16 + 16) % 16;   // every loaded column has a position
    if (2 * pr * pws * 80 > 160 * 1024) return;
    const size_t wbytes = (size_t)((p.K + bm - 1) / bm) * bm * Cz * Rz * Sz * 2;
    const size_t zbytes = (size_t)p.N * Cz * zh * zw * 2;
    if (align256(wbytes) + align256(zbytes) > budget) return;
    if ((long long)p.N * Cz * zh * zw * 2 > kMaxTensorBytes) return;
    pl->algo = ALGO_PATCH;
    pl->s2d = 1;
    pl->bm = bm;
    pl->bn = tr * p.Q;
    pl->wm = 2;
    pl->tr = tr;
    pl->vw = vw;
    pl->pws = (int)pws;
    pl->m_tiles = (p.K + bm - 1) / bm;
    pl->n_tiles = ((p.P + tr - 1) / tr) * p.N;
    pl->nz = 1;
    pl->wt = 1;
    pl->wt_offset = 0;
    pl->wt_bytes = wbytes;
    pl->zh = zh;
    pl->zw = zw;
    pl->z_offset = align256(wbytes);
    pl->z_bytes = zbytes;
    pl->cols = (long long)p.N * p.P * p.Q;
    pl->red = (long long)Cz * Rz * Sz;
}

// 1x1 bf16 forward / backward-data with no padding and equal strides 1 or 2 and
// an input of exactly stride x output size: one GEMM per image (rows = output
// channels in tiles of 256, columns = whole output rows of 128 pixels or fewer,
// reduction in chunks of 32 channels).  Backward-data reads a transposed filter copy from
// the workspace.
static void choose_pointwise(const Problem &p, size_t budget, Plan *pl, const PlanHints &h) {
    if (!allowed(h, ALGO_POINTWISE)) return;
    if (p.dtype != MICONV_BF16 || p.R != 1 || p.S != 1 || p.ph != 0 || p.pw != 0) return;
    if (p.sh != p.sw || (p.sh != 1 && p.sh != 2)) return;
    if (p.H != p.sh * p.P || p.W != p.sw * p.Q) return;
    const bool fwd = p.pass == FWD;
    const int red = fwd ? p.C : p.K;
    if (red % 32 != 0 || p.Q % 4 != 0 || p.Q > 128) return;
    if (fwd && p.sh == 2 && p.W % 8 != 0) return;
    const size_t wbytes = fwd ? 0 : (size_t)p.K * p.C * 2;
    if (align256(wbytes) > budget) return;
    const int tr = 128 / p.Q < p.P ? 128 / p.Q : p.P;
    pl->algo = ALGO_POINTWISE;
    pl->bm = 256;
    pl->bn = tr * p.Q;
    pl->wm = 4;
    pl->tr = tr;
    pl->m_tiles = ((fwd ? p.K : p.C) + 255) / 256;
    pl->n_tiles = ((p.P + tr - 1) / tr) * p.N;
    pl->nz = 1;
    pl->wt = !fwd;
    pl->wt_offset = 0;
    pl->wt_bytes = wbytes;
}

// Stride-1 bf16 backward-filter: a work-group owns (filter rows x channel block x
// all taps) over a range of output-row bands; split-K over the bands.
// Target split count scaled by the hints (at least 1).
static long long hinted_splits(long long want, const PlanHints &h) {
    if (h.one_split) return 1;
    if (h.split_shift > 0) want <<= h.split_shift;
    if (h.split_shift < 0) want >>= -h.split_shift;
    return want < 1 ? 1 : want;
}

// 1x1 bf16 backward-filter with no padding, equal strides 1 or 2 and an input of exactly
// stride x output size: one GEMM (rows k, columns c in 128 x 128 tiles) over the flat
// pixel index in steps of 64, split-K to about one work-group per CU within the budget.
// 8-pixel dy pieces stay in one image (P*Q % 8 == 0) and 4-pixel x pieces in one row
// (Q % 4 == 0); x rows start 16-byte aligned at stride 2 (W % 8 == 0); an image holds at
// least 64 pixels and as many rows as a 64-pixel step spans.
static void choose_pointwise_bwdf(const Problem &p, size_t budget, Plan *pl, const PlanHints &h) {
    if (!allowed(h, ALGO_POINTWISE)) return;
    if (p.dtype != MICONV_BF16 || p.R != 1 || p.S != 1 || p.ph != 0 || p.pw != 0) return;
    if (p.sh != p.sw || (p.sh != 1 && p.sh != 2)) return;
    if (p.H != p.sh * p.P || p.W != p.sw * p.Q) return;
    const long long PQ = (long long)p.P * p.Q, total = p.N * PQ;
    if (PQ % 8 != 0 || p.Q % 4 != 0 || p.W % (p.sh == 2 ? 8 : 4) != 0) return;
    // the kernel's pixel positions advance 64 pixels per step with one image wrap and one row
    // wrap at most
    if (PQ < 64 || 64 / p.Q + (64 % p.Q ? 1 : 0) > p.P) return;
    const long long mt = cdiv(p.K, 128), ct = cdiv(p.C, 128), steps = cdiv(total, 64);
    long long want = hinted_splits(cdiv(kCUs, mt * ct), h);
    if (want > steps) want = steps;
    const size_t per = (size_t)p.K * p.C * 4;
    if (want > 1) {
        const long long fit = (long long)(budget / align256(per));
        if (fit < 2) want = 1;
        else if (want > fit) want = fit;
    }
    const long long per_split = cdiv(steps, want);
    const long long splits = cdiv(steps, per_split);
    pl->algo = ALGO_POINTWISE;
    pl->bm = 128;
    pl->bn = 128;
    pl->wm = 2;
    pl->k16 = 1;
    pl->stream = 0;
    pl->pair = 0;
    pl->m_tiles = (int)mt;
    pl->n_tiles = (int)ct;
    pl->chunk = (int)(per_split * 64);
    pl->splits = (int)splits;
    pl->nz = (int)splits;
    pl->wt = 0;
    pl->wt_bytes = 0;
    pl->part_offset = 0;
    pl->part_bytes = splits > 1 ? per * splits : 0;
}

// Fill schedule of the 16x16x32 backward-filter kernel's stream form, run as the
// kernel runs it: the patch of image i of a split is filled (one item per step,
// two items) from the first step after the last step that reads image i - 2 (step
// s covers the split's pixels 32s .. 32s + 31).  True when every image's patch is
// stored at least two steps before the first step that reads it (the B reads of a
// step are issued during the step before).  Each image's timing depends on P*Q
// alone and repeats with a period of at most 32 images, so 70 images cover
// every split.
static bool stream_schedule_ok(long long PQ, long long nimg) {
    long long fimg = 2, fitem = 0, fstep = ((fimg - 1) * PQ - 1) / 32 + 1;
    const long long nsteps = (nimg * PQ + 31) / 32;
    for (long long s = 0; s < nsteps && fimg < nimg; ++s) {
        if (s < fstep) continue;
        if (++fitem < 2) continue;
        if (s > (fimg * PQ) / 32 - 2) return false;   // item 1 stored at step s
        fitem = 0;
        ++fimg;
        fstep = ((fimg - 1) * PQ - 1) / 32 + 1;
    }
    return true;
}

static void choose_bwdf_patch(const Problem &p, size_t budget, Plan *pl, const PlanHints &h) {
    if (!allowed(h, ALGO_PATCH)) return;
    if (p.dtype != MICONV_BF16 || p.sh != 1 || p.sw != 1) return;
    if (p.R * p.S > 9 || p.W % 2 != 0) return;
    if (p.ph > p.R - 1 || p.pw > p.S - 1) return;
    const int bc = 32;
    if (p.C % bc != 0) return;
    const int noct = bc / 8, pwc = p.Q + p.S - 1;
    // 3x3 filters: the 16x16x32 kernel (64- or 128-row tiles), bands of at most 224
    // pixels (7 steps); its patch is two 16-channel sub-patches of 32-byte positions,
    // and a row stride congruent to Q (mod 8) keeps the 8 consecutive positions of
    // one read pass on distinct bank groups across row wraps.  It stages dy in
    // 4-pixel pieces, so P*Q and the band's pixel count must be multiples of 4.
    // Other shapes: the 32x32x16 kernel (64 or 128 rows), 64-byte positions, whose
    // transpose reads need a row stride congruent to Q (mod 4).
    int tr = 0, vw = 2, pws = pwc, bm = 64;
    bool k16 = false, stream = false;
    for (int attempt = 0; attempt < 2 && tr < 1; ++attempt) {
        k16 = attempt == 0 && p.R == 3 && p.S == 3 && !h.no_k16;
        bm = p.K <= 64 ? 64 : 128;
        vw = p.W % 8 == 0 ? 8 : (p.W % 4 == 0 ? 4 : 2);
        if (k16 && bm == 128 && vw == 8) vw = 4;   // register budget of the 128-row form
        const int G = p.W / vw;
        pws = k16 ? pwc + ((p.Q - pwc) % 8 + 8) % 8 : pwc + ((p.Q - pwc) % 4 + 4) % 4;
        // 16x16x32 kernel, stream form: whole images (patch of the whole image, three
        // dy slots, two work-groups per CU), P*Q a multiple of 4, the fill schedule met
        if (k16 && !h.no_stream && (bm == 64 || vw == 2)) {   // 128 rows: 4-byte fill loads (registers)
            const long long pr = p.P + p.R - 1, PQ = (long long)p.P * p.Q;
            if (noct * pr * G <= 512 && (long long)bwdf16s_lds_bytes(bm, (int)pr, pws) <= 78 * 1024 && PQ % 4 == 0 &&
                stream_schedule_ok(PQ, 70)) {
                stream = true;
                tr = p.P;
                break;
            }
        }
        // largest band (whole output rows) whose patch fits the LDS budget (two
        // work-groups per CU) and the fill registers
        tr = p.P;
        while (tr > 0) {
            const long long pr = tr + p.R - 1;
            const long long lds = k16 ? (long long)bwdf16_lds_bytes(bm, (int)pr, pws) : 2LL * pr * pws * 64;
            if (noct * pr * G <= 512 && lds <= 78 * 1024 && (!k16 || (long long)tr * p.Q <= 224)) break;
            --tr;
        }
        if (k16 && tr >= 1 && ((long long)p.P * p.Q % 4 != 0 || (long long)tr * p.Q % 4 != 0)) tr = 0;
    }
    if (tr < 1) return;
    const long long bands = (long long)p.N * ((p.P + tr - 1) / tr);
    const int m_tiles = (p.K + bm - 1) / bm, c_tiles = p.C / bc;
    const long long tiles = (long long)m_tiles * c_tiles;
    // about two work-groups per CU; one for the banded 16x16x32 form (resnet3x3: 128 splits
    // of 7 bands ran 3-5 % faster than 224 of 4, with 43 % fewer partial sums)
    long long splits = hinted_splits(cdiv((k16 && !stream ? 1LL : 2LL) * kCUs, tiles), h);
    if (splits > bands) splits = bands;
    const size_t per = (size_t)p.K * p.C * p.R * p.S * 4;
    if (splits > 1) {
        long long fit = (long long)(budget / align256(per));
        if (fit < 2) splits = 1;
        else if (splits > fit) splits = fit;
    }
    const long long bps = cdiv(bands, splits);
    splits = cdiv(bands, bps);
    pl->algo = ALGO_PATCH;
    pl->bm = bm;
    pl->bn = bc;
    pl->wm = bm == 64 ? 2 : 4;
    pl->tr = tr;
    pl->vw = vw;
    pl->pws = pws;
    pl->m_tiles = m_tiles;
    pl->n_tiles = c_tiles;
    pl->splits = (int)splits;
    pl->nz = (int)splits;
    pl->chunk = (int)bps;   // bands per split
    // pair form (32x32x16 kernel, 64 filter rows, 3x3, exactly two bands per split):
    // both patches are filled first and each wave pair takes one band
    pl->k16 = k16;
    pl->stream = stream;
    pl->pair = !k16 && bm == 64 && p.R == 3 && p.S == 3 && bps == 2;
    pl->part_offset = 0;
    pl->part_bytes = splits > 1 ? per * splits : 0;
}

// Pairs of dx rows per work-group of the MFMA few-channel backward-data form.
// Two work-groups fit a CU (LDS and registers); each costs about four dy-row
// loads of warm-up besides its pairs, so the cost of PB pairs per work-group is
// rounds * (PB + 3/4) with rounds = ceil(N * ceil(pairs / PB) / (2 * CUs)).
static int tinyc_pairs(const Problem &p) {
    const int npairs = (p.H + 1) / 2;
    int best = 1;
    long long best_cost = -1;
    for (int pb = 1; pb <= npairs; ++pb) {
        const long long groups = (long long)p.N * cdiv(npairs, pb);
        const long long rounds = (groups + 2 * kCUs - 1) / (2 * kCUs);
        const long long cost = rounds * (4LL * pb + 3);
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = pb; }
    }
    return best;
}

void make_plan(const Problem &p, size_t ws_limit, Plan *out, const PlanHints &h) {
    Plan pl = {};
    pl.pass = p.pass;
    pl.dtype = p.dtype;
    const int es = p.dtype == MICONV_BF16 ? 2 : 4;
    pl.vec = 16 / es;
    const size_t budget = ws_limit < kWsCap ? ws_limit : kWsCap;
    const long long RS = (long long)p.R * p.S;
    size_t used = 0;

    if (p.pass == FWD || p.pass == BWD_DATA) {
        pl.bk_bytes = 64;
        long long rows = p.pass == FWD ? p.K : p.C;
        long long redc = p.pass == FWD ? p.C : p.K;   // channels inside one tap
        long long cols, red;
        if (p.pass == FWD) {
            cols = (long long)p.N * p.P * p.Q;
            red = RS * p.C;
            pl.nz = 1;
        } else {
            cols = 0;
            red = 0;
            for (int fh = 0; fh < p.sh; ++fh)
                for (int fw = 0; fw < p.sw; ++fw) {
                    PhaseDim dh = phase_dim(fh, p.sh, p.ph, p.H, p.R);
                    PhaseDim dw = phase_dim(fw, p.sw, p.pw, p.W, p.S);
                    long long c = (long long)p.N * dh.na * dw.na;
                    long long r = (long long)dh.nu * dw.nu * p.K;
                    if (c > cols) cols = c;
                    if (r > red) red = r;
                }
            pl.nz = p.sh * p.sw;
        }
        int bm = h.bm == 32 || h.bm == 64 || h.bm == 128 ? h.bm : (rows <= 32 ? 32 : (rows <= 64 ? 64 : 128));
        // fp32: 128 x 128 tiles that leave CUs idle give way to 32 x 256 tiles where those fill
        // more of the chip (the deconvolution's backward-data: 128 tiles against 256)
        if (h.bm == 0 && bm == 128 && p.dtype == MICONV_F32) {
            const long long t128 = cdiv(rows, 128) * cdiv(cols, 128) * pl.nz;
            const long long t32 = cdiv(rows, 32) * cdiv(cols, 256) * pl.nz;
            if (t128 < kCUs && t32 > t128) bm = 32;
        }
        if (bm == 32) {
            pl.bm = 32; pl.bn = 256; pl.wm = 1;
        } else if (bm == 64) {
            pl.bm = 64; pl.bn = 256; pl.wm = 1;
        } else {
            pl.bm = 128; pl.bn = 128; pl.wm = 2;
        }
        pl.cvec = (redc % pl.vec) == 0;
        pl.rows = rows;
        pl.cols = cols;
        pl.red = red;
        pl.m_tiles = (int)cdiv(rows, pl.bm);
        pl.n_tiles = (int)cdiv(cols > 0 ? cols : 1, pl.bn);
        // tap-major filter copy: forward K x (R*S) x C, backward-data (R*S) x C x K.
        // A 1x1 forward filter is already in that order.
        size_t wbytes = (size_t)p.K * p.C * RS * es;
        bool need = !(p.pass == FWD && RS == 1);
        if (!need) {
            pl.wt = 1;
        } else if (align256(wbytes) <= budget) {
            pl.wt = 1;
            pl.wt_offset = 0;
            pl.wt_bytes = wbytes;
            used = align256(wbytes);
        } else {
            pl.wt = 0;
        }
        pl.splits = 1;
        choose_patch(p, budget, &pl, h);
        choose_patch_phases(p, budget, &pl, h);
        if (pl.algo == ALGO_PATCH) used = align256(pl.wt_bytes);
        choose_pointwise(p, budget, &pl, h);
        if (pl.algo == ALGO_POINTWISE) used = align256(pl.wt_bytes);
        choose_patch_s2d(p, budget, &pl, h);
        if (pl.s2d) used = align256(pl.wt_bytes) + align256(pl.z_bytes);
        // fp32 forward with at most 4 input channels, 7 filter rows, column stride 2 (the 7x7
        // stem): the few-channel MFMA kernel, runs of output rows, two work-groups per CU
        if (allowed(h, ALGO_TINYC) && !h.no_tc_mma && p.pass == FWD && p.dtype == 0 && p.K == 64 && p.C <= 4 &&
            p.R == 7 && p.S >= 4 && p.sw == 2 && p.C * RS <= 4 * kTcFwdSteps && p.Q <= 4 * kTcQT &&
            2 * (4 * kTcQT - 1) + p.S <= kTcXWP) {
            const long long orows = (long long)p.N * p.P;
            pl.algo = ALGO_TINYC;
            pl.tc_rows = (int)cdiv(orows, 2LL * kCUs);
            pl.wt = 0;
            pl.wt_bytes = 0;
            pl.s2d = 0;
            used = 0;
        }
        // backward-data with at most 4 input channels: as a GEMM it has C rows
        // (mostly padding in an MFMA tile); fp32 vector ALUs, no workspace, for
        // fp32 and bf16 inputs alike.
        if (allowed(h, ALGO_TINYC) && p.pass == BWD_DATA && p.C <= 4 && p.sh <= 2 && p.sw <= 2 && p.R <= 16 &&
            p.S <= 16) {
            pl.algo = ALGO_TINYC;
            pl.wt = 0;
            pl.wt_bytes = 0;
            used = 0;
            // fp32 at stride 2 with 7 filter rows: the MFMA form (C*S columns of a 32-wide tile)
            if (p.dtype == 0 && p.sh == 2 && p.sw == 2 && p.R == 7 && p.C * p.S <= 32 && p.Q <= 128 &&
                (p.K == 32 || p.K == 64) && 124LL * p.P * p.Q < (1LL << 31) && !h.no_tc_mma)
                pl.tc_pairs = tinyc_pairs(p);
        }
    } else {
        // backward-filter: reduction over pixels; 64 pixels per LDS row.
        pl.bk_bytes = 64 * es;
        const int bk = 64;
        long long rows = p.K, cols = RS * p.C, red = (long long)p.N * p.P * p.Q;
        pl.bm = h.bm == 64 || h.bm == 128 ? h.bm : (rows <= 64 ? 64 : 128);
        pl.bn = 128;
        pl.wm = 2;
        pl.cvec = (p.C % pl.vec) == 0;
        pl.pqvec = ((long long)p.P * p.Q) % pl.vec == 0;
        pl.rows = rows;
        pl.cols = cols;
        pl.red = red;
        pl.m_tiles = (int)cdiv(rows, pl.bm);
        pl.n_tiles = (int)cdiv(cols, pl.bn);
        long long tiles = (long long)pl.m_tiles * pl.n_tiles;
        // enough work-groups for two waves of the chip, at least 8 reduction tiles each; in
        // fp32 (reduction steps twice as long) one wave when that leaves each split at most
        // 2048 pixels (longer splits then lose more to cold reads than they save in partials)
        const long long one_wave = cdiv(kCUs, tiles);
        const bool short_splits = p.dtype == MICONV_F32 && cdiv(red, one_wave) <= 2048;
        long long want = hinted_splits(short_splits ? one_wave : cdiv(2LL * kCUs, tiles), h);
        long long maxs = red / (8LL * bk);
        if (want > maxs) want = maxs;
        if (want < 1) want = 1;
        size_t per = (size_t)rows * cols * 4;
        if (want > 1) {
            long long fit = (long long)(budget / align256(per));
            if (fit < 2) want = 1;
            else if (want > fit) want = fit;
        }
        long long chunk = cdiv(cdiv(red, want), bk) * bk;
        long long splits = cdiv(red, chunk);
        pl.chunk = (int)chunk;
        pl.splits = (int)splits;
        pl.nz = (int)splits;
        if (splits > 1) {
            pl.part_offset = 0;
            pl.part_bytes = per * splits;
            used = align256(pl.part_bytes);
        }
        choose_bwdf_patch(p, budget, &pl, h);
        if (pl.algo == ALGO_PATCH) used = pl.splits > 1 ? align256(pl.part_bytes) : 0;
        // stride 2, or stride 1 where the patch kernel does not apply
        if (pl.algo != ALGO_PATCH || p.sh == 2) choose_pointwise_bwdf(p, budget, &pl, h);
        if (pl.algo == ALGO_POINTWISE) used = pl.splits > 1 ? align256(pl.part_bytes) : 0;
        // fp32, at most 4 input channels, 7 filter rows, column stride 2 (the 7x7 stem): the
        // few-channel MFMA kernel, two work-groups per CU (its registers allow two waves per
        // SIMD), when the partial sums of at least 64 splits fit the budget
        if (allowed(h, ALGO_TINYC) && !h.no_tc_mma && p.dtype == 0 && p.K == 64 && p.C <= 4 && p.R == 7 &&
            p.sw == 2 && p.C * RS <= 160 && p.Q % 4 == 0 && p.Q <= 4 * kTcQT && 2 * (4 * kTcQT - 1) + p.S <= kTcXWP) {
            const long long orows = (long long)p.N * p.P;
            const size_t per = (size_t)p.K * p.C * RS * 4;
            long long want = hinted_splits(2LL * kCUs, h);
            if (want > orows) want = orows;
            if (want > 1) {
                const long long fit = (long long)(budget / align256(per));
                if (want > fit) want = fit < 1 ? 1 : fit;
            }
            if (want >= 64 || want == orows || h.one_split) {
                const long long rpw = cdiv(orows, want < 1 ? 1 : want);
                const long long splits = cdiv(orows, rpw);
                pl.algo = ALGO_TINYC;
                pl.tc_rows = (int)rpw;
                pl.splits = (int)splits;
                pl.nz = (int)splits;
                pl.chunk = 0;
                pl.part_offset = 0;
                pl.part_bytes = splits > 1 ? per * splits : 0;
                used = splits > 1 ? align256(pl.part_bytes) : 0;
            }
        }
    }
    pl.ws_used = used;
    *out = pl;
}

void describe_plan(const Plan &pl, char *buf, size_t buflen) {
    static const char *names[] = {"fwd", "bwd_data", "bwd_filter"};
    if (!buf || buflen == 0) return;
    char tc[48];
    if (pl.pass != BWD_DATA)
        snprintf(tc, sizeof tc, " form=mfma rows=%d", pl.tc_rows);
    else
        snprintf(tc, sizeof tc, " form=mfma pairs=%d", pl.tc_pairs);
    snprintf(buf, buflen,
             "pass=%s dtype=%s algo=%s gemm=%lldx%lldx%lld tile=%dx%dx%dB waves_m=%d grid=%dx%dx%d "
             "cvec=%d pqvec=%d wt=%d splits=%d chunk=%d%s%s ws=%zu",
             names[pl.pass], pl.dtype ? "bf16" : "f32",
             pl.algo == ALGO_PATCH ? "patch"
                                   : (pl.algo == ALGO_TINYC ? "tinyc" : (pl.algo == ALGO_POINTWISE ? "pointwise" : "igemm")),
             pl.rows,
             pl.cols, pl.red, pl.bm, pl.bn,
             pl.bk_bytes, pl.wm, pl.m_tiles, pl.n_tiles, pl.nz, pl.cvec, pl.pqvec, pl.wt, pl.splits,
             pl.chunk,
             pl.pass == BWD_FILTER && pl.algo == ALGO_POINTWISE ? " mma=16x16x32"
             : pl.pass == BWD_FILTER && pl.algo == ALGO_PATCH
                 ? (pl.pair ? (pl.k16 ? " form=pair mma=16x16x32" : " form=pair mma=32x32x16")
                            : (pl.k16 ? (pl.stream ? " form=stream mma=16x16x32" : " form=bands mma=16x16x32")
                                      : " form=bands mma=32x32x16"))
                 : "",
             pl.phases > 1 ? " phases=4 form=phase-patch"
                           : (pl.s2d ? " form=space-to-depth"
                                     : (pl.algo == ALGO_PATCH && pl.tail
                                            ? " form=tail16"
                                            : (pl.algo == ALGO_TINYC && (pl.tc_pairs || pl.tc_rows) ? tc : ""))),
             pl.ws_used);
}

bool same_plan(const Plan &a, const Plan &b) {
    return a.algo == b.algo && a.bm == b.bm && a.bn == b.bn && a.wm == b.wm && a.tr == b.tr && a.vw == b.vw &&
           a.pws == b.pws && a.wt == b.wt && a.wt_bytes == b.wt_bytes && a.splits == b.splits &&
           a.chunk == b.chunk && a.k16 == b.k16 && a.stream == b.stream && a.pair == b.pair && a.phases == b.phases &&
           a.s2d == b.s2d && a.tail == b.tail && a.tc_pairs == b.tc_pairs && a.tc_rows == b.tc_rows &&
           a.m_tiles == b.m_tiles &&
           a.n_tiles == b.n_tiles && a.nz == b.nz;
}

int enumerate_plans(const Problem &p, size_t ws_limit, Plan *out, int max) {
    if (max <= 0) return 0;
    const int generic = 1 << ALGO_IGEMM;
    PlanHints hs[kMaxCandidates * 2];
    int nh = 0;
    hs[nh++] = PlanHints();   // the default choice first
    Plan def;
    make_plan(p, ws_limit, &def);
    if (p.pass == FWD || p.pass == BWD_DATA) {
        if (def.algo == ALGO_PATCH) {   // shorter patch tiles; seven full blocks for a tail form
            for (int d = 2; d <= 4; d *= 2)
                if (def.tr / d >= 1) { hs[nh] = PlanHints(); hs[nh].max_tr = def.tr / d; ++nh; }
            if (def.tail) { hs[nh] = PlanHints(); hs[nh].no_tail = 1; ++nh; }
        }
        if (def.algo == ALGO_TINYC && (def.tc_pairs || def.tc_rows)) {   // the vector-ALU form / generic kernel
            hs[nh] = PlanHints(); hs[nh].no_tc_mma = 1; ++nh;
        }
        if (def.algo == ALGO_POINTWISE) {   // the patch kernel where it also applies
            hs[nh] = PlanHints(); hs[nh].families &= ~(1 << ALGO_POINTWISE); ++nh;
        }
        for (int bm : {0, 32, 64, 128}) {   // the generic implicit GEMM with each tile height
            hs[nh] = PlanHints(); hs[nh].families = generic; hs[nh].bm = bm; ++nh;
        }
    } else {
        for (int fam : {0xF, generic}) {
            for (int s = 0; s < 4; ++s) {   // default, half, double, one split
                PlanHints h;
                h.families = fam;
                if (s == 1) h.split_shift = -1;
                if (s == 2) h.split_shift = 1;
                if (s == 3) h.one_split = 1;
                hs[nh++] = h;
            }
        }
        PlanHints h;
        h.no_stream = 1;
        hs[nh++] = h;
        h.no_stream = 0;
        h.no_k16 = 1;
        hs[nh++] = h;
        h.families = generic;
        h.no_k16 = 0;
        h.bm = 64; hs[nh++] = h;
        h.bm = 128; hs[nh++] = h;
        if (def.algo == ALGO_TINYC) {   // the generic kernel with its own split counts
            PlanHints hn;
            hn.no_tc_mma = 1;
            hs[nh++] = hn;
        }
        PlanHints hp;   // the pointwise kernel where the patch kernel is the default (1x1, stride 1)
        hp.families = generic | (1 << ALGO_POINTWISE);
        hs[nh++] = hp;
    }
    int n = 0;
    for (int i = 0; i < nh && n < max; ++i) {
        Plan pl;
        make_plan(p, ws_limit, &pl, hs[i]);
        bool dup = false;
        for (int j = 0; j < n && !dup; ++j) dup = same_plan(out[j], pl);
        if (!dup) out[n++] = pl;
    }
    return n;
}

// ------------------------------------------------------------------ plan cache
namespace {

struct CacheKey {
    int v[15];        // pass, dtype, 13 sizes
    size_t budget;    // effective budget of a default entry; kTuned for a tuned plan
    bool operator==(const CacheKey &o) const { return budget == o.budget && memcmp(v, o.v, sizeof v) == 0; }
};

struct CacheHash {
    size_t operator()(const CacheKey &k) const {
        uint64_t h = 1469598103934665603ull ^ (uint64_t)k.budget;
        for (int x : k.v) h = (h ^ (uint32_t)x) * 1099511628211ull;
        return (size_t)h;
    }
};

constexpr size_t kTuned = ~(size_t)0;
constexpr size_t kMaxDefaultEntries = 4096;

std::mutex g_mu;
std::unordered_map<CacheKey, Plan, CacheHash> g_cache;
int g_tuned = 0;

CacheKey key_of(const Problem &p, size_t budget) {
    CacheKey k;
    const int v[15] = {p.pass, p.dtype, p.N, p.C, p.H, p.W, p.K, p.R, p.S, p.ph, p.pw, p.sh, p.sw, p.P, p.Q};
    memcpy(k.v, v, sizeof v);
    k.budget = budget;
    return k;
}

}  // namespace

void cached_plan(const Problem &p, size_t ws_limit, Plan *out) {
    const size_t budget = ws_limit < kWsCap ? ws_limit : kWsCap;
    {
        std::lock_guard<std::mutex> g(g_mu);
        auto t = g_cache.find(key_of(p, kTuned));
        if (t != g_cache.end() && t->second.ws_used <= budget) {
            *out = t->second;
            return;
        }
        auto d = g_cache.find(key_of(p, budget));
        if (d != g_cache.end()) {
            *out = d->second;
            return;
        }
    }
    Plan pl;
    make_plan(p, budget, &pl);
    std::lock_guard<std::mutex> g(g_mu);
    if (g_cache.size() - g_tuned >= kMaxDefaultEntries) {   // bounded: drop the default entries
        for (auto it = g_cache.begin(); it != g_cache.end();)
            it = it->first.budget == kTuned ? std::next(it) : g_cache.erase(it);
    }
    g_cache[key_of(p, budget)] = pl;
    *out = pl;
}

void set_tuned_plan(const Problem &p, const Plan &pl) {
    std::lock_guard<std::mutex> g(g_mu);
    auto r = g_cache.insert_or_assign(key_of(p, kTuned), pl);
    if (r.second) ++g_tuned;
}

void drop_tuned_plan(const Problem &p) {
    std::lock_guard<std::mutex> g(g_mu);
    g_tuned -= (int)g_cache.erase(key_of(p, kTuned));
}

void clear_plan_cache() {
    std::lock_guard<std::mutex> g(g_mu);
    g_cache.clear();
    g_tuned = 0;
}

void plan_cache_counts(int *tuned, int *total) {
    std::lock_guard<std::mutex> g(g_mu);
    if (tuned) *tuned = g_tuned;
    if (total) *total = (int)g_cache.size();
}

}  // namespace miconv
