// tinyc.hip -- backward-data for very few input channels (C <= 4), strides 1 or 2
// (fp32 or bf16 inputs, fp32 arithmetic and output).
//
// dx[n,c,i,j] = sum over k and the taps (r, s) with (i + ph - r) and (j + pw - s)
// divisible by the strides of W[k,c,r,s] * dy[n, k, (i + ph - r)/sh, (j + pw - s)/sw]
// (only taps whose dy index is inside the image contribute).
//
// As an implicit GEMM this has only C rows, so MFMA tiles would be mostly
// padding.  Two forms: for fp32 at stride 2 with 7 filter rows (the 7x7 stem)
// the MFMA form below regroups the sums so that the C * S (channel, filter
// column) pairs are the GEMM's columns; every other shape runs on the vector
// ALUs in fp32 (tinyc_bwd_data).  In the vector form a work-group owns
// a 16 x 64 tile of dx of one image.  Per chunk of 8 output channels k it
// stages in LDS the dy window the tile reads (zeros outside the image) and the
// chunk's filter as one 16-byte vector of (up to) 4 input channels per (k, r, s),
// read by every lane at the same address.  Each wave takes the pixels of one
// stride phase (i mod sh, j mod sw) of the tile, so all its lanes walk the same
// taps; a lane owns 4 consecutive pixels of one phase row x C accumulators.
// Those 4 pixels read overlapping dy columns at consecutive taps of a filter
// row, so the row segment they need (taps + 3 values) is loaded into
// registers once per filter row and every tap reads it from there.
#include "device.h"
#include "launch.h"

namespace miconv {

namespace {
constexpr int TH = 16, TW = 64, KC = 8;
}

template <int ES, int CM, int NSM>
__global__ __launch_bounds__(256) void tinyc_bwd_data(TCArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tiles_w = (a.W + TW - 1) / TW, tiles_h = (a.H + TH - 1) / TH;
    const int bid = blockIdx.x;
    const int tw = bid % tiles_w, rest = bid / tiles_w;
    const int th = rest % tiles_h, n = rest / tiles_h;
    const int i0 = th * TH, j0 = tw * TW;

    // dy window of the tile: rows p_lo .. p_lo+DH-1, columns q_lo .. q_lo+DW-1,
    // stored with a row stride DWs = 1 (mod 32) so the rows a wave reads spread
    // over the LDS banks
    auto floordiv = [](int x, int d) { return x >= 0 ? x / d : -((-x + d - 1) / d); };
    const int p_lo = floordiv(i0 + a.ph - (a.R - 1), a.sh), q_lo = floordiv(j0 + a.pw - (a.S - 1), a.sw);
    const int DH = a.DH, DW = a.DW, DWs = a.DWs;   // host: DH = (TH - 1 + R - 1)/sh + 2, DW likewise
    float *dyw = (float *)smem;                         // [KC][DH][DWs]
    float4 *wl = (float4 *)(smem + a.dyw_bytes);        // [KC][R][S] x 4 channels

    // this wave's stride phase; a lane owns 4 consecutive pixels of one phase row.
    // Phases have different tap counts (a 7x7 filter at stride 2: 16, 12, 12, 9)
    // and waves are placed on SIMDs by index, so the phase order is rotated per
    // work-group to spread the heavy phase over all SIMDs.
    const int nph = a.sh * a.sw, wpp = 4 / nph;
    const int wrot = (wave + bid) & 3;
    const int f = wrot / wpp, sub = wrot - f * wpp;
    const int ri = f / a.sw, rj = f - ri * a.sw;
    const int lpr = TW / a.sw / 4, rows_w = 64 / lpr;   // lanes per phase row, phase rows per wave
    // first tap of the phase along each dimension: r = r0, r0 + sh, ...
    const int r0 = ((i0 + ri + a.ph) % a.sh + a.sh) % a.sh, s0 = ((j0 + rj + a.pw) % a.sw + a.sw) % a.sw;
    const int nr = r0 < a.R ? (a.R - r0 + a.sh - 1) / a.sh : 0, ns = s0 < a.S ? (a.S - s0 + a.sw - 1) / a.sw : 0;
    const int aa = sub * rows_w + lane / lpr, b0 = 4 * (lane % lpr);
    const int pix_i = i0 + aa * a.sh + ri, pix_j0 = j0 + b0 * a.sw + rj;
    // window position of tap (r0, s0) for the lane's last pixel (e = 3); tap
    // (r0 + u*sh, s0 + v*sw) of pixel e reads u rows up and 3 - e + v columns left of it
    const int prow = (pix_i + a.ph - r0) / a.sh - p_lo, pcol3 = (pix_j0 + a.pw - s0) / a.sw + 3 - q_lo;
    const int base = prow * DWs + pcol3;

    float acc[4][CM];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int c = 0; c < CM; ++c) acc[e][c] = 0.f;

    const int plane = a.P * a.Q;
    const int RS = a.R * a.S;
    const rsrc_t rdy = make_rsrc(a.DY, a.dy_bytes), rw = make_rsrc(a.Wt, a.w_bytes);
    for (int k0 = 0; k0 < a.K; k0 += KC) {
        __syncthreads();   // every wave is done with the previous chunk
        // one window element per thread and step, four steps' loads in flight
        // before their LDS stores
        const int total = KC * DH * DW;
        for (int t0 = tid; t0 < total; t0 += 4 * 256) {
            uint32_t val[4];
            int dst[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = t0 + u * 256;
                const int kk = (int)fdiv((uint32_t)t, a.fd_DHW), rem = t - kk * DH * DW;
                const int row = (int)fdiv((uint32_t)rem, a.fd_DW), col = rem - row * DW;
                const int k = k0 + kk, p = p_lo + row, q = q_lo + col;
                const bool ok = t < total && k < a.K && (unsigned)p < (unsigned)a.P && (unsigned)q < (unsigned)a.Q;
                const uint32_t off = ok ? (uint32_t)(((n * a.K + k) * plane + p * a.Q + q) * ES) : kOOB;
                val[u] = ld_elem<ES>(rdy, off);
                dst[u] = t < total ? (kk * DH + row) * DWs + col : -1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (dst[u] >= 0) dyw[dst[u]] = ES == 4 ? __uint_as_float(val[u]) : __uint_as_float(val[u] << 16);
        }
        for (int t = tid; t < KC * RS; t += 256) {
            const int kk = t / RS, rs = t - kk * RS;
            const int k = k0 + kk;
            float wv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool ok = k < a.K && c < a.C;
                const uint32_t off = ok ? (uint32_t)(((k * a.C + c) * RS + rs) * ES) : kOOB;
                const uint32_t v = ld_elem<ES>(rw, off);
                wv[c] = ES == 4 ? __uint_as_float(v) : __uint_as_float(v << 16);
            }
            wl[t] = make_float4(wv[0], wv[1], wv[2], wv[3]);
        }
        __syncthreads();
        for (int kk = 0; kk < KC; ++kk) {
            const float *d = dyw + kk * DH * DWs + base;
            const float4 *wk = wl + kk * RS;
            for (int u = 0; u < nr; ++u) {
                // the dy row segment every tap of this filter row reads: vals[m] is
                // m columns left of the last pixel's (r, s0) position
                const float *dr = d - u * DWs;
                float vals[NSM + 3];
#pragma unroll
                for (int m = 0; m < NSM + 3; ++m) vals[m] = m < ns + 3 ? dr[-m] : 0.f;
                const float4 *wr = wk + (r0 + u * a.sh) * a.S + s0;
#pragma unroll
                for (int v = 0; v < NSM; ++v) {
                    if (v < ns) {
                        const float4 w4 = wr[v * a.sw];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float x = vals[3 - e + v];
                            acc[e][0] += w4.x * x;
                            if constexpr (CM > 1) acc[e][1] += w4.y * x;
                            if constexpr (CM > 2) acc[e][2] += w4.z * x;
                            if constexpr (CM > 3) acc[e][3] += w4.w * x;
                        }
                    }
                }
            }
        }
    }
    if (pix_i >= a.H) return;
    const int HW = a.H * a.W;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int pj = pix_j0 + e * a.sw;
        if (pj >= a.W) continue;
        const size_t o = (size_t)n * a.C * HW + (size_t)pix_i * a.W + pj;
#pragma unroll
        for (int c = 0; c < CM; ++c)
            out_store(a.DX, o + (size_t)c * HW, acc[e][c], a.epi, a.has_epi, a.epi.bias ? a.epi.bias[c] : 0.0f);
    }
}

// ------------------------------------------------------------------ MFMA form
// fp32 inputs, stride 2 both ways, a 7-row filter, C * S <= 32, Q <= 128, K = 32 or 64.
//
// Summing over the filter rows first gives, for a dx row i, a channel c, a filter
// column s and a dy column q,
//     G[c, s][i][q] = sum over k and the rows r with (i + ph - r) even of
//                     W[k, c, r, s] * dy[n, k, (i + ph - r) / 2, q],
// a GEMM with the dy columns as rows (M), the C * S pairs (c, s) as columns (N)
// and (k, r) as the reduction, on v_mfma_f32_32x32x2f32; then
//     dx[n, c, i, j] = sum over s with (j + pw - s) even of G[c, s][i][(j + pw - s) / 2].
// The C x (R*S) GEMM of the direct form has C rows; this one has C * S columns
// (the stem's 21 fill 66 % of a 32-column tile) and no padding in the reduction.
//
// A work-group takes PB consecutive pairs of dx rows (2m, 2m + 1) of one image.
// Pair m reads the four dy rows m + phq + DMIN .. m + phq + DMAX (the two rows'
// taps have opposite parities), so consecutive pairs share three: the rows live
// in a register ring of five, each pair loading the one the next pair adds.
// Wave w owns dy columns 32w .. 32w + 31; lane (q, h) holds k = 32h + t of
// column q for t = 0..31, the A operand of MFMA t.  The filter sits in LDS as
// [r][c*S + s][k] (rows padded to 68 floats), read as 16-byte B fragments for
// four MFMAs.  G goes through LDS for the column sums, which also apply the
// epilogue at the one store of each dx value.
template <int R, int PHP>
struct TmTaps {
    // dy row offset of tap r for dx row 2m + e, relative to m + phq (exact: e + PHP - r is even)
    static constexpr bool live(int e, int r) { return ((e + PHP + r) & 1) == 0; }
    static constexpr int drow(int e, int r) { return (e + PHP - r) / 2; }
    static constexpr int dmin() {
        int m = 1 << 20;
        for (int e = 0; e < 2; ++e)
            for (int r = 0; r < R; ++r)
                if (live(e, r) && drow(e, r) < m) m = drow(e, r);
        return m;
    }
    static constexpr int dmax() {
        int m = -(1 << 20);
        for (int e = 0; e < 2; ++e)
            for (int r = 0; r < R; ++r)
                if (live(e, r) && drow(e, r) > m) m = drow(e, r);
        return m;
    }
};

constexpr int kTmKP = kTcKP, kTmJP = kTcJP;   // LDS row pitches (floats) of the filter and of G

template <int R, int PHP>
__global__ __launch_bounds__(256) void tinyc_mfma_bwd_data(TCArgs a) {
    using TT = TmTaps<R, PHP>;
    constexpr int DMIN = TT::dmin(), DMAX = TT::dmax(), NR = DMAX - DMIN + 1, NRING = NR + 1;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, jl = lane & 31, h = lane >> 5;
    const int CS = a.C * a.S;
    const int n = blockIdx.x / a.nbands, band = blockIdx.x - n * a.nbands;
    const int npairs = (a.H + 1) >> 1, m_beg = band * a.PB;
    const int PBe = min(a.PB, npairs - m_beg);
    float *wl = (float *)smem;                 // [R][CS][kTmKP]
    float *gl = wl + R * CS * kTmKP;           // [2][CS][kTmJP]

    // dy rows into the ring: lane's column jc, k = 32h + t
    const rsrc_t rdy = make_rsrc(a.DY, a.dy_bytes);
    // K is 32 or 64, so a lane half's 32 channels are all present or all absent.  An
    // absent row, column or half gets the base kOOB, past the buffer's end, so its
    // loads read zeros; a present one stays inside dy for all 32 channels.  The
    // channel step t * P*Q*4 is the uniform offset of the load (kOOB plus it stays
    // below 2^32: the plan bounds P*Q), so every load is issued unconditionally and
    // needs no address register of its own.
    const int jc = wave * 32 + jl, kq = 32 * h;
    const uint32_t pq4 = (uint32_t)(a.P * a.Q) * 4u;
    const int ibase = m_beg + a.phq;           // dy row of offset 0 for the band's first pair
    float ring[NRING][32];
    auto load_row = [&](float(&dst)[32], int i) {
        const bool ok = (unsigned)i < (unsigned)a.P && jc < a.Q && kq < a.K;
        const uint32_t base = ok ? (uint32_t)((((n * a.K + kq) * a.P + i) * a.Q + jc) * 4) : kOOB;
#pragma unroll
        for (int t = 0; t < 32; ++t)
            dst[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdy, (int)base, (int)(t * pq4), 0));
    };
#pragma unroll
    for (int d = DMIN; d <= DMAX; ++d) load_row(ring[d - DMIN], ibase + d);

    // the filter: wl[r][c*S + s][k] = W[k, c, r, s], zero for k >= K
    for (int t = tid; t < R * CS * kTmKP / 4; t += 256) ((f32x4 *)wl)[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    {
        const float *W = (const float *)a.Wt;
        const int rows = a.K * a.C * R;       // filter rows (k, c, r) of S values
        for (int t = tid; t < rows; t += 256) {
            const int r = t % R, kc = t / R;
            const int c = kc % a.C, k = kc / a.C;
            const float *src = W + (size_t)t * a.S;
            float *dst = wl + (r * CS + c * a.S) * kTmKP + k;
            for (int s = 0; s < a.S; ++s) dst[s * kTmKP] = src[s];
        }
    }
    __syncthreads();

    const int colc = jl < CS ? jl : CS - 1;    // columns past C*S compute unused values
    const float *wlane = wl + colc * kTmKP + kq;
    const int rstride = CS * kTmKP;

    for (int m0 = 0; m0 < PBe; m0 += NRING) {
#pragma unroll
        for (int u = 0; u < NRING; ++u) {
            const int m = m0 + u;
            if (m >= PBe) break;
            // the row the next pair adds (past the band's last pair it is read and unused)
            load_row(ring[(u + NR) % NRING], ibase + m + DMAX + 1);
            f32x16 acc[2];
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[e][v] = 0.f;
            // taps two at a time (opposite parities, so the two dx rows' sums interleave),
            // the last filter rows first: they read the oldest dy rows, and the row
            // loaded during the previous pair comes last
#pragma unroll
            for (int r0 = R - 1; r0 >= 0; r0 -= 2) {
#pragma unroll
                for (int qd = 0; qd < 8; ++qd) {
                    const f32x4 b0 = *(const f32x4 *)(wlane + r0 * rstride + 4 * qd);
                    f32x4 b1 = b0;
                    if (r0 >= 1) b1 = *(const f32x4 *)(wlane + (r0 - 1) * rstride + 4 * qd);
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
#pragma unroll
                        for (int dr = 0; dr < 2; ++dr) {
                            const int r = r0 - dr;
                            if (r < 0) continue;
                            const int e = (PHP + r) & 1;
                            const int slot = (u + TT::drow(e, r) - DMIN) % NRING;
                            acc[e] = __builtin_amdgcn_mfma_f32_32x32x2f32(ring[slot][4 * qd + z],
                                                                          dr ? b1[z] : b0[z], acc[e], 0, 0, 0);
                        }
                    }
                }
            }
            __syncthreads();   // the previous pair's column sums are done with G
            if (jl < CS) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    float *g = gl + (e * CS + jl) * kTmJP + wave * 32 + 4 * h;
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd)
                        *(f32x4 *)(g + 8 * qd) =
                            f32x4{acc[e][4 * qd], acc[e][4 * qd + 1], acc[e][4 * qd + 2], acc[e][4 * qd + 3]};
                }
            }
            __syncthreads();
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * (m_beg + m) + e;
                if (i >= a.H) continue;
                for (int c = 0; c < a.C; ++c) {
                    const float *g = gl + (e * CS + c * a.S) * kTmJP;
                    const float bias = a.has_epi && a.epi.bias ? a.epi.bias[c] : 0.0f;
                    const size_t orow = ((size_t)(n * a.C + c) * a.H + i) * a.W;
                    for (int j = tid; j < a.W; j += 256) {
                        float v = 0.f;
                        for (int s = (j + a.pw) & 1; s < a.S; s += 2) {
                            const int q = (j + a.pw - s) >> 1;
                            if ((unsigned)q < (unsigned)a.Q) v += g[s * kTmJP + q];
                        }
                        out_store(a.DX, orow + j, v, a.epi, a.has_epi, bias);
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ backward-filter, MFMA form
// dW[k, c, r, s] = sum over (n, p, q) of dy[n, k, p, q] * x[n, c, sh*p + r - ph, 2q + s - pw]
// for fp32, K = 64, C <= 4, 7 filter rows, column stride 2, C*R*S <= 160 and Q a
// multiple of 4, at most 4 * QT (the 7x7 stem).
//
// A GEMM with rows k, columns the C*R*S filter values in tap-major order
// (tap * C + c; 147 of 160 for the stem, ten tiles of 16) and the output pixels as
// the reduction, on v_mfma_f32_16x16x4f32.  A work-group takes a run of output
// rows (n, p); wave w owns k = 16w .. 16w + 15 and all ten column tiles.  Per
// output row the C * R input rows it reads go to LDS, double buffered, with zeros
// outside the image; the B fragment of a filter value is then one 4-byte read at
// a fixed offset per pixel.  The row's pixels are split into four runs of QT, run
// g feeding lane group g of the MFMA reduction (pixel g*QT + t in MFMA t), so a
// lane's A values for four consecutive MFMAs are one 16-byte load of dy.  A
// work-group's sums are one split of the fixed-order split-K reduce, or dW itself
// when there is one split.
DEVI uint32_t opaque_u32(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Input rows of output row `row` = n * P + p for one LDS stage ([C][R][kTcXWP]
// floats): thread tid loads column tid (input column tid - pw) of each of the C * R
// rows into xr, zeros outside the image (tc_load_x), and stores them (tc_store_x).
template <int R>
DEVI void tc_load_x(const TFArgs &a, rsrc_t rx, int row, int tid, float (&xr)[4 * R]) {
    const int n = row / a.P, p = row - n * a.P;
    const int iw = tid - a.pw;
    const bool colok = (unsigned)iw < (unsigned)a.W;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (c >= a.C) break;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int ih = a.sh * p - a.ph + r;
            const bool ok = colok && (unsigned)ih < (unsigned)a.H;
            const uint32_t off = opaque_u32(ok ? (uint32_t)((((n * a.C + c) * a.H + ih) * a.W + iw) * 4) : kOOB);
            xr[c * R + r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx, (int)off, 0, 0));
        }
    }
}
template <int R>
DEVI void tc_store_x(const TFArgs &a, const float (&xr)[4 * R], char *stage, int tid) {
    if (tid >= kTcXWP) return;
    float *dst = (float *)stage + tid;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (c >= a.C) break;
#pragma unroll
        for (int r = 0; r < R; ++r) dst[(c * R + r) * kTcXWP] = xr[c * R + r];
    }
}
template <int R>
DEVI void tc_stage_x(const TFArgs &a, rsrc_t rx, int row, char *stage, int tid) {
    float xr[4 * R];
    tc_load_x<R>(a, rx, row, tid, xr);
    tc_store_x<R>(a, xr, stage, tid);
}

template <int R, int QT>
__global__ __launch_bounds__(256) void tinyc_mfma_bwd_filter(TFArgs a) {
    constexpr int SW = 2, NT = 10, NU = QT / 4, CM = 4, XWP = kTcXWP;
    static_assert(QT % 4 == 0 && CM * R * XWP * 4 <= kTcStage, "16-byte dy loads; the LDS stage");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, kl = lane & 15, g = lane >> 4;
    const int row_beg = blockIdx.x * a.rpw, row_end = min(a.rows, row_beg + a.rpw);
    const rsrc_t rx = make_rsrc(a.X, a.x_bytes), rdy = make_rsrc(a.DY, a.dy_bytes);

    // B addresses (stage 0; stage 1 is kTcStage further): column tile j, lane column
    // kl -> filter value col = tap * C + c; columns past C*R*S read the last one and
    // are never stored
    uint32_t bofs[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int col = min(16 * j + kl, a.CRS - 1);
        const int t = col / a.C, c = col - t * a.C;
        const int r = t / a.S, s = t - r * a.S;
        bofs[j] = (uint32_t)(((c * R + r) * XWP + s + g * QT * SW) * 4);
    }

    auto stage_x = [&](int row, int stage) { tc_stage_x<R>(a, rx, row, smem + stage * kTcStage, tid); };
    // A: dy of k = 16 * wave + kl at pixels g*QT + 4u .. + 3
    f32x4 av[2][NU];
    auto load_a = [&](f32x4(&dst)[NU], int row) {
        const int n = row / a.P, p = row - n * a.P;
        const int k = 16 * wave + kl;
        const uint32_t base = (uint32_t)((((n * a.K + k) * a.P + p) * a.Q + g * QT) * 4);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const uint32_t off = opaque_u32(g * QT + 4 * u < a.Q ? base + 16u * u : kOOB);
            dst[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rdy, (int)off, 0, 0));
        }
    };

    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int stage, const f32x4(&A)[NU]) {
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int t = 4 * u + z;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const float b = *(const float *)(smem + bofs[j] + stage * kTcStage + t * SW * 4);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[u][z], b, acc[j], 0, 0, 0);
                }
            }
    };

    load_a(av[0], row_beg);
    stage_x(row_beg, 0);
    __syncthreads();
    // two rows per trip so the stage and the A set are fixed per half; the next row's
    // dy is loaded before the current row's MFMAs, its input rows after them (past
    // the last row both re-read the last row, unused)
    for (int row = row_beg; row < row_end; row += 2) {
        int nxt = min(row + 1, row_end - 1);
        load_a(av[1], nxt);
        compute(0, av[0]);
        stage_x(nxt, 1);
        __syncthreads();
        if (row + 1 >= row_end) break;
        nxt = min(row + 2, row_end - 1);
        load_a(av[0], nxt);
        compute(1, av[1]);
        stage_x(nxt, 0);
        __syncthreads();
    }

    // D: lane (kl, g) holds k = 16 * wave + 4g + v of column 16j + kl
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int col = 16 * j + kl;
        if (col >= a.CRS) continue;
        const int t = col / a.C, c = col - t * a.C;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int k = 16 * wave + 4 * g + v;
            if (a.direct)
                out_store(a.out, (uint32_t)((k * a.C + c) * a.RS + t), acc[j][v], a.epi, a.has_epi);
            else
                a.out[(uint32_t)((blockIdx.x * a.K + k) * a.CRS + col)] = acc[j][v];
        }
    }
}

int launch_tinyc_bwdf(const Plan &pl, const Problem &p, const void *x, const void *dy, float *dw, void *ws,
                      hipStream_t st, const Epi *epi) {
    // the plan checked fp32, K == 64, C <= 4, R == 7, sw == 2, C*R*S <= 160, Q % 4 == 0, Q <= 112
    TFArgs a = {};
    if (epi) a.epi = *epi;
    a.has_epi = epi ? 1 : 0;
    a.X = x;
    a.DY = dy;
    a.x_bytes = (uint32_t)((size_t)p.N * p.C * p.H * p.W * 4);
    a.dy_bytes = (uint32_t)((size_t)p.N * p.K * p.P * p.Q * 4);
    a.C = p.C; a.H = p.H; a.W = p.W; a.K = p.K; a.R = p.R; a.S = p.S;
    a.ph = p.ph; a.pw = p.pw; a.sh = p.sh; a.P = p.P; a.Q = p.Q;
    a.RS = p.R * p.S;
    a.CRS = p.C * a.RS;
    a.rows = p.N * p.P;
    a.rpw = pl.tc_rows;
    a.direct = pl.splits == 1;
    float *part = pl.splits > 1 ? (float *)((char *)ws + pl.part_offset) : dw;
    a.out = part;
    const size_t lds = kTcBwdfLds;
    const void *k = (const void *)tinyc_mfma_bwd_filter<7, kTcQT>;
    hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return MICONV_ERR_HIP;
    void *args[] = {&a};
    e = hipLaunchKernel(k, dim3(pl.splits), dim3(256), args, lds, st);
    if (e != hipSuccess) return MICONV_ERR_HIP;
    if (pl.splits > 1) return launch_splitk_reduce(part, dw, p.K, p.C, a.RS, pl.splits, st, epi);
    return MICONV_OK;
}

// ------------------------------------------------------------------ forward, MFMA form
// y[n, k, p, q] = sum over (c, r, s) of W[k, c, r, s] * x[n, c, sh*p + r - ph, 2q + s - pw]
// for fp32, K = 64, C <= 4, 7 filter rows, S >= 4, column stride 2, C*R*S <= 148
// and Q <= 112 (the 7x7 stem).
//
// A GEMM with rows k, the output pixels of a row as columns (seven tiles of 16 for
// Q = 112) and the C*R*S filter values as the reduction (steps of 4: 37 for the
// stem's 147), on v_mfma_f32_16x16x4f32.  A work-group takes a run of output rows;
// wave w owns k = 16w .. 16w + 15 and keeps its A operand (the filter, 4 values
// per lane and step, zero past C*R*S) in registers for the whole run.  The input
// rows go to LDS as in the backward-filter kernel; the B fragment of step t is one
// 4-byte read at a per-lane offset (filter value 4t + g of lane group g, pixel
// lane % 16) plus a fixed offset per pixel tile.
template <int R, int NKS, int NPT>
__global__ __launch_bounds__(256) void tinyc_mfma_fwd(TFArgs a) {
    constexpr int SW = 2, XWP = kTcXWP;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, kl = lane & 15, g = lane >> 4;
    const int row_beg = blockIdx.x * a.rpw, row_end = min(a.rows, row_beg + a.rpw);
    const rsrc_t rx = make_rsrc(a.X, a.x_bytes);
    const int k = 16 * wave + kl;

    // A: filter value 4t + g of row k, zero past C*R*S
    float wa[NKS];
    {
        const float *W = (const float *)a.Wt;
#pragma unroll
        for (int t = 0; t < NKS; ++t) wa[t] = 4 * t + g < a.CRS ? W[k * a.CRS + 4 * t + g] : 0.f;
    }
    // B of step t: value crs = 4t + g = cr * S + s sits at LDS row cr, column s + 2 * pixel.
    // Walked by additions (S >= 4: one column wrap per step); values past C*R*S read
    // value g, which meets a zero filter value.
    const int s0 = g % a.S;
    const uint32_t off0 = (uint32_t)(((g / a.S) * XWP + s0 + SW * kl) * 4);
    const uint32_t wrap_add = (uint32_t)((XWP - a.S) * 4);

    auto compute_store = [&](int stage, int row) {
        f32x4 acc[NPT];
#pragma unroll
        for (int j = 0; j < NPT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const char *sb = smem + stage * kTcStage;
        uint32_t off = opaque_u32(off0);   // recomputed per row, not kept in registers per step
        int sc = s0;
#pragma unroll
        for (int t = 0; t < NKS; ++t) {
            const uint32_t use = 4 * t + g < a.CRS ? off : off0;
#pragma unroll
            for (int j = 0; j < NPT; ++j) {
                const float b = *(const float *)(sb + use + j * 16 * SW * 4);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[t], b, acc[j], 0, 0, 0);
            }
            sc += 4;
            const bool wrap = sc >= a.S;
            sc = wrap ? sc - a.S : sc;
            off += wrap ? 16u + wrap_add : 16u;
        }
        // D: lane (kl, g) holds k = 16 * wave + 4g + v at pixel 16j + kl
        const int n = row / a.P, p = row - n * a.P;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int ko = 16 * wave + 4 * g + v;
            const float bk = a.has_epi && a.epi.bias ? a.epi.bias[ko] : 0.f;
            const uint32_t orow = (uint32_t)(((n * a.K + ko) * a.P + p) * a.Q);
#pragma unroll
            for (int j = 0; j < NPT; ++j) {
                const int q = 16 * j + kl;
                if (q < a.Q) out_store(a.out, orow + q, acc[j][v], a.epi, a.has_epi, bk);
            }
        }
    };

    tc_stage_x<R>(a, rx, row_beg, smem, tid);
    __syncthreads();
    float xr[4 * R];
    for (int row = row_beg; row < row_end; row += 2) {
        // the next row's input rows are loaded before this row's MFMAs and stored after
        // them (past the last row they re-read the last row, unused)
        tc_load_x<R>(a, rx, min(row + 1, row_end - 1), tid, xr);
        compute_store(0, row);
        tc_store_x<R>(a, xr, smem + kTcStage, tid);
        __syncthreads();
        if (row + 1 >= row_end) break;
        tc_load_x<R>(a, rx, min(row + 2, row_end - 1), tid, xr);
        compute_store(1, row + 1);
        tc_store_x<R>(a, xr, smem, tid);
        __syncthreads();
    }
}

int launch_tinyc_fwd(const Plan &pl, const Problem &p, const void *x, const void *w, float *y, hipStream_t st,
                     const Epi *epi) {
    // the plan checked fp32, K == 64, C <= 4, R == 7, S >= 4, sw == 2, C*R*S <= 148, Q <= 112
    TFArgs a = {};
    if (epi) a.epi = *epi;
    a.has_epi = epi ? 1 : 0;
    a.X = x;
    a.Wt = w;
    a.out = y;
    a.x_bytes = (uint32_t)((size_t)p.N * p.C * p.H * p.W * 4);
    a.C = p.C; a.H = p.H; a.W = p.W; a.K = p.K; a.R = p.R; a.S = p.S;
    a.ph = p.ph; a.pw = p.pw; a.sh = p.sh; a.P = p.P; a.Q = p.Q;
    a.RS = p.R * p.S;
    a.CRS = p.C * a.RS;
    a.rows = p.N * p.P;
    a.rpw = pl.tc_rows;
    const void *k = (const void *)tinyc_mfma_fwd<7, kTcFwdSteps, kTcQT * 4 / 16>;
    hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTcBwdfLds);
    if (e != hipSuccess) return MICONV_ERR_HIP;
    void *args[] = {&a};
    e = hipLaunchKernel(k, dim3((p.N * p.P + a.rpw - 1) / a.rpw), dim3(256), args, kTcBwdfLds, st);
    return e == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
}

template <int ES, int NSM>
static const void *tinyc_kernel(int C) {
    switch (C) {
        case 1: return (const void *)tinyc_bwd_data<ES, 1, NSM>;
        case 2: return (const void *)tinyc_bwd_data<ES, 2, NSM>;
        case 3: return (const void *)tinyc_bwd_data<ES, 3, NSM>;
        default: return (const void *)tinyc_bwd_data<ES, 4, NSM>;
    }
}

template <int ES>
static const void *tinyc_select(int C, int nsmax) {
    if (nsmax <= 4) return tinyc_kernel<ES, 4>(C);
    if (nsmax <= 8) return tinyc_kernel<ES, 8>(C);
    return tinyc_kernel<ES, 16>(C);
}

int launch_tinyc(const Plan &pl, const Problem &p, const void *dy, const void *w, float *dx, hipStream_t st,
                 const Epi *epi) {
    TCArgs a = {};
    if (epi) a.epi = *epi;
    a.has_epi = epi ? 1 : 0;
    if (pl.tc_pairs > 0) {
        // the MFMA form (the plan checked fp32, stride 2, R == 7, C*S <= 32, Q <= 128, K = 32 or 64)
        a.DY = dy;
        a.Wt = w;
        a.DX = dx;
        a.dy_bytes = (uint32_t)((size_t)p.N * p.K * p.P * p.Q * 4);
        a.w_bytes = (uint32_t)((size_t)p.K * p.C * p.R * p.S * 4);
        a.N = p.N; a.C = p.C; a.H = p.H; a.W = p.W; a.K = p.K; a.R = p.R; a.S = p.S;
        a.ph = p.ph; a.pw = p.pw; a.sh = p.sh; a.sw = p.sw; a.P = p.P; a.Q = p.Q;
        a.PB = pl.tc_pairs;
        a.nbands = ((p.H + 1) / 2 + a.PB - 1) / a.PB;
        a.phq = p.ph / 2;
        const size_t lds = tinyc_mfma_lds_bytes(p.R, p.C, p.S);
        const void *k = (p.ph & 1) ? (const void *)tinyc_mfma_bwd_data<7, 1> : (const void *)tinyc_mfma_bwd_data<7, 0>;
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return MICONV_ERR_HIP;
        void *args[] = {&a};
        e = hipLaunchKernel(k, dim3(p.N * a.nbands), dim3(256), args, lds, st);
        return e == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
    }
    const int es = p.dtype ? 2 : 4;
    a.DY = dy;
    a.Wt = w;
    a.DX = dx;
    a.dy_bytes = (uint32_t)((size_t)p.N * p.K * p.P * p.Q * es);
    a.w_bytes = (uint32_t)((size_t)p.K * p.C * p.R * p.S * es);
    a.N = p.N; a.C = p.C; a.H = p.H; a.W = p.W; a.K = p.K; a.R = p.R; a.S = p.S;
    a.ph = p.ph; a.pw = p.pw; a.sh = p.sh; a.sw = p.sw; a.P = p.P; a.Q = p.Q;
    a.DH = (TH - 1 + p.R - 1) / p.sh + 2;
    a.DW = (TW - 1 + p.S - 1) / p.sw + 2;
    a.DWs = a.DW + ((1 - a.DW) % 32 + 32) % 32;
    a.fd_DW = make_fdiv((uint32_t)a.DW);
    a.fd_DHW = make_fdiv((uint32_t)(a.DH * a.DW));
    a.dyw_bytes = (int)(((size_t)KC * a.DH * a.DWs * 4 + 15) / 16 * 16);
    const size_t lds = (size_t)a.dyw_bytes + (size_t)KC * p.R * p.S * 16;
    const int blocks = p.N * ((p.H + TH - 1) / TH) * ((p.W + TW - 1) / TW);
    // taps per column phase, at most ceil(S / sw)
    const int nsmax = (p.S + p.sw - 1) / p.sw;
    const void *k = p.dtype ? tinyc_select<2>(p.C, nsmax) : tinyc_select<4>(p.C, nsmax);
    hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return MICONV_ERR_HIP;
    void *args[] = {&a};
    e = hipLaunchKernel(k, dim3(blocks), dim3(256), args, lds, st);
    return e == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
}

}  // namespace miconv
