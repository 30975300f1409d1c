// patch.hip -- stride-1 convolution with one LDS input patch shared by every
// filter tap (bf16 inputs, fp32 accumulation and output).
//
// Form computed:  O[n,m,p,q] = sum_{t=(r,s), c} Wt[m,t,c] * X~(n, c, p - ph + r, q - pw + s)
//   forward:        X = x,  Wt[k][t][c] = W[k][c][t],                  pads (ph, pw)
//   backward-data:  X = dy, Wt[c][t'][k] = W[k][c][R*S-1-t'] (rotated), pads (R-1-ph, S-1-pw)
// (with stride 1 the adjoint in x is a correlation of dy with the filter
// rotated by 180 degrees and its K and C roles exchanged).
//
// Work-group tile: BM output channels x TR whole output rows of one image.
// Per 32-channel chunk the input rows the tile needs (TR + R - 1 of them,
// padded to Wo + S - 1 columns) are loaded once with 16/8/4-byte row loads,
// transposed 8x8 in registers into a channel-contiguous patch
// [row][col][32 channels] and reused by all R*S taps: the MFMA B fragment of
// a pixel at tap (r, s) is 16 contiguous bytes at patch position
// (row + r, col + s).  Padding rows come from out-of-range buffer loads
// (zero), padding columns are zeroed once and never written.  Two patch
// buffers: the next chunk is loaded and stored while the current one is in
// use, so there is one barrier per chunk and none per tap.
// Each wave owns distinct filter rows, so its filter fragments are loaded
// straight from global memory (L2) into registers in MFMA layout, two steps
// ahead; B fragments of the next tap are read while this tap's MFMAs run.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace miconv {

namespace {

constexpr int CK = 32;    // channels per chunk = one MFMA reduction step per tap
constexpr int CPB = 80;   // bytes per patch position and per filter row: 64 data + 16 pad
constexpr int MAXI = 2;   // patch-fill items per thread (host guarantees 4*PR*G <= 512)

// One fill item: 8 channels x VW columns of one input row.
template <int VW>
struct FillItem {
    uint32_t d[8][VW / 2 > 0 ? VW / 2 : 1];
};

// Item `it` of a patch of channel octets: octet o, patch row pr, column group g.
// Items are fixed per thread, so they are decoded once per work-group.
struct ItemPos {
    int g, pr, o;
    bool ok;  // it < number of items
};

DEVI ItemPos item_pos(int it, int nitems, int G, int PR) {
    ItemPos q;
    q.ok = it < nitems;
    const int itq = q.ok ? it : 0;
    q.g = itq % G;
    const int rest = itq / G;
    q.pr = rest % PR;
    q.o = rest / PR;
    return q;
}

// X is [N][Cx][Hi][Wi]; patch row pr holds input row p0 - ph + pr.
template <int VW>
DEVI void fill_load(rsrc_t rx, const ItemPos &q, int Cx, int Hi, int Wi, int ph, int n, int p0, int c0,
                    FillItem<VW> &f) {
    const int ih = p0 - ph + q.pr;
    const bool ok = q.ok && (unsigned)ih < (unsigned)Hi;
    const uint32_t plane = (uint32_t)Hi * Wi * 2;
    const uint32_t base = ok ? (uint32_t)((((n * Cx + c0 + q.o * 8) * Hi + ih) * Wi + q.g * VW) * 2) : kOOB;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t off = base + (uint32_t)j * plane;
        if constexpr (VW == 8) {
            const u32x4 v = ld_vec(rx, off);
            f.d[j][0] = v[0]; f.d[j][1] = v[1]; f.d[j][2] = v[2]; f.d[j][3] = v[3];
        } else if constexpr (VW == 4) {
            const u32x2 v = ld_b64(rx, off);
            f.d[j][0] = v[0]; f.d[j][1] = v[1];
        } else {
            f.d[j][0] = ld_elem<4>(rx, off);
        }
    }
}

// Transposes 8 channels x VW columns into VW 16-byte channel vectors and stores
// them at patch[pr][pw + g*VW + i][o*8 .. o*8+7] (CPB bytes per position).
template <int VW, int CPB>
DEVI void fill_store(char *patch, const ItemPos &q, int PWs, int pw, const FillItem<VW> &f) {
    if (!q.ok) return;
    char *dst = patch + ((q.pr * PWs + pw + q.g * VW) * CPB + q.o * 16);
#pragma unroll
    for (int i = 0; i < VW; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_amdgcn_perm(f.d[2 * e + 1][i >> 1], f.d[2 * e][i >> 1], sel);
        *(u32x4 *)(dst + i * CPB) = v;
    }
}

}  // namespace

template <int BM, int WM, int WN, int NBW, int VW>
__global__ __launch_bounds__(256, 2) void patch_kernel(PatchArgs a) {
    constexpr int WTM = BM / WM, TMB = WTM / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, lh = lane >> 5;
    const int wm = wave % WM, wn = wave / WM;

    // filter-row tile outermost: the work-groups an XCD runs together share one
    // filter slice in that XCD's L2
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int per_m = a.row_tiles * a.N;
    const int mt = logical / per_m, rest = logical - mt * per_m;
    const int rt = rest % a.row_tiles, n = rest / a.row_tiles;
    const int m0 = mt * BM, p0 = rt * a.TR;
    const int rows_here = min(a.TR, a.Ho - p0);
    const int npx = rows_here * a.Wo;
    const int T = a.R * a.S;
    const int nchunks = a.Cr / CK, nsteps = nchunks * T;
    const int patch_bytes = a.PR * a.PWs * CPB;

    const rsrc_t rx = make_rsrc(a.X, a.x_bytes), rw = make_rsrc(a.Wt, a.w_bytes);

    // two patch buffers; zero both once: the padding columns are never written again
    for (int o = tid * 16; o < 2 * patch_bytes; o += 256 * 16) *(u32x4 *)(smem + o) = u32x4{0, 0, 0, 0};

    // this lane's pixel of each of the wave's pixel blocks (invalid pixels read
    // position 0; their results are never stored)
    int pbase[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int idx = (wn + WN * j) * 32 + lr;
        const int pr = idx / a.Wo, pc = idx - pr * a.Wo;
        pbase[j] = (idx < npx ? (pr * a.PWs + pc) * CPB : 0) + lh * 16;
    }

    // filter fragments straight from global memory in MFMA layout: row
    // (m0 + wm*WTM + i*32 + lr), 8 channels at (chunk*32 + u*16 + lh*8) of tap t
    uint32_t arow[TMB];
#pragma unroll
    for (int i = 0; i < TMB; ++i) {
        const int m = m0 + wm * WTM + i * 32 + lr;
        arow[i] = m < a.M ? (uint32_t)(m * T * a.Cr + lh * 8) * 2 : kOOB;
    }
    u32x4 af[2][TMB][2];
    // Step state, advanced incrementally (no divisions in the loop): chunk ci,
    // tap t = (r, s), the filter byte offset (t*Cr + ci*32)*2 and the patch
    // byte offset of the tap in chunk ci's buffer.
    struct StepPos {
        int ci, t, r, s, aoff, boff;
    };
    auto advance = [&](StepPos q) {
        if (++q.t == T) {
            q.t = 0;
            q.r = 0;
            q.s = 0;
            ++q.ci;
        } else if (++q.s == a.S) {
            q.s = 0;
            ++q.r;
        }
        q.aoff = (q.t * a.Cr + q.ci * CK) * 2;
        q.boff = (q.ci & 1) * patch_bytes + (q.r * a.PWs + q.s) * CPB;
        return q;
    };
    auto load_a = [&](const StepPos &q, u32x4 (&dst)[TMB][2]) {
#pragma unroll
        for (int i = 0; i < TMB; ++i)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                dst[i][u] = ld_vec(rw, arow[i] == kOOB ? kOOB : arow[i] + (uint32_t)q.aoff + u * 32);
    };

    const int nitems = 4 * a.PR * a.G;
    ItemPos items[MAXI];
#pragma unroll
    for (int k = 0; k < MAXI; ++k) items[k] = item_pos(tid + k * 256, nitems, a.G, a.PR);
    FillItem<VW> fi;   // one fill item in flight per thread
    auto load_item = [&](int ci, int k) {
        fill_load<VW>(rx, items[k], a.Cr, a.Hi, a.Wi, a.ph, n, p0, ci * CK, fi);
    };
    auto store_item = [&](int buf, int k) {
        fill_store<VW, CPB>(smem + buf * patch_bytes, items[k], a.PWs, a.pw, fi);
    };
    f32x16 acc[TMB][NBW];
#pragma unroll
    for (int i = 0; i < TMB; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // B fragments of one k16 half of a step: 32 pixels x 8 channels per block
    u32x4 fb[2][NBW];
    auto load_b = [&](const StepPos &q, int u, u32x4 (&dst)[NBW]) {
        const char *B = smem + q.boff + u * 32;
#pragma unroll
        for (int j = 0; j < NBW; ++j) dst[j] = *(const u32x4 *)(B + pbase[j]);
    };
    auto mfma_half = [&](const u32x4 (&A)[TMB][2], int u, const u32x4 (&B)[NBW]) {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int i = 0; i < TMB; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, A[i][u]), __builtin_bit_cast(bf16x8, B[j]), acc[i][j], 0, 0, 0);
    };

    StepPos cur = {0, 0, 0, 0, 0, 0};
    load_a(cur, af[0]);
    __syncthreads();  // zeroing done before the fill overwrites data columns
#pragma unroll
    for (int k = 0; k < MAXI; ++k) {
        load_item(0, k);
        store_item(0, k);
    }
    __syncthreads();
    load_b(cur, 0, fb[0]);

    // One step = one (chunk, tap) pair, two k16 halves.  While the MFMAs of one
    // half run, the B fragments of the following half are read.  CUR selects the
    // register set of this step's filter fragments; the loop is unrolled by two
    // so that every register array index is a compile-time constant.
    auto body = [&](auto cur_c, int step) {
        constexpr int CUR = decltype(cur_c)::value;
        const bool more = step + 1 < nsteps;
        const StepPos nxt = more ? advance(cur) : cur;
        // the next chunk's patch, one fill item per step (steps 0 .. MAXI-1 of this
        // chunk): global loads now, LDS store after this step's MFMAs
        const bool refill = cur.t < MAXI && cur.ci + 1 < nchunks;
        const bool chunk_end = cur.t == T - 1;
        load_b(cur, 1, fb[1]);
        mfma_half(af[CUR], 0, fb[0]);
        // Global loads are issued only after the first half's MFMAs (which wait
        // for this step's filter fragments): in-order load counters would
        // otherwise make that wait cover these newer loads as well.
        __builtin_amdgcn_sched_barrier(0);
        load_a(nxt, af[CUR ^ 1]);
        if (refill) load_item(cur.ci + 1, cur.t == 0 ? 0 : 1);
        // unconditional (the count of outstanding LDS reads stays static); at a
        // chunk end these are re-read from the new patch after the barrier
        load_b(nxt, 0, fb[0]);
        mfma_half(af[CUR], 1, fb[1]);
        if (refill) store_item((cur.ci + 1) & 1, cur.t == 0 ? 0 : 1);  // that buffer was last read in chunk ci - 1
        if (chunk_end && T < MAXI && cur.ci + 1 < nchunks) {
#pragma unroll
            for (int k = 1; k < MAXI; ++k) {  // filters with fewer taps than fill items
                if (k < T) continue;
                load_item(cur.ci + 1, k);
                store_item((cur.ci + 1) & 1, k);
            }
        }
        if (chunk_end && more) {
            __syncthreads();  // next chunk's patch complete; every wave is done with this one
            load_b(nxt, 0, fb[0]);
        }
        cur = nxt;
    };
    for (int step = 0; step < nsteps; step += 2) {
        body(std::integral_constant<int, 0>(), step);
        if (step + 1 < nsteps) body(std::integral_constant<int, 1>(), step + 1);
    }

    // epilogue: fp32 stores, 32 consecutive pixels per accumulator register
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int idx = (wn + WN * j) * 32 + lr;
        if (idx >= npx) continue;
        const int pr = idx / a.Wo, pc = idx - pr * a.Wo;
        float *o = a.O + ((size_t)n * a.M * a.Ho + p0 + pr) * a.Wo + pc;
#pragma unroll
        for (int i = 0; i < TMB; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * WTM + i * 32 + acc_row(v, lh);
                if (m < a.M) o[(size_t)m * a.Ho * a.Wo] = acc[i][j][v];
            }
    }
}

// Rotated, transposed filter for stride-1 backward-data: wt[c][t'][k] = w[k][c][T-1-t'].
__global__ __launch_bounds__(256) void filter_to_ctk_rot(const uint16_t *__restrict__ w, uint16_t *__restrict__ wt,
                                                         int K, int C, int T) {
    const long long total = (long long)K * C * T;
    for (long long e = blockIdx.x * 256LL + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
        const int c = (int)(e / ((long long)T * K));
        const int rem = (int)(e - (long long)c * T * K), tt = rem / K, k = rem - tt * K;
        wt[e] = w[((long long)k * C + c) * T + (T - 1 - tt)];
    }
}

// Launch of one patch configuration; returns a hipError_t.
template <int BM, int WM, int WN, int NBW, int VW>
static hipError_t patch_go(const PatchArgs &a, int grid, size_t lds, hipStream_t st) {
    auto k = patch_kernel<BM, WM, WN, NBW, VW>;
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int BM, int WM, int WN, int NBW>
static hipError_t patch_vw(const PatchArgs &a, int vw, int grid, size_t lds, hipStream_t st) {
    if (vw == 8) return patch_go<BM, WM, WN, NBW, 8>(a, grid, lds, st);
    if (vw == 4) return patch_go<BM, WM, WN, NBW, 4>(a, grid, lds, st);
    return patch_go<BM, WM, WN, NBW, 2>(a, grid, lds, st);
}

int launch_patch(const Plan &pl, const Problem &p, const void *in0, const void *in1, float *out, void *ws,
                 hipStream_t st) {
    const int T = p.R * p.S;
    PatchArgs a = {};
    uint16_t *wt = (uint16_t *)((char *)ws + pl.wt_offset);
    const long long kcrs = (long long)p.K * p.C * T;
    const int blocks = (int)((kcrs + 255) / 256 < 4096 ? (kcrs + 255) / 256 : 4096);
    if (p.pass == FWD) {
        hipLaunchKernelGGL(filter_to_ktc<uint16_t>, dim3(blocks), dim3(256), 0, st, (const uint16_t *)in1, wt, p.K,
                           p.C, T);
        a.X = in0;
        a.x_bytes = (uint32_t)((size_t)p.N * p.C * p.H * p.W * 2);
        a.Cr = p.C; a.Hi = p.H; a.Wi = p.W; a.M = p.K;
        a.ph = p.ph; a.pw = p.pw; a.Ho = p.P; a.Wo = p.Q;
    } else {
        hipLaunchKernelGGL(filter_to_ctk_rot, dim3(blocks), dim3(256), 0, st, (const uint16_t *)in1, wt, p.K, p.C,
                           T);
        a.X = in0;
        a.x_bytes = (uint32_t)((size_t)p.N * p.K * p.P * p.Q * 2);
        a.Cr = p.K; a.Hi = p.P; a.Wi = p.Q; a.M = p.C;
        a.ph = p.R - 1 - p.ph; a.pw = p.S - 1 - p.pw; a.Ho = p.H; a.Wo = p.W;
    }
    if (hipGetLastError() != hipSuccess) return MICONV_ERR_HIP;
    a.Wt = wt;
    a.w_bytes = (uint32_t)(kcrs * 2);
    a.O = out;
    a.N = p.N; a.R = p.R; a.S = p.S;
    a.TR = pl.tr;
    a.row_tiles = (a.Ho + a.TR - 1) / a.TR;
    a.m_tiles = pl.m_tiles;
    a.PWc = a.Wo + p.S - 1;
    a.PWs = pl.pws;
    a.PR = a.TR + p.R - 1;
    a.G = a.Wi / pl.vw;
    const int grid = pl.m_tiles * a.row_tiles * p.N;
    const size_t lds = 2 * (size_t)a.PR * a.PWs * CPB;
    hipError_t e;
    if (pl.bm == 64)
        e = patch_vw<64, 2, 2, 7>(a, pl.vw, grid, lds, st);
    else
        e = patch_vw<128, 4, 1, 7>(a, pl.vw, grid, lds, st);
    return e == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
}

// ------------------------------------------------------------------ backward-filter
// dW[k,c,t] = sum over output pixels of dy[n,k,p,q] * x~(n, c, p - ph + r, q - pw + s), stride 1.
// Work-group tile: BM filter rows (k) x 32 channels x all R*S (<= 9) taps, over a
// contiguous range of bands (TR whole output rows of one image) -- one split of
// the pixel reduction.  Per band, the x patch [row][col][32 channels] is filled
// once (16/8/4-byte row loads, 8x8 register transposes) and serves every tap;
// two patch buffers, so the next band is filled while this one is in use and
// there is one barrier per band.  Each wave loads its dy rows straight from
// global memory in MFMA layout (8 consecutive pixels per lane), one step ahead.
// The MFMA B fragment (4 consecutive pixels of one channel per lane and read)
// comes from ds_read_b64_tr_b16 on the channel-contiguous patch, so any tap
// shift is a plain address offset.  Positions are 64 bytes apart: the four
// positions one 32-lane read touches cover all 64 banks once; the row stride
// is congruent to Q (mod 4) so row wraps keep that property.
// Each wave owns one 32-row block x all taps (9 accumulators); with BM = 64 the
// two k16 halves of every 32-pixel step go to different waves, whose sums are
// added through LDS at the end.
template <int BM, int VW, int AV>
__global__ __launch_bounds__(256, 2) void bwdf_patch_kernel(BFArgs a) {
    constexpr int BC = 32, CPBF = 64, NOCT = 4, TMAX = 9;
    constexpr int WM = BM / 32, WU = 4 / WM, NU = 2 / WU;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, lh = lane >> 5;
    const int wm = wave % WM, wu = wave / WM;
    const int grp = lane >> 4, L = lane & 15;

    const int tiles = a.m_tiles * a.c_tiles;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int z = logical / tiles, tile = logical - z * tiles;
    const int m0 = (tile % a.m_tiles) * BM, c0 = (tile / a.m_tiles) * BC;
    const int total_bands = a.N * a.row_bands;
    const int b_begin = z * a.bands_per_split, b_end = min(total_bands, b_begin + a.bands_per_split);
    const int T = a.R * a.S;
    const int patch_bytes = a.PR * a.PWs * CPBF;
    const rsrc_t rx = make_rsrc(a.X, a.x_bytes), rdy = make_rsrc(a.DY, a.dy_bytes);

    for (int o = tid * 16; o < 2 * patch_bytes; o += 256 * 16) *(u32x4 *)(smem + o) = u32x4{0, 0, 0, 0};

    auto band_geom = [&](int b, int &n, int &p0, int &npx) {
        n = b / a.row_bands;
        p0 = (b - n * a.row_bands) * a.TR;
        npx = min(a.TR, a.P - p0) * a.Q;
    };

    const int nitems = NOCT * a.PR * a.G;
    ItemPos items[MAXI];
#pragma unroll
    for (int k = 0; k < MAXI; ++k) items[k] = item_pos(tid + k * 256, nitems, a.G, a.PR);
    FillItem<VW> fi;  // one fill item in flight per thread
    auto load_item = [&](int b, int k) {
        int n, p0, npx;
        band_geom(b, n, p0, npx);
        fill_load<VW>(rx, k == 0 ? items[0] : items[1], a.C, a.H, a.W, a.ph, n, p0, c0, fi);
    };
    auto store_item = [&](int buf, int k) {
        fill_store<VW, CPBF>(smem + buf * patch_bytes, k == 0 ? items[0] : items[1], a.PWs, a.pw, fi);
    };

    // dy fragments: row (m0 + wm*32 + lr), 8 pixels at ps*32 + u*16 + lh*8 of band b
    const int krow = m0 + wm * 32 + lr;
    u32x4 af[2][NU];
    auto load_a = [&](int b, int ps, u32x4 (&dst)[NU]) {
        int n, p0, npx;
        band_geom(b, n, p0, npx);
        const uint32_t rowoff = (uint32_t)(((n * a.K + krow) * a.P + p0) * a.Q);
        const bool kok = krow < a.K;
#pragma unroll
        for (int uu = 0; uu < NU; ++uu) {
            const int u = WU == 2 ? wu : uu;
            const int px = ps * 32 + u * 16 + lh * 8;
            if constexpr (AV == 8) {
                dst[uu] = ld_vec(rdy, kok && px < npx ? (rowoff + px) * 2 : kOOB);
            } else if constexpr (AV == 4) {
                const u32x2 lo = ld_b64(rdy, kok && px < npx ? (rowoff + px) * 2 : kOOB);
                const u32x2 hi = ld_b64(rdy, kok && px + 4 < npx ? (rowoff + px + 4) * 2 : kOOB);
                dst[uu] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            } else {
                uint32_t e[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    e[j] = ld_elem<2>(rdy, kok && px + j < npx ? (rowoff + px + j) * 2 : kOOB);
                dst[uu] = pack<2>(e);
            }
        }
    };

    f32x16 acc[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;

    // channel byte offset this lane's transpose reads start at (groups 0/1 and
    // 2/3 read channels 0-15 / 16-31, four channels per lane)
    const int choff = 32 * (grp & 1) + 8 * (L & 3);
    // patch byte offset of each tap, computed once (no divisions in the loop)
    int toffs[TMAX];
    {
        int r = 0, s = 0;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            toffs[t] = (r * a.PWs + s) * CPBF;
            if (++s == a.S) {
                s = 0;
                ++r;
            }
        }
    }

    auto mfma_step = [&](const char *patch, int ps, int npx, const u32x4 (&A)[NU]) {
#pragma unroll
        for (int uu = 0; uu < NU; ++uu) {
            const int u = WU == 2 ? wu : uu;
            int pos[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ip = ps * 32 + u * 16 + 8 * lh + 4 * h + (L >> 2);
                const int pr = (int)fdiv((uint32_t)ip, a.fd_Q), pc = ip - pr * a.Q;
                pos[h] = (ip < npx ? (pr * a.PWs + pc) * CPBF : 0) + choff;
            }
#pragma unroll
            for (int t = 0; t < TMAX; ++t) {
                if (t < T) {  // predicated, not `break`: keeps acc[] indices compile-time
                    const int toff = toffs[t];
                    typedef short i16x4 __attribute__((ext_vector_type(4)));
                    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(__attribute__((address_space(3))) char *)(patch + pos[0] + toff));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(__attribute__((address_space(3))) char *)(patch + pos[1] + toff));
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                    const u32x4 fb = u32x4{l2[0], l2[1], h2[0], h2[1]};
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, A[uu]), __builtin_bit_cast(bf16x8, fb), acc[t], 0, 0, 0);
                }
            }
        }
    };

    if (b_begin < b_end) {
        load_a(b_begin, 0, af[0]);
        __syncthreads();  // zeroing done before the fill overwrites data columns
#pragma unroll
        for (int k = 0; k < MAXI; ++k) {
            load_item(b_begin, k);
            store_item(0, k);
        }
        __syncthreads();
    }
    // steps run over (band, pixel step); CUR selects this step's dy registers and
    // the loop is unrolled by two so register array indices are compile-time
    int b = b_begin, ps = 0, n = 0, p0 = 0, npx = 0;
    if (b < b_end) band_geom(b, n, p0, npx);
    auto body = [&](auto cur_c) {
        constexpr int CUR = decltype(cur_c)::value;
        const int nps = (npx + 31) / 32;
        const bool last = ps + 1 == nps;
        const int nb = last ? b + 1 : b, nps_next = last ? 0 : ps + 1;
        const int bi = (b - b_begin) & 1;
        // the next band's patch, one fill item per step (its first MAXI steps)
        const bool refill = ps < MAXI && b + 1 < b_end;
        mfma_step(smem + bi * patch_bytes, ps, npx, af[CUR]);
        __builtin_amdgcn_sched_barrier(0);
        if (nb < b_end) load_a(nb, nps_next, af[CUR ^ 1]);
        if (refill) {
            load_item(b + 1, ps == 0 ? 0 : 1);
            store_item(bi ^ 1, ps == 0 ? 0 : 1);  // that buffer was last read in band b - 1
        }
        if (last) {
            if (nps < MAXI && b + 1 < b_end) {
#pragma unroll
                for (int k = 1; k < MAXI; ++k) {  // bands with fewer steps than fill items
                    if (k < nps) continue;
                    load_item(b + 1, k);
                    store_item(bi ^ 1, k);
                }
            }
            __syncthreads();  // next band's patch complete; every wave is done with this one
            b = nb;
            ps = 0;
            if (b < b_end) band_geom(b, n, p0, npx);
        } else {
            ++ps;
        }
    };
    while (b < b_end) {
        body(std::integral_constant<int, 0>());
        if (b < b_end) body(std::integral_constant<int, 1>());
    }

    // two waves per row block: the second adds its sums to the first through LDS
    if (WU == 2) {
        float *red = (float *)smem;  // WM waves x 16 floats x 64 lanes per tap
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t >= T) continue;
            __syncthreads();
            if (wu == 1)
#pragma unroll
                for (int v = 0; v < 16; ++v) red[(wm * 16 + v) * 64 + lane] = acc[t][v];
            __syncthreads();
            if (wu == 0)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[t][v] += red[(wm * 16 + v) * 64 + lane];
        }
    }

    // epilogue: partial sums [z][K][T][C] (or dW [K][C][T] with a single split)
    if (WU == 2 && wu != 0) return;
    const int c = c0 + lr;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t >= T) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int k = m0 + wm * 32 + acc_row(v, lh);
            if (k >= a.K) continue;
            if (a.direct)
                a.out[((size_t)k * a.C + c) * T + t] = acc[t][v];
            else
                a.out[(((size_t)z * a.K + k) * T + t) * a.C + c] = acc[t][v];
        }
    }
}

template <int BM, int VW, int AV>
static hipError_t bwdf_go(const BFArgs &a, int grid, size_t lds, hipStream_t st) {
    auto k = bwdf_patch_kernel<BM, VW, AV>;
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int BM>
static hipError_t bwdf_vw(const BFArgs &a, int vw, int av, int grid, size_t lds, hipStream_t st) {
    if (vw == 8) {
        if (av == 8) return bwdf_go<BM, 8, 8>(a, grid, lds, st);
        if (av == 4) return bwdf_go<BM, 8, 4>(a, grid, lds, st);
        return bwdf_go<BM, 8, 1>(a, grid, lds, st);
    }
    if (vw == 4) {
        if (av == 8) return bwdf_go<BM, 4, 8>(a, grid, lds, st);
        if (av == 4) return bwdf_go<BM, 4, 4>(a, grid, lds, st);
        return bwdf_go<BM, 4, 1>(a, grid, lds, st);
    }
    if (av == 8) return bwdf_go<BM, 2, 8>(a, grid, lds, st);
    if (av == 4) return bwdf_go<BM, 2, 4>(a, grid, lds, st);
    return bwdf_go<BM, 2, 1>(a, grid, lds, st);
}

int launch_bwdf_patch(const Plan &pl, const Problem &p, const void *x, const void *dy, float *dw, void *ws,
                      hipStream_t st) {
    BFArgs a = {};
    a.X = x;
    a.DY = dy;
    a.x_bytes = (uint32_t)((size_t)p.N * p.C * p.H * p.W * 2);
    a.dy_bytes = (uint32_t)((size_t)p.N * p.K * p.P * p.Q * 2);
    a.N = p.N; a.C = p.C; a.H = p.H; a.W = p.W; a.K = p.K; a.R = p.R; a.S = p.S;
    a.ph = p.ph; a.pw = p.pw; a.P = p.P; a.Q = p.Q;
    a.TR = pl.tr;
    a.row_bands = (p.P + pl.tr - 1) / pl.tr;
    a.m_tiles = pl.m_tiles;
    a.c_tiles = pl.n_tiles;
    a.splits = pl.splits;
    a.bands_per_split = pl.chunk;
    a.PWc = p.Q + p.S - 1;
    a.PWs = pl.pws;
    a.PR = pl.tr + p.R - 1;
    a.G = p.W / pl.vw;
    a.direct = pl.splits == 1;
    a.fd_Q = make_fdiv((uint32_t)p.Q);
    float *part = pl.splits > 1 ? (float *)((char *)ws + pl.part_offset) : dw;
    a.out = part;
    size_t lds = 2 * (size_t)a.PR * a.PWs * 64;                         // two patch buffers
    if (lds < (size_t)2 * 16 * 64 * 4) lds = (size_t)2 * 16 * 64 * 4;  // epilogue reduction buffer
    const int grid = pl.m_tiles * pl.n_tiles * pl.splits;
    const int av = (p.P * p.Q) % 8 == 0 && (pl.tr * p.Q) % 8 == 0 ? 8 : ((p.P * p.Q) % 4 == 0 && (pl.tr * p.Q) % 4 == 0 ? 4 : 1);
    hipError_t e = pl.bm == 64 ? bwdf_vw<64>(a, pl.vw, av, grid, lds, st) : bwdf_vw<128>(a, pl.vw, av, grid, lds, st);
    if (e != hipSuccess) return MICONV_ERR_HIP;
    if (pl.splits > 1) return launch_splitk_reduce(part, dw, p.K, p.C, p.R * p.S, pl.splits, st);
    return MICONV_OK;
}

}  // namespace miconv
