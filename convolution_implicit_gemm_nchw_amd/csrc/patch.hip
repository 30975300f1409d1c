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
#include <mutex>
#include <type_traits>

#include "device.h"
#include "launch.h"
#include "patch_common.h"

namespace miconv {



// Persistent: the grid holds as many work-groups as are resident at once and
// each walks the tiles first, first + grid, ...  The chunk pipeline runs on
// across tile boundaries: during the last chunk of a tile the first chunk of
// the next tile is filled, and the finished tile's fp32 stores drain while the
// next tile's MFMAs run.
// v[ph] for a work-group-uniform phase index, by selects on the kernel arguments (a
// dynamic index into an argument array would move the arguments to private memory).
DEVI int phase_sel(const int (&v)[4], int ph) {
    return ph == 0 ? v[0] : (ph == 1 ? v[1] : (ph == 2 ? v[2] : v[3]));
}

// Fused-epilogue store of one 32x32 accumulator block (bits, the lane's 16
// values): value v sits in block row r = row0 + (v >> 2) * 8 + (v & 3), whose
// output row is r + 4*lh (folded into pix, as in the caller).  Rows >= M and
// pixels outside the tile are outside `ro`'s range (loads give 0, stores are
// dropped); the bias comes from the LDS copy `bs` at row mbase + r (clamped to
// M - 1).  Done in two halves of 8 values, each half's previous outputs loaded
// (when beta != 0) before any of its stores, so only 8 old values are live.
template <int EPI>
DEVI void store_block_epi(const PatchArgs &a, rsrc_t ro, uint32_t pix, const u32x16 &bits, int row0, int HoWo,
                          const float *bs, int mbase) {
    constexpr int OES = EPI == 2 ? 2 : 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float old[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int v = 8 * h + u, mrow = row0 + (v >> 2) * 8 + (v & 3);
            const int off = (int)(pix + (uint32_t)(mrow * HoWo * OES));
            if constexpr (EPI == 2)
                old[u] = a.epi.beta != 0.0f ? bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(ro, off, 0, 0)) : 0.0f;
            else
                old[u] = a.epi.beta != 0.0f
                             ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, off, 0, 0))
                             : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int v = 8 * h + u, mrow = row0 + (v >> 2) * 8 + (v & 3);
            const int off = (int)(pix + (uint32_t)(mrow * HoWo * OES));
            const float val = epi_apply(a.epi, __uint_as_float(bits[v]), bs[min(mbase + mrow, a.M - 1)], old[u]);
            if constexpr (EPI == 2)
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(val), ro, off, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ro, off, 0, 0);
        }
    }
}

template <int BM, int WM, int WN, int NBW, int VW, int OCC, int EPI>
__global__ __launch_bounds__(256, OCC) void patch_kernel(PatchArgs a) {
    constexpr int WTM = BM / WM, TMB = WTM / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, lh = lane >> 5;
    const int wm = wave % WM, wn = wave / WM;
    const int T = a.R * a.S;
    const int nchunks = a.Cr / CK;
    const int patch_bytes = a.PR * a.PWs * CPB;
    const int HoWo = a.Ho * a.Wo;

    // filter-row tile outermost; in every round the work-groups of one XCD take
    // one contiguous range of tiles (shared filter rows and halo rows in its L2)
    const int per_m = a.row_tiles * a.N, ntiles = a.m_tiles * per_m;
    const int G = gridDim.x;
    const int first = xcd_remap(blockIdx.x, G);
    const int mine = (ntiles - 1 - first) / G + 1;   // the host launches at most ntiles work-groups
    auto tile_at = [&](int k) __attribute__((always_inline)) {
        Tile tl;
        const int L = first + k * G;
        const int mt = L / per_m, rest = L - mt * per_m;
        const int n = rest / a.row_tiles, rt = rest - n * a.row_tiles;
        // work-group-uniform values (scalar registers; the store resource below
        // must not look divergent)
        tl.n = uniform(n);
        tl.p0 = uniform(rt * a.TR);
        tl.m0 = uniform(mt * BM);
        tl.npx = uniform(min(a.TR, a.Ho - rt * a.TR) * a.Wo);
        return tl;
    };

    // buffer resources are rebuilt from the (scalar) kernel arguments at each use

    // two patch buffers; zero both once: the padding columns are never written again
    for (int o = tid * 16; o < 2 * patch_bytes; o += 256 * 16) *(u32x4 *)(smem + o) = u32x4{0, 0, 0, 0};
    if constexpr (EPI) {   // the bias of every filter row, after the two patch buffers
        float *bs = (float *)(smem + 2 * patch_bytes);
        for (int m = tid; m < a.M; m += 256) bs[m] = a.epi.bias ? a.epi.bias[m] : 0.0f;
    }

    // this lane's pixel of each of the wave's pixel blocks; pixels past the end of
    // a short band read patch rows that hold zeros or halo and are never stored
    int pbase[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int idx = (wn + WN * j) * 32 + lr;
        const int pr = idx / a.Wo, pc = idx - pr * a.Wo;
        pbase[j] = (idx < a.TR * a.Wo ? (pr * a.PWs + pc) * CPB : 0) + lh * 16;
    }

    // Filter fragments straight from global memory.  The filter copy is in MFMA
    // fragment order: 1 KB per (32-row block, chunk, tap, k16 half), lane l's
    // 16 bytes at l*16 (row 32*block + l%32, channels chunk*32 + half*16 +
    // (l/32)*8 .. +7), rows padded with zeros to whole tiles: one fully
    // coalesced 1 KB load per fragment, its offset uniform but for l*16.
    const uint32_t frag_stride = (uint32_t)T * nchunks * 2048;   // bytes per 32-row block
    const uint32_t alane = (uint32_t)lane * 16 + (uint32_t)(wm * TMB) * frag_stride;
    u32x4 af[2][TMB][2];
    // Step state, advanced incrementally (no divisions in the loop): chunk ci,
    // tap t = (r, s), patch buffer par, the tile's first filter row m0, the
    // filter byte offset ((m0*T + t)*Cr + ci*32)*2 and the patch byte offset of
    // the tap in buffer par.
    struct StepPos {
        int ci, t, r, s, par, m0;
        uint32_t aoff;   // fragment offset of (m0/32, t, ci)
        int boff;
    };
    auto advance = [&](StepPos q, int next_m0) __attribute__((always_inline)) {
        if (++q.t == T) {
            q.t = 0;
            q.r = 0;
            q.s = 0;
            q.par ^= 1;
            if (++q.ci == nchunks) {
                q.ci = 0;
                q.m0 = next_m0;
            }
        } else if (++q.s == a.S) {
            q.s = 0;
            ++q.r;
        }
        q.aoff = (uint32_t)(q.m0 / 32) * frag_stride + (uint32_t)(q.ci * T + q.t) * 2048;
        q.boff = q.par * patch_bytes + (q.r * a.PWs + q.s) * CPB;
        return q;
    };
    auto load_a = [&](const StepPos &q, u32x4 (&dst)[TMB][2]) {
#pragma unroll
        for (int i = 0; i < TMB; ++i)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                dst[i][u] = ld_vec_s(make_rsrc(a.Wt, a.w_bytes), alane, q.aoff + i * frag_stride + u * 1024);
    };

    const int nitems = 4 * a.PR * a.G;
    ItemPos items[MAXI];
#pragma unroll
    for (int k = 0; k < MAXI; ++k) items[k] = item_pos(tid + k * 256, nitems, a.G, a.PR);
    FillItem<VW> fi;   // one fill item in flight per thread
    auto load_item = [&](int n, int p0, int ci, int k) __attribute__((always_inline)) {
        fill_load<VW>(make_rsrc(a.X, a.x_bytes), items[k], a.Cr, a.Hi, a.Wi, a.ph, n, p0, ci * CK, fi);
    };
    auto store_item = [&](int buf, int k) __attribute__((always_inline)) {
        fill_store<VW, CPB>(smem + buf * patch_bytes, items[k], a.PWs, a.pw, fi);
    };
    f32x16 acc[TMB][NBW];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TMB; ++i)
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    };
    zero_acc();

    // fp32 stores of a finished tile: register v of block (i, j) holds filter row
    // m0 + wm*WTM + i*32 + acc_row(v, lh) at pixel idx of the tile (the tile's
    // pixels are contiguous in the output plane).  Rows >= M and pixels >= npx
    // get an out-of-range offset and are dropped.
    auto store_tile = [&](const Tile &tl) __attribute__((always_inline)) {
        const size_t base = ((size_t)tl.n * a.M + tl.m0) * HoWo + (size_t)tl.p0 * a.Wo;
        constexpr int OES = EPI == 2 ? 2 : 4;   // output element bytes
        const long long room = (long long)(a.M - tl.m0) * HoWo * OES;
        const rsrc_t ro = make_rsrc((char *)a.O + base * OES, (uint32_t)(room < 0x7fffffffLL ? room : 0x7fffffffLL));
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int idx = (wn + WN * j) * 32 + lr;
            const uint32_t pix = idx < tl.npx ? (uint32_t)((lh * 4 * HoWo + idx) * OES) : kOOB;
#pragma unroll
            for (int i = 0; i < TMB; ++i) {
                // cast the whole vector: a bit_cast of one subscripted element is
                // lowered to element 0
                const u32x16 bits = __builtin_bit_cast(u32x16, acc[i][j]);
                if constexpr (EPI) {
                    store_block_epi<EPI>(a, ro, pix, bits, wm * WTM + i * 32, HoWo,
                                         (const float *)(smem + 2 * patch_bytes), tl.m0 + 4 * lh);
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int mrow = wm * WTM + i * 32 + (v >> 2) * 8 + (v & 3);
                        __builtin_amdgcn_raw_buffer_store_b32(bits[v], ro, (int)(pix + (uint32_t)(mrow * HoWo * 4)),
                                                              0, 0);
                    }
                }
            }
        }
    };

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

    int ktile = 0;
    Tile cur_t = tile_at(0);
    Tile nxt_t = mine > 1 ? tile_at(1) : cur_t;
    StepPos cur = {0, 0, 0, 0, 0, cur_t.m0, (uint32_t)(cur_t.m0 / 32) * frag_stride, 0};
    load_a(cur, af[0]);
    __syncthreads();  // zeroing done before the fill overwrites data columns
#pragma unroll
    for (int k = 0; k < MAXI; ++k) {
        load_item(cur_t.n, cur_t.p0, 0, k);
        store_item(0, k);
    }
    __syncthreads();
    load_b(cur, 0, fb[0]);

    // One step = one (tile, chunk, tap) triple, two k16 halves.  While the MFMAs
    // of one half run, the B fragments of the following half are read.  CUR
    // selects the register set of this step's filter fragments; the loop is
    // unrolled by two so that every register array index is a compile-time
    // constant.
    const int nsteps = mine * nchunks * T;
    static_assert(MAXI == 2, "the fill schedule below places two items per chunk");
    const int FD = (T - 1) / 2;   // fill distance in steps (0: fill at the chunk end)
    auto body = [&](auto cur_c, int step) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur_c)::value;
        const bool more = step + 1 < nsteps;
        const StepPos nxt = more ? advance(cur, nxt_t.m0) : cur;
        const bool chunk_end = cur.t == T - 1;
        const bool tile_end = chunk_end && cur.ci == nchunks - 1;
        // the chunk after this one in the stream (this tile's next chunk, or the
        // next tile's first), one fill item in flight per thread: item 0's global
        // loads in step 0 of the chunk, its LDS store in step FD, item 1's loads
        // in step FD and its store in step 2*FD <= T-1.  A store comes before
        // the step's own global loads: the wait for its data then covers only
        // loads issued steps earlier (the load counter is in order).  Filters
        // with fewer than 3 taps fill the whole patch at the chunk end.
        const bool same = cur.ci + 1 < nchunks;
        const bool fill_any = same || ktile + 1 < mine;
        const int fn = same ? cur_t.n : nxt_t.n, fp0 = same ? cur_t.p0 : nxt_t.p0, fci = same ? cur.ci + 1 : 0;
        const bool spread = FD > 0;
        const bool fill_load_now = spread && fill_any && (cur.t == 0 || cur.t == FD);
        const bool fill_store_now = spread && fill_any && (cur.t == FD || cur.t == 2 * FD);
        load_b(cur, 1, fb[1]);
        mfma_half(af[CUR], 0, fb[0]);
        // Global loads are issued only after the first half's MFMAs (which wait
        // for this step's filter fragments): in-order load counters would
        // otherwise make that wait cover these newer loads as well.
        __builtin_amdgcn_sched_barrier(0);
        if (fill_store_now) store_item(cur.par ^ 1, cur.t == FD ? 0 : 1);  // that buffer was last read a chunk ago
        load_a(nxt, af[CUR ^ 1]);
        if (fill_load_now) load_item(fn, fp0, fci, cur.t == 0 ? 0 : 1);
        // unconditional (the count of outstanding LDS reads stays static); at a
        // chunk end these are re-read from the new patch after the barrier
        load_b(nxt, 0, fb[0]);
        mfma_half(af[CUR], 1, fb[1]);
        if (chunk_end && !spread && fill_any) {
#pragma unroll
            for (int k = 0; k < MAXI; ++k) {
                load_item(fn, fp0, fci, k);
                store_item(cur.par ^ 1, k);
            }
        }
        if (chunk_end && more) {
            __syncthreads();  // next chunk's patch complete; every wave is done with this one
            load_b(nxt, 0, fb[0]);
        }
        if (tile_end) {
            store_tile(cur_t);
            zero_acc();
            ++ktile;
            cur_t = nxt_t;
            if (ktile + 1 < mine) nxt_t = tile_at(ktile + 1);
        }
        cur = nxt;
    };
    for (int step = 0; step < nsteps; step += 2) {
        body(std::integral_constant<int, 0>(), step);
        if (step + 1 < nsteps) body(std::integral_constant<int, 1>(), step + 1);
    }
}


// The same computation with the filter size fixed at compile time (R x S taps,
// 3 <= R*S).  Taps are unrolled inside each chunk, so the fill schedule, the
// register sets and every patch and filter offset but the row stride are
// constants; all global loads are unconditional (the last chunk of a stream
// refills its own data into the idle buffer), so the load counter waits are
// exact; the only data-dependent branch is the tile epilogue after a chunk.
// PH: backward-data by stride phases (a.nph phases, tiles of one band's phases
// adjacent, per-phase patch offsets, filter fragments and output placement).
// TL: after the NBW 32-pixel blocks, one 16-pixel tail block on 16x16x32 MFMAs
// (for tiles of NBW*32 + 1 .. NBW*32 + 16 pixels, such as one 14 x 14 image: six
// blocks and a tail instead of seven blocks, the last holding 4 pixels).  Its B
// fragment is one 16-byte read per lane (pixel lane % 16, channel octet lane / 16);
// its A operand is the tap's two k16 filter fragments rearranged across lanes by
// two permlane swaps after the tap's 32x32 MFMAs: 16x16 operand h (rows 16h..16h+15
// of the 32-row block) takes lane rows 2h / 2h + 1 of each k16 fragment.
template <int BM, int WM, int WN, int NBW, int VW, int OCC, int R, int S, int EPI, bool PH, bool TL = false>
__global__ __launch_bounds__(256, OCC) void patch_ct_kernel(PatchArgs a) {
    constexpr int T = R * S;
    static_assert(!TL || (WN == 1 && !PH && BM == 128 && T % 3 == 0), "the tail form: one wave column, 3x3 taps");
    static_assert(T >= 3, "the fill schedule needs three taps");
    static_assert(MAXI == 2, "the fill schedule places two items per chunk");
    // fill schedule: item 0 loads at tap 0 and stores at FD; item 1 loads at FD and stores
    // at 2*FD.  With 4 taps (F2) a chunk is too short for that: both items load at tap 0
    // into two register sets and store at taps 2 and 3.
    constexpr bool F2 = T == 4;
    constexpr int FD = (T - 1) / 2;
    constexpr int WTM = BM / WM, TMB = WTM / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, lh = lane >> 5;
    const int wm = wave % WM, wn = wave / WM;
    const int nchunks = a.Cr / CK;
    const int patch_bytes = a.PR * a.PWs * CPB;
    const int rowb = a.PWs * CPB;
    const int OHW = PH ? a.OHW : a.Ho * a.Wo;   // output plane (all of dx when computing by phases)
    const int nph = PH ? a.nph : 1;

    const int per_m = a.row_tiles * a.N * nph, ntiles = a.m_tiles * per_m;
    const int G = gridDim.x;
    const int first = xcd_remap(blockIdx.x, G);
    const int mine = (ntiles - 1 - first) / G + 1;
    auto tile_at = [&](int k) __attribute__((always_inline)) {
        Tile tl;
        const int L = first + k * G;
        const int mt = L / per_m, rest = L - mt * per_m;
        const int nrt = PH ? rest / nph : rest, ph = rest - nrt * nph;   // one band's phases are neighbours
        const int n = nrt / a.row_tiles, rt = nrt - n * a.row_tiles;
        tl.n = uniform(n);
        tl.p0 = uniform(rt * a.TR);
        tl.m0 = uniform(mt * BM);
        tl.npx = uniform(min(a.TR, a.Ho - rt * a.TR) * a.Wo);
        tl.ph = PH ? uniform(ph) : 0;
        return tl;
    };

    for (int o = tid * 16; o < 2 * patch_bytes; o += 256 * 16) *(u32x4 *)(smem + o) = u32x4{0, 0, 0, 0};
    if constexpr (EPI) {   // the bias of every filter row, after the two patch buffers
        float *bs = (float *)(smem + 2 * patch_bytes);
        for (int m = tid; m < a.M; m += 256) bs[m] = a.epi.bias ? a.epi.bias[m] : 0.0f;
    }

    int pbase[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int idx = (wn + WN * j) * 32 + lr;
        const int pr = idx / a.Wo, pc = idx - pr * a.Wo;
        pbase[j] = (idx < a.TR * a.Wo ? (pr * a.PWs + pc) * CPB : 0) + lh * 16;
    }
    int pbt = 0;   // tail block: pixel NBW*32 + lane % 16, channel octet lane / 16
    if constexpr (TL) {
        const int idx = NBW * 32 + (lane & 15);
        const int pr = idx / a.Wo, pc = idx - pr * a.Wo;
        pbt = (idx < a.TR * a.Wo ? (pr * a.PWs + pc) * CPB : 0) + (lane >> 4) * 16;
    }

    // filter fragments: 1 KB per (32-row block, chunk, tap, k16 half), lane l at l*16
    const uint32_t frag_stride = (uint32_t)nchunks * T * 2048;
    const uint32_t alane = (uint32_t)lane * 16 + (uint32_t)(wm * TMB) * frag_stride;
    auto abase = [&](int m0, int ci, int ph) __attribute__((always_inline)) {
        const uint32_t b = (uint32_t)(m0 / 32) * frag_stride + (uint32_t)ci * (T * 2048);
        return PH ? b + (uint32_t)ph * a.wt_phase : b;
    };
    auto boff = [&](int ph) __attribute__((always_inline)) { return PH ? phase_sel(a.ph_boff, ph) : 0; };
    auto load_a = [&](uint32_t base, int t, u32x4 (&dst)[TMB][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TMB; ++i)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                dst[i][u] = ld_vec_s(make_rsrc(a.Wt, a.w_bytes), alane, base + i * frag_stride + t * 2048 + u * 1024);
    };

    const int nitems = 4 * a.PR * a.G;
    ItemPos items[MAXI];
#pragma unroll
    for (int k = 0; k < MAXI; ++k) items[k] = item_pos(tid + k * 256, nitems, a.G, a.PR);
    FillItem<VW> fis[F2 ? 2 : 1];
    auto load_item = [&](int n, int p0, int ci, int k) __attribute__((always_inline)) {
        fill_load<VW>(make_rsrc(a.X, a.x_bytes), items[k], a.Cr, a.Hi, a.Wi, a.ph, n, p0, ci * CK, fis[F2 ? k : 0]);
    };
    auto store_item = [&](int buf_off, int k) __attribute__((always_inline)) {
        fill_store<VW, CPB>(smem + buf_off, items[k], a.PWs, a.pw, fis[F2 ? k : 0]);
    };

    f32x16 acc[TMB][NBW];
    f32x4 acct[TL ? TMB : 1][2];   // tail: rows 16h + 4*(lane / 16) + v of block i, pixel lane % 16
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TMB; ++i)
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
        if constexpr (TL) {
#pragma unroll
            for (int i = 0; i < TMB; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acct[i][h][v] = 0.0f;
        }
    };
    zero_acc();
    auto store_tile = [&](const Tile &tl) __attribute__((always_inline)) {
        const int inplane = PH ? (phase_sel(a.ph_i0, tl.ph) + a.osh * tl.p0) * a.OW + phase_sel(a.ph_j0, tl.ph)
                               : tl.p0 * a.Wo;
        const size_t base = ((size_t)tl.n * a.M + tl.m0) * OHW + (size_t)inplane;
        constexpr int OES = EPI == 2 ? 2 : 4;   // output element bytes
        const long long room = ((long long)(a.M - tl.m0) * OHW - inplane) * OES;
        const rsrc_t ro = make_rsrc((char *)a.O + base * OES, (uint32_t)(room < 0x7fffffffLL ? room : 0x7fffffffLL));
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int idx = (wn + WN * j) * 32 + lr;
            // the pixel's offset from the tile's first output pixel (rows and columns
            // strided by osh / osw when computing by phases)
            int pout = idx;
            if constexpr (PH) {
                const int pr = idx / a.Wo, pc = idx - pr * a.Wo;
                pout = pr * a.osh * a.OW + pc * a.osw;
            }
            const uint32_t pix = idx < tl.npx ? (uint32_t)((lh * 4 * OHW + pout) * OES) : kOOB;
#pragma unroll
            for (int i = 0; i < TMB; ++i) {
                const u32x16 bits = __builtin_bit_cast(u32x16, acc[i][j]);
                if constexpr (EPI) {
                    store_block_epi<EPI>(a, ro, pix, bits, wm * WTM + i * 32, OHW,
                                         (const float *)(smem + 2 * patch_bytes), tl.m0 + 4 * lh);
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int mrow = wm * WTM + i * 32 + (v >> 2) * 8 + (v & 3);
                        __builtin_amdgcn_raw_buffer_store_b32(bits[v], ro, (int)(pix + (uint32_t)(mrow * OHW * 4)),
                                                              0, 0);
                    }
                }
            }
        }
        if constexpr (TL) {   // the tail block (plain pixel placement: TL excludes phases)
            // lane offsets computed here, not kept from before the chunk loop (registers)
            int tlane = lane;
            asm volatile("" : "+v"(tlane));
            const int idx = NBW * 32 + (tlane & 15);
            const uint32_t pix = idx < tl.npx ? (uint32_t)(idx * OES) : kOOB;
#pragma unroll
            for (int i = 0; i < TMB; ++i) {
                const int row0 = wm * WTM + i * 32 + 4 * (tlane >> 4);
                if constexpr (EPI) {   // per 16-row half: its 4 previous values, then its 4 stores
                    const float *bs = (const float *)(smem + 2 * patch_bytes);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        float old[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int off = (int)(pix + (uint32_t)((row0 + h * 16 + v) * OHW * OES));
                            if constexpr (EPI == 2)
                                old[v] = a.epi.beta != 0.0f
                                             ? bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(ro, off, 0, 0))
                                             : 0.0f;
                            else
                                old[v] = a.epi.beta != 0.0f
                                             ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, off, 0, 0))
                                             : 0.0f;
                        }
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int mrow = row0 + h * 16 + v;
                            const int off = (int)(pix + (uint32_t)(mrow * OHW * OES));
                            const float val =
                                epi_apply(a.epi, acct[i][h][v], bs[min(tl.m0 + mrow, a.M - 1)], old[v]);
                            if constexpr (EPI == 2)
                                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(val), ro, off, 0, 0);
                            else
                                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ro, off, 0, 0);
                        }
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int mrow = row0 + (u >> 2) * 16 + (u & 3);
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acct[i][u >> 2][u & 3]), ro,
                                                              (int)(pix + (uint32_t)(mrow * OHW * 4)), 0, 0);
                    }
                }
            }
        }
    };

    // B fragments (one register set, rolled): at patch byte offset `off`
    // (buffer + row, uniform) plus a compile-time column/half offset.  In each
    // half-step, right after the MFMAs of block j the block's fragment of the
    // next half-step is read into the same registers; the six MFMAs of the
    // other blocks cover the LDS latency.
    u32x4 fb[NBW];
    auto load_b = [&](int off, int imm) __attribute__((always_inline)) {
        const char *B = smem + off + imm;
#pragma unroll
        for (int j = 0; j < NBW; ++j) fb[j] = *(const u32x4 *)(B + pbase[j]);
    };
    auto mfma_half = [&](const u32x4 (&A)[TMB][2], int u, bool roll, int off, int imm) __attribute__((always_inline)) {
        const char *B = smem + off + imm;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
#pragma unroll
            for (int i = 0; i < TMB; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, A[i][u]), __builtin_bit_cast(bf16x8, fb[j]), acc[i][j], 0, 0, 0);
            if (roll) {
                fb[j] = *(const u32x4 *)(B + pbase[j]);
                __builtin_amdgcn_sched_group_barrier(0x008, TMB, 0);   // the block's MFMAs
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // then its next read
            }
        }
    };

    // tail block: after a tap's 32x32 MFMAs its two k16 fragments (lane rows R0..R3 of 16
    // lanes: rows 0-15 / 16-31 of the block x channel octet 2u / 2u+1) are rearranged in
    // place into the two 16x16x32 A operands [f0.R0 f0.R2 f1.R0 f1.R2] (rows 0-15,
    // octets 0..3) and [f0.R1 f0.R3 f1.R1 f1.R3] (rows 16-31): a 32-lane swap of f0's
    // upper half with f1's lower half, then a 16-lane swap of the odd rows of the first
    // with the even rows of the second.  The set is reloaded afterwards for a later tap.
    u32x4 fbt = {0, 0, 0, 0};
    auto tail_mfma = [&](u32x4 (&A)[TMB][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TMB; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const auto p = __builtin_amdgcn_permlane32_swap(A[i][0][e], A[i][1][e], false, false);
                const auto q = __builtin_amdgcn_permlane16_swap(p[0], p[1], false, false);
                A[i][0][e] = q[0];
                A[i][1][e] = q[1];
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
                acct[i][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, A[i][h]), __builtin_bit_cast(bf16x8, fbt), acct[i][h], 0, 0, 0);
        }
    };

    // stream state (work-group uniform)
    int ktile = 0, ci = 0;
    Tile cur_t = tile_at(0);
    Tile nxt_t = mine > 1 ? tile_at(1) : cur_t;
    // filter fragments AD steps ahead, in NA register sets:
    //  - 64-row form, T = 6 or 9: AD = 5 (the fragments travel from L2 for about 5 of its
    //    short steps), six sets; global step P*T + t (P = chunk parity) uses set
    //    (P*T + t) % 6, which repeats every two chunks since 2T % 6 == 0;
    //  - T = 4: four sets, step t uses set t and loads step t + AD into set (t + AD) % 4;
    //    AD = 3 on the 64-row form (the set step t - 1 has finished with), 2 on the
    //    128-row form (registers);
    //  - other multiples of 3: AD = 2, step t uses set t % 3;
    //  - else AD = 1, two sets by step parity.
    constexpr bool DEEP = BM == 64 && T % 3 == 0 && T >= 6;
    constexpr int AD = DEEP ? 5 : (T == 4 ? (BM == 64 ? 3 : 2) : (T % 3 == 0 ? 2 : 1));
    constexpr int NA = DEEP ? 6 : (T == 4 ? 4 : AD + 1);
    u32x4 af[NA][TMB][2];
    static_for<0, AD>([&](auto tc) __attribute__((always_inline)) {
        constexpr int t = decltype(tc)::value;
        load_a(abase(cur_t.m0, 0, cur_t.ph), t, af[t]);
    });
    __syncthreads();
#pragma unroll
    for (int k = 0; k < MAXI; ++k) {
        load_item(cur_t.n, cur_t.p0, 0, k);
        store_item(0, k);
    }
    __syncthreads();
    load_b(boff(cur_t.ph), 0);

    const int nch_total = mine * nchunks;
    auto chunk = [&](auto par_c, int g) __attribute__((always_inline)) {
        constexpr int P = decltype(par_c)::value;   // patch buffer of this chunk
        const bool tile_last = ci == nchunks - 1;
        const bool more = g + 1 < nch_total;
        // the next chunk of the stream; the stream's last chunk refills itself
        // into the idle buffer (never read again)
        const bool nt = tile_last && more;
        const int fn = nt ? nxt_t.n : cur_t.n, fp0 = nt ? nxt_t.p0 : cur_t.p0;
        const int fci = tile_last ? (more ? 0 : ci) : ci + 1;
        const int fm0 = nt ? nxt_t.m0 : cur_t.m0, fph = nt ? nxt_t.ph : cur_t.ph;
        const uint32_t a_cur = abase(cur_t.m0, ci, cur_t.ph), a_nxt = abase(fm0, fci, fph);
        // B reads start at the tile's phase offset into the shared patch layout
        const int buf = (P ? patch_bytes : 0) + boff(cur_t.ph), nbuf = P ? 0 : patch_bytes;
        static_for<0, T>([&](auto t_c) __attribute__((always_inline)) {
            constexpr int t = decltype(t_c)::value;
            constexpr int r = t / S, s = t % S;
            constexpr int CUR = DEEP ? (P * T + t) % 6 : (T == 4 ? t : (AD == 2 ? t % 3 : (P * T + t) & 1));
            constexpr int NXT = DEEP ? (P * T + t + AD) % 6
                                     : (T == 4 ? (t + AD) % 4 : (AD == 2 ? (t + 2) % 3 : CUR ^ 1));
            // half 0 (channels 0..15 of the chunk), rolling in half 1 of this tap
            mfma_half(af[CUR], 0, true, buf + r * rowb, s * CPB + 32);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (F2) {
                if constexpr (t == 2 || t == 3) store_item(nbuf, t - 2);
            } else if constexpr (t == FD || t == 2 * FD) {
                store_item(nbuf, t == FD ? 0 : 1);
            }
            if constexpr (t + AD < T)
                load_a(a_cur, t + AD, af[NXT]);
            else
                load_a(a_nxt, t + AD - T, af[NXT]);
            if constexpr (F2) {
                if constexpr (t == 0) {
                    load_item(fn, fp0, fci, 0);
                    load_item(fn, fp0, fci, 1);
                }
            } else if constexpr (t == 0 || t == FD) {
                load_item(fn, fp0, fci, t == 0 ? 0 : 1);
            }
            if constexpr (TL) fbt = *(const u32x4 *)(smem + buf + r * rowb + s * CPB + pbt);
            __builtin_amdgcn_sched_barrier(0);
            // half 1, rolling in half 0 of the next tap (of this chunk)
            constexpr int r1 = (t + 1) / S, s1 = (t + 1) % S;
            mfma_half(af[CUR], 1, t + 1 < T, buf + r1 * rowb, s1 * CPB);
            if constexpr (TL) tail_mfma(af[CUR]);
            __builtin_amdgcn_sched_barrier(0);
        });
        __syncthreads();   // next chunk's patch complete; every wave is done with this one
        load_b(nbuf + boff(fph), 0);
        if (tile_last) {
            store_tile(cur_t);
            zero_acc();
            ++ktile;
            cur_t = nxt_t;
            if (ktile + 1 < mine) nxt_t = tile_at(ktile + 1);
            ci = 0;
        } else {
            ++ci;
        }
    };
    for (int g = 0; g < nch_total; g += 2) {
        chunk(std::integral_constant<int, 0>(), g);
        if (g + 1 < nch_total) chunk(std::integral_constant<int, 1>(), g + 1);
    }
}

// Filter copy in MFMA fragment order for the patch kernels (one thread per 16
// bytes).  Fragment (mb, ci, t, u) is 1 KB at ((mb*nchunks + ci)*T + t)*2 + u;
// lane l holds row m = 32*mb + l%32 and channels ci*32 + u*16 + (l/32)*8 .. +7
// of tap t.  Forward: A[m][t][c] = w[m][c][t] (m = k).  Backward-data
// (rotated, K and C exchanged): A[m][t][k] = w[k][m][T-1-t] (m = c).  Rows
// m >= M are zero.
__global__ __launch_bounds__(256) void filter_to_frag(const uint16_t *__restrict__ w, uint16_t *__restrict__ wt,
                                                      int K, int C, int T, int M, int Cr, int nvec, int bwd) {
    const int v = blockIdx.x * 256 + threadIdx.x;
    if (v >= nvec) return;
    const int nchunks = Cr / 32;
    const int lane = v & 63, u = (v >> 6) & 1;
    const int rest = v >> 7;                 // (mb*nchunks + ci)*T + t
    const int t = rest % T, mc = rest / T;
    const int ci = mc % nchunks, mb = mc / nchunks;
    const int m = mb * 32 + (lane & 31);
    const int c0 = ci * 32 + u * 16 + (lane >> 5) * 8;
    uint32_t d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t lo = 0, hi = 0;
        if (m < M) {
            const int ca = c0 + 2 * e, cb = ca + 1;
            if (!bwd) {
                lo = w[((size_t)m * C + ca) * T + t];
                hi = w[((size_t)m * C + cb) * T + t];
            } else {
                lo = w[((size_t)ca * C + m) * T + (T - 1 - t)];
                hi = w[((size_t)cb * C + m) * T + (T - 1 - t)];
            }
        }
        d[e] = lo | (hi << 16);
    }
    *(u32x4 *)(wt + (size_t)v * 8) = u32x4{d[0], d[1], d[2], d[3]};
}

// Filter copy for backward-data by stride phases, in the same fragment order per
// phase (phase f = fh*sw + fw, `per` vectors each): sub-tap t = u*nuw + v of phase f
// is the filter tap (fh + sh*(nuh-1-u), fw + sw*(nuw-1-v)) -- the phase's taps,
// reversed -- and A[m][t][k] = w[k][m][r][s] (m = c).  Rows m >= M are zero.
__global__ __launch_bounds__(256) void filter_to_frag_phases(const uint16_t *__restrict__ w, uint16_t *__restrict__ wt,
                                                             int C, int R, int S, int M, int Cr, int sw_, int sh_,
                                                             int nuh, int nuw, int per, int total) {
    const int gv = blockIdx.x * 256 + threadIdx.x;
    if (gv >= total) return;
    const int f = gv / per, v = gv - f * per;
    const int fh = f / sw_, fw = f - fh * sw_;
    const int T = nuh * nuw, nchunks = Cr / 32;
    const int lane = v & 63, u = (v >> 6) & 1;
    const int rest = v >> 7;                 // (mb*nchunks + ci)*T + t
    const int t = rest % T, mc = rest / T;
    const int ci = mc % nchunks, mb = mc / nchunks;
    const int m = mb * 32 + (lane & 31);
    const int c0 = ci * 32 + u * 16 + (lane >> 5) * 8;
    const int tu = t / nuw, tv = t - tu * nuw;
    const int r = fh + sh_ * (nuh - 1 - tu), s = fw + sw_ * (nuw - 1 - tv);
    uint32_t d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t lo = 0, hi = 0;
        if (m < M) {
            const int ka = c0 + 2 * e, kb = ka + 1;
            lo = w[(((size_t)ka * C + m) * R + r) * S + s];
            hi = w[(((size_t)kb * C + m) * R + r) * S + s];
        }
        d[e] = lo | (hi << 16);
    }
    *(u32x4 *)(wt + (size_t)gv * 8) = u32x4{d[0], d[1], d[2], d[3]};
}

// The same copy for large filters, one work-group per (32-row block mb, 32-channel
// chunk ci): the 32 source rows' 32*T contiguous elements (forward: rows m of
// W[m][ci*32..][t]; backward-data: rows k = ci*32.. of W[k][mb*32..][t]) are read
// with 16-byte loads into LDS (row stride padded by 2 elements for the banks),
// then the 2*T fragments of the block are written with 16-byte stores, lane
// after lane.  Needs M % 32 == 0 (no padding rows) and 2*T KB of LDS.
__global__ __launch_bounds__(256) void filter_to_frag_tiled(const uint16_t *__restrict__ w, uint16_t *__restrict__ wt,
                                                            int C, int T, int Cr, int bwd) {
    extern __shared__ uint16_t slab[];   // [32][32*T + 2]
    const int nchunks = Cr / 32;
    const int mb = blockIdx.x / nchunks, ci = blockIdx.x - mb * nchunks;
    const int rl = 32 * T, rs = rl + 2;   // row length, LDS row stride (elements)
    const int vpr = rl / 8;               // 16-byte vectors per row
    for (int q = threadIdx.x; q < 32 * vpr; q += 256) {
        const int row = q / vpr, v = q - row * vpr;
        const size_t src = bwd ? ((size_t)(ci * 32 + row) * C + mb * 32) * T : ((size_t)(mb * 32 + row) * C + ci * 32) * T;
        const u32x4 d = *(const u32x4 *)(w + src + (size_t)v * 8);
        uint32_t *dst = (uint32_t *)(slab + row * rs + v * 8);   // 4-byte aligned (rs is even)
        dst[0] = d[0];
        dst[1] = d[1];
        dst[2] = d[2];
        dst[3] = d[3];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < 128 * T; q += 256) {
        const int lane = q & 63, u = (q >> 6) & 1, t = q >> 7;
        const int ml = lane & 31, cl = u * 16 + (lane >> 5) * 8;
        uint32_t d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t lo, hi;
            if (!bwd) {   // A[m][t][c] = w[m][c][t]
                lo = slab[ml * rs + (cl + 2 * e) * T + t];
                hi = slab[ml * rs + (cl + 2 * e + 1) * T + t];
            } else {      // A[m][t][k] = w[k][m][T-1-t]
                lo = slab[(cl + 2 * e) * rs + ml * T + (T - 1 - t)];
                hi = slab[(cl + 2 * e + 1) * rs + ml * T + (T - 1 - t)];
            }
            d[e] = lo | (hi << 16);
        }
        const size_t vec = (((size_t)blockIdx.x * T + t) * 2 + u) * 64 + lane;
        *(u32x4 *)(wt + vec * 8) = u32x4{d[0], d[1], d[2], d[3]};
    }
}

// Work-groups of `func` (block threads, lds bytes of dynamic LDS) that the current
// device holds at once.  Cached per (device, kernel, lds); the occupancy query
// is host-only work.
hipError_t resident_slots(const void *func, int threads, size_t lds, int *slots) {
    struct Entry {
        int dev;
        const void *func;
        size_t lds;
        int slots;
    };
    static std::mutex mu;
    static Entry cache[64];
    static int used = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    {
        std::lock_guard<std::mutex> g(mu);
        for (int i = 0; i < used; ++i)
            if (cache[i].dev == dev && cache[i].func == func && cache[i].lds == lds) {
                *slots = cache[i].slots;
                return hipSuccess;
            }
    }
    int cus = 0, per = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, func, threads, lds);
    if (e != hipSuccess) return e;
    const int n = (per > 0 ? per : 1) * (cus > 0 ? cus : 1);
    std::lock_guard<std::mutex> g(mu);
    if (used < 64) cache[used++] = Entry{dev, func, lds, n};
    *slots = n;
    return hipSuccess;
}

// Launch of one patch configuration: at most one work-group per resident slot,
// each with the same number of tiles; returns a hipError_t.
template <int BM, int WM, int WN, int NBW, int VW, int OCC, int EPI>
static hipError_t patch_go(const PatchArgs &a, int ntiles, size_t lds, hipStream_t st) {
    auto k = patch_kernel<BM, WM, WN, NBW, VW, OCC, EPI>;
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int slots = 0;
    e = resident_slots((const void *)k, 256, lds, &slots);
    if (e != hipSuccess) return e;
    // as many tiles for every work-group (ceil(tiles / slots) each), not one per slot
    const int per = (ntiles + slots - 1) / slots, grid = (ntiles + per - 1) / per;
    hipLaunchKernelGGL(k, dim3(grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int BM, int WM, int WN, int NBW, int VW, int OCC, int R, int S, int EPI, bool PH = false, bool TL = false>
static hipError_t patch_ct_go(const PatchArgs &a, int ntiles, size_t lds, hipStream_t st) {
    auto k = patch_ct_kernel<BM, WM, WN, NBW, VW, OCC, R, S, EPI, PH, TL>;
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int slots = 0;
    e = resident_slots((const void *)k, 256, lds, &slots);
    if (e != hipSuccess) return e;
    // as many tiles for every work-group (ceil(tiles / slots) each), not one per slot
    const int per = (ntiles + slots - 1) / slots, grid = (ntiles + per - 1) / per;
    hipLaunchKernelGGL(k, dim3(grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int BM, int WM, int WN, int NBW, int OCC, int EPI>
static hipError_t patch_vw(const PatchArgs &a, int vw, int ntiles, size_t lds, hipStream_t st) {
    // 2 x 2 taps: backward-data by stride phases, and (64-row form) any other 2 x 2 run --
    // the space-to-depth forward -- as a single phase of the same kernel
    if (a.R == 2 && a.S == 2 && (a.nph > 1 || BM == 64)) {
        if (vw == 2) return patch_ct_go<BM, WM, WN, NBW, 2, OCC, 2, 2, EPI, true>(a, ntiles, lds, st);
        if constexpr (BM == 64) {   // the plan gives the 128-row form column groups of 2
            if (vw == 8) return patch_ct_go<BM, WM, WN, NBW, 8, OCC, 2, 2, EPI, true>(a, ntiles, lds, st);
            if (vw == 4) return patch_ct_go<BM, WM, WN, NBW, 4, OCC, 2, 2, EPI, true>(a, ntiles, lds, st);
        }
        return hipErrorInvalidValue;
    }
    if (a.nph > 1) return hipErrorInvalidValue;   // phases run on the compile-time-tap kernel only
    if (a.R == 3 && a.S == 3) {
        if (vw == 8) return patch_ct_go<BM, WM, WN, NBW, 8, OCC, 3, 3, EPI>(a, ntiles, lds, st);
        if (vw == 4) return patch_ct_go<BM, WM, WN, NBW, 4, OCC, 3, 3, EPI>(a, ntiles, lds, st);
        return patch_ct_go<BM, WM, WN, NBW, 2, OCC, 3, 3, EPI>(a, ntiles, lds, st);
    }
    if (vw == 8) {   // the plan gives the 128-row form column groups of 4 or 2
        if constexpr (BM == 64) return patch_go<BM, WM, WN, NBW, 8, OCC, EPI>(a, ntiles, lds, st);
        return hipErrorInvalidValue;
    }
    if (vw == 4) return patch_go<BM, WM, WN, NBW, 4, OCC, EPI>(a, ntiles, lds, st);
    return patch_go<BM, WM, WN, NBW, 2, OCC, EPI>(a, ntiles, lds, st);
}

static int run_patch(const Plan &pl, PatchArgs &a, int ntiles, size_t lds, hipStream_t st, const Epi *epi);

// Space-to-depth regrouping for the stride-2 forward (4x4 filters): z[n][(2a + b)*C + c][i][j]
// = x[n][c][2(i + u0[a]) + a][2(j + u0[b]) + b], zero outside x and for j >= Q + 1 (the
// pitch zw is a multiple of 8).  One thread writes 8 consecutive j of one z row for both
// column phases b (two 16-byte stores).  With an even W, x column pairs (2d, 2d + 1) are one
// 4-byte word, and phase b takes half b of word j + u0[b]: the thread loads the words
// jg*8 + min(u0) .. jg*8 + 7 + max(u0) (at most 10) once for both phases.
__global__ __launch_bounds__(256) void space_to_depth(const uint16_t *__restrict__ x, uint16_t *__restrict__ z,
                                                      uint32_t x_bytes, int C, int H, int W, int zh, int zw, int zwc,
                                                      int uh0, int uh1, int uw0, int uw1, int nvec) {
    const int v = blockIdx.x * 256 + threadIdx.x;
    if (v >= nvec) return;
    const int groups = zw / 8;
    int rest = v;
    const int jg = rest % groups;
    rest /= groups;
    const int i = rest % zh;
    rest /= zh;
    const int a = rest & 1;
    const int nc = rest >> 1;   // n*C + c
    const int n = nc / C, c = nc - n * C;
    const int ih = 2 * (i + (a ? uh1 : uh0)) + a;
    const bool row_ok = (unsigned)ih < (unsigned)H;
    const rsrc_t rx = make_rsrc(x, x_bytes);
    const size_t rowe = ((size_t)nc * H + (row_ok ? ih : 0)) * W;   // first element of the x row
    uint32_t out[2][4];
    if ((W & 1) == 0) {
        const int umin = uw0 < uw1 ? uw0 : uw1;
        const int d0 = jg * 8 + umin, W2 = W >> 1;
        uint32_t wd[10];
#pragma unroll
        for (int k = 0; k < 10; ++k) {
            const int d = d0 + k;
            const bool ok = row_ok && (unsigned)d < (unsigned)W2;
            wd[k] = ok ? ld_elem<4>(rx, (uint32_t)((rowe + 2 * (size_t)d) * 2)) : 0u;
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int off = (b ? uw1 : uw0) - umin;   // 0, 1 or 2
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t h[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int jj = 2 * e + q;
                    const uint32_t word = off == 0 ? wd[jj] : (off == 1 ? wd[jj + 1] : wd[jj + 2]);
                    const uint32_t val = b ? (word >> 16) : (word & 0xffffu);
                    h[q] = jg * 8 + jj < zwc ? val : 0u;
                }
                out[b][e] = h[0] | (h[1] << 16);
            }
        }
    } else {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t h[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int j = jg * 8 + 2 * e + q;
                    const int iw = 2 * (j + (b ? uw1 : uw0)) + b;
                    const bool ok = row_ok && j < zwc && (unsigned)iw < (unsigned)W;
                    h[q] = ok ? (ld_elem<2>(rx, (uint32_t)((rowe + iw) * 2)) & 0xffffu) : 0u;
                }
                out[b][e] = h[0] | (h[1] << 16);
            }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const size_t plane = (size_t)n * 4 * C + (size_t)(2 * a + b) * C + c;
        *(u32x4 *)(z + (plane * zh + i) * zw + jg * 8) = u32x4{out[b][0], out[b][1], out[b][2], out[b][3]};
    }
}

// Filter copy for the space-to-depth forward, in the patch kernels' fragment order over
// the regrouped problem: rows m = k, channels (2a + b)*C + c, taps t = v*2 + w (2 x 2);
// tap (v, w) of phase (a, b) is the filter tap (2(u0[a] + v) + a + ph, 2(u0[b] + w) + b + pw).
// Rows m >= K are zero.
__global__ __launch_bounds__(256) void filter_to_frag_s2d(const uint16_t *__restrict__ w, uint16_t *__restrict__ wt,
                                                          int K, int C, int uh0, int uh1, int uw0, int uw1, int ph,
                                                          int pw, int nvec) {
    const int v = blockIdx.x * 256 + threadIdx.x;
    if (v >= nvec) return;
    constexpr int T = 4;
    const int Cz = 4 * C, nchunks = Cz / 32;
    const int lane = v & 63, u = (v >> 6) & 1;
    const int rest = v >> 7;                 // (mb*nchunks + ci)*T + t
    const int t = rest % T, mc = rest / T;
    const int ci = mc % nchunks, mb = mc / nchunks;
    const int m = mb * 32 + (lane & 31);
    const int c0 = ci * 32 + u * 16 + (lane >> 5) * 8;
    const int tv = t >> 1, tw = t & 1;
    uint32_t d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t half[2] = {0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int cz = c0 + 2 * e + h;
            const int ab = cz / C, c = cz - ab * C, a = ab >> 1, b = ab & 1;
            const int r = 2 * ((a ? uh1 : uh0) + tv) + a + ph, s = 2 * ((b ? uw1 : uw0) + tw) + b + pw;
            if (m < K) half[h] = w[(((size_t)m * C + c) * 4 + r) * 4 + s];
        }
        d[e] = half[0] | (half[1] << 16);
    }
    *(u32x4 *)(wt + (size_t)v * 8) = u32x4{d[0], d[1], d[2], d[3]};
}

static int s2d_u0(int a, int pad) {
    const int r0 = ((a + pad) % 2 + 2) % 2;
    return (r0 - pad - a) / 2;
}

// Forward at stride 2 with a 4x4 filter by space-to-depth (plan.s2d): z and the 2 x 2
// sub-filters into the workspace, then the stride-1 2 x 2 correlation of z (pad 0, Q + 1
// of z's zw columns read) on the 64-row compile-time-tap patch kernel.
static int launch_patch_s2d(const Plan &pl, const Problem &p, const void *x, const void *w, float *y, void *ws,
                            hipStream_t st, const Epi *epi) {
    const int uh0 = s2d_u0(0, p.ph), uh1 = s2d_u0(1, p.ph), uw0 = s2d_u0(0, p.pw), uw1 = s2d_u0(1, p.pw);
    const int Cz = 4 * p.C;
    if (pl.bm != 64 || Cz % 32 != 0 || pl.zw % 8 != 0 || pl.zh != p.P + 1 || pl.zw < p.Q + 1) return MICONV_ERR_HIP;
    uint16_t *wt = (uint16_t *)((char *)ws + pl.wt_offset);
    uint16_t *z = (uint16_t *)((char *)ws + pl.z_offset);
    const int nvw = (int)(pl.wt_bytes / 16);   // m_tiles*64 rows x 4 taps x Cz, 8 per vector
    if ((size_t)nvw * 16 != (size_t)pl.m_tiles * 64 * 4 * Cz * 2) return MICONV_ERR_HIP;
    hipLaunchKernelGGL(filter_to_frag_s2d, dim3((nvw + 255) / 256), dim3(256), 0, st, (const uint16_t *)w, wt, p.K,
                       p.C, uh0, uh1, uw0, uw1, p.ph, p.pw, nvw);
    const long long nvz = (long long)p.N * Cz * pl.zh * (pl.zw / 8);   // 16-byte vectors of z
    if ((size_t)nvz * 16 != pl.z_bytes) return MICONV_ERR_HIP;
    const long long nth = nvz / 2;   // one thread per vector pair (both column phases)
    hipLaunchKernelGGL(space_to_depth, dim3((unsigned)((nth + 255) / 256)), dim3(256), 0, st, (const uint16_t *)x, z,
                       (uint32_t)((size_t)p.N * p.C * p.H * p.W * 2), p.C, p.H, p.W, pl.zh, pl.zw, p.Q + 1, uh0, uh1,
                       uw0, uw1, (int)nth);
    if (hipGetLastError() != hipSuccess) return MICONV_ERR_HIP;
    PatchArgs a = {};
    a.X = z;
    a.x_bytes = (uint32_t)pl.z_bytes;
    a.Cr = Cz; a.Hi = pl.zh; a.Wi = pl.zw; a.M = p.K;
    a.ph = 0; a.pw = 0; a.Ho = p.P; a.Wo = p.Q;
    a.Wt = wt;
    a.w_bytes = (uint32_t)pl.wt_bytes;
    a.O = y;
    a.N = p.N; a.R = 2; a.S = 2;
    a.TR = pl.tr;
    a.row_tiles = (a.Ho + a.TR - 1) / a.TR;
    a.m_tiles = pl.m_tiles;
    a.PWc = a.Wo + 1;
    a.PWs = pl.pws;
    a.PR = a.TR + 1;
    a.G = a.Wi / pl.vw;
    a.nph = 1; a.osh = 1; a.osw = 1; a.OW = a.Wo; a.OHW = a.Ho * a.Wo;
    // every loaded z column (zw per row, from position 0) lands inside its patch row
    if (a.PWs < a.Wi || 4 * a.PR * a.G > 512) return MICONV_ERR_HIP;
    const int ntiles = pl.m_tiles * a.row_tiles * p.N;
    const size_t lds = 2 * (size_t)a.PR * a.PWs * CPB;
    return run_patch(pl, a, ntiles, lds, st, epi);
}

// Backward-data by stride phases (plan.phases > 1): every phase (fh, fw) is a
// stride-1 correlation of dy with its 2 x 2 taps reversed (filter_to_frag_phases)
// and padding nu - 1 - base, written to dx rows i0 + 2a and columns j0 + 2b.  The
// patch is filled once per band with the largest padding of any phase; a phase
// with less padding starts its reads the difference further into it.
static int launch_patch_phases(const Plan &pl, const Problem &p, const void *dy, const void *w, float *dx,
                               void *ws, hipStream_t st, const Epi *epi);
static int run_patch(const Plan &pl, PatchArgs &a, int ntiles, size_t lds, hipStream_t st, const Epi *epi);

int launch_patch(const Plan &pl, const Problem &p, const void *in0, const void *in1, float *out, void *ws,
                 hipStream_t st, const Epi *epi) {
    if (pl.phases > 1) return launch_patch_phases(pl, p, in0, in1, out, ws, st, epi);
    if (pl.s2d) return launch_patch_s2d(pl, p, in0, in1, out, ws, st, epi);
    const int T = p.R * p.S;
    PatchArgs a = {};
    uint16_t *wt = (uint16_t *)((char *)ws + pl.wt_offset);
    const int Mr = p.pass == FWD ? p.K : p.C, Crr = p.pass == FWD ? p.C : p.K;
    const int nvec = (int)(pl.wt_bytes / 16);   // m_tiles*bm rows x T x Cr, 8 per vector
    const size_t slab = (size_t)32 * (32 * T + 2) * 2;
    if (Mr % 32 == 0 && nvec >= 65536 && slab <= 64 * 1024)   // large filters: tiled copy
        hipLaunchKernelGGL(filter_to_frag_tiled, dim3((Mr / 32) * (Crr / 32)), dim3(256), slab, st,
                           (const uint16_t *)in1, wt, p.C, T, Crr, p.pass == FWD ? 0 : 1);
    else
        hipLaunchKernelGGL(filter_to_frag, dim3((nvec + 255) / 256), dim3(256), 0, st, (const uint16_t *)in1, wt,
                           p.K, p.C, T, Mr, Crr, nvec, p.pass == FWD ? 0 : 1);
    if (p.pass == FWD) {
        a.X = in0;
        a.x_bytes = (uint32_t)((size_t)p.N * p.C * p.H * p.W * 2);
        a.Cr = p.C; a.Hi = p.H; a.Wi = p.W; a.M = p.K;
        a.ph = p.ph; a.pw = p.pw; a.Ho = p.P; a.Wo = p.Q;
    } else {
        a.X = in0;
        a.x_bytes = (uint32_t)((size_t)p.N * p.K * p.P * p.Q * 2);
        a.Cr = p.K; a.Hi = p.P; a.Wi = p.Q; a.M = p.C;
        a.ph = p.R - 1 - p.ph; a.pw = p.S - 1 - p.pw; a.Ho = p.H; a.Wo = p.W;
    }
    if (hipGetLastError() != hipSuccess) return MICONV_ERR_HIP;
    a.Wt = wt;
    a.w_bytes = (uint32_t)pl.wt_bytes;
    a.O = out;
    a.N = p.N; a.R = p.R; a.S = p.S;
    a.TR = pl.tr;
    a.row_tiles = (a.Ho + a.TR - 1) / a.TR;
    a.m_tiles = pl.m_tiles;
    a.PWc = a.Wo + p.S - 1;
    a.PWs = pl.pws;
    a.PR = a.TR + p.R - 1;
    a.G = a.Wi / pl.vw;
    a.nph = 1; a.osh = 1; a.osw = 1; a.OW = a.Wo; a.OHW = a.Ho * a.Wo;
    const int ntiles = pl.m_tiles * a.row_tiles * p.N;
    const size_t lds = 2 * (size_t)a.PR * a.PWs * CPB;
    return run_patch(pl, a, ntiles, lds, st, epi);
}

// The tail form (plan.tail): 128 filter rows, 3x3, six 32-pixel blocks and a 16-pixel tail,
// 4-byte fill loads.
template <int EPI>
static hipError_t patch_tail_vw(const PatchArgs &a, int vw, int ntiles, size_t lds, hipStream_t st) {
    if (a.R != 3 || a.S != 3 || a.nph != 1 || vw != 2) return hipErrorInvalidValue;
    return patch_ct_go<128, 4, 1, 6, 2, 2, 3, 3, EPI, false, true>(a, ntiles, lds, st);
}

static int run_patch(const Plan &pl, PatchArgs &a, int ntiles, size_t lds, hipStream_t st, const Epi *epi) {
    hipError_t e;
    if (pl.tail && pl.bm == 128 && pl.phases <= 1 && !pl.s2d) {
        if (epi) {
            a.epi = *epi;
            const size_t lds_b = lds + ((size_t)a.M * 4 + 15) / 16 * 16;   // plus the bias copy
            e = epi->out_bf16 ? patch_tail_vw<2>(a, pl.vw, ntiles, lds_b, st)
                              : patch_tail_vw<1>(a, pl.vw, ntiles, lds_b, st);
        } else {
            e = patch_tail_vw<0>(a, pl.vw, ntiles, lds, st);
        }
    } else if (epi) {   // forward: bias over K rows; backward-data (deconvolution forward): over C rows
        a.epi = *epi;
        const size_t lds_b = lds + ((size_t)a.M * 4 + 15) / 16 * 16;   // plus the bias copy
        if (epi->out_bf16)
            e = pl.bm == 64 ? patch_vw<64, 2, 2, 4, 2, 2>(a, pl.vw, ntiles, lds_b, st)
                            : patch_vw<128, 4, 1, 7, 2, 2>(a, pl.vw, ntiles, lds_b, st);
        else
            e = pl.bm == 64 ? patch_vw<64, 2, 2, 4, 2, 1>(a, pl.vw, ntiles, lds_b, st)
                            : patch_vw<128, 4, 1, 7, 2, 1>(a, pl.vw, ntiles, lds_b, st);
    } else {
        e = pl.bm == 64 ? patch_vw<64, 2, 2, 4, 2, 0>(a, pl.vw, ntiles, lds, st)
                        : patch_vw<128, 4, 1, 7, 2, 0>(a, pl.vw, ntiles, lds, st);
    }
    return e == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
}

static int launch_patch_phases(const Plan &pl, const Problem &p, const void *dy, const void *w, float *dx,
                               void *ws, hipStream_t st, const Epi *epi) {
    PatchArgs a = {};
    const int nph = p.sh * p.sw;
    if (nph > 4) return MICONV_ERR_HIP;
    PhaseDim dh[4], dwd[4];
    int pmax_h = 0, pmin_h = 1 << 30, pmax_w = 0, pmin_w = 1 << 30;
    for (int f = 0; f < p.sh; ++f) {
        dh[f] = phase_dim(f, p.sh, p.ph, p.H, p.R);
        const int pad = dh[f].nu - 1 - dh[f].base;
        pmax_h = max(pmax_h, pad);
        pmin_h = min(pmin_h, pad);
    }
    for (int f = 0; f < p.sw; ++f) {
        dwd[f] = phase_dim(f, p.sw, p.pw, p.W, p.S);
        const int pad = dwd[f].nu - 1 - dwd[f].base;
        pmax_w = max(pmax_w, pad);
        pmin_w = min(pmin_w, pad);
    }
    const int nuh = dh[0].nu, nuw = dwd[0].nu, T = nuh * nuw;
    const int m_rows = pl.m_tiles * pl.bm;
    const int per = (m_rows / 32) * (p.K / 32) * T * 128;   // 16-byte vectors per phase
    uint16_t *wt = (uint16_t *)((char *)ws + pl.wt_offset);
    if ((size_t)per * nph * 16 != pl.wt_bytes) return MICONV_ERR_HIP;
    hipLaunchKernelGGL(filter_to_frag_phases, dim3((per * nph + 255) / 256), dim3(256), 0, st, (const uint16_t *)w, wt,
                       p.C, p.R, p.S, p.C, p.K, p.sw, p.sh, nuh, nuw, per, per * nph);
    if (hipGetLastError() != hipSuccess) return MICONV_ERR_HIP;
    a.X = dy;
    a.x_bytes = (uint32_t)((size_t)p.N * p.K * p.P * p.Q * 2);
    a.Cr = p.K; a.Hi = p.P; a.Wi = p.Q; a.M = p.C;
    a.ph = pmax_h; a.pw = pmax_w;   // the patch holds dy rows from p0 - pmax_h, columns from -pmax_w
    a.Ho = dh[0].na; a.Wo = dwd[0].na;
    a.Wt = wt;
    a.w_bytes = (uint32_t)pl.wt_bytes;
    a.O = dx;
    a.N = p.N; a.R = nuh; a.S = nuw;
    a.TR = pl.tr;
    a.row_tiles = (a.Ho + a.TR - 1) / a.TR;
    a.m_tiles = pl.m_tiles;
    a.PWc = a.Wo + nuw - 1 + (pmax_w - pmin_w);
    a.PWs = pl.pws;
    a.PR = a.TR + nuh - 1 + (pmax_h - pmin_h);
    a.G = a.Wi / pl.vw;
    a.nph = nph; a.osh = p.sh; a.osw = p.sw; a.OW = p.W; a.OHW = p.H * p.W;
    a.wt_phase = (uint32_t)per * 16;
    for (int fh = 0; fh < p.sh; ++fh)
        for (int fw = 0; fw < p.sw; ++fw) {
            const int f = fh * p.sw + fw;
            a.ph_i0[f] = dh[fh].i0;
            a.ph_j0[f] = dwd[fw].i0;
            a.ph_boff[f] = (pmax_h - (dh[fh].nu - 1 - dh[fh].base)) * a.PWs * CPB +
                           (pmax_w - (dwd[fw].nu - 1 - dwd[fw].base)) * CPB;
        }
    const int ntiles = pl.m_tiles * a.row_tiles * p.N * nph;
    const size_t lds = 2 * (size_t)a.PR * a.PWs * CPB;
    return run_patch(pl, a, ntiles, lds, st, epi);
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
// dy is read from HBM once and its latency is long next to one step's MFMAs
// (9 or 18 of them), so the dy fragments go through a register ring DA steps
// deep: step i loads the fragments of step i + DA - 1.  A second cursor walks
// the steps ahead of the current one; past the split's last band it loads
// zeros (out-of-range offsets), so every step issues the same loads.
// PAIR (64 filter rows, two bands per split): both bands' patches are
// filled first, then the two waves of each row block take one band each with
// both k16 halves of every step -- half the dependent steps per wave, twice
// the independent MFMAs per step -- and their sums are added at the end.
template <int BM, int VW, int AV, int TC, bool PAIR>
__global__ __launch_bounds__(256, 2) void bwdf_patch_kernel(BFArgs a) {
    constexpr int BC = 32, CPBF = 64, NOCT = 4, TMAX = 9;
    constexpr int WM = BM / 32, WU = PAIR ? 1 : 4 / WM, NU = 2 / WU, WB = PAIR ? 4 / WM : 1;
    static_assert(!PAIR || WB == 2, "pair mode needs two waves per row block");
    constexpr int DA = AV == 1 ? (NU == 1 ? 3 : 2) : (PAIR ? 3 : 4);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, lh = lane >> 5;
    const int wm = wave % WM, wu = PAIR ? 0 : wave / WM, wb = PAIR ? wave / WM : 0;
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

    auto band_geom = [&](int b, int &n, int &p0, int &npx) __attribute__((always_inline)) {
        n = (int)fdiv((uint32_t)b, a.fd_rb);
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
    u32x4 af[DA][NU];
    auto load_a = [&](int b, int ps, u32x4 (&dst)[NU]) {
        int n, p0, npx;
        const bool bok = b < b_end;
        band_geom(bok ? b : b_begin, n, p0, npx);
        const uint32_t rowoff = (uint32_t)(((n * a.K + krow) * a.P + p0) * a.Q);
        const bool kok = bok && krow < a.K;
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

    auto mfma_step = [&](const char *patch, int ps, int npx, const u32x4 (&A)[NU]) __attribute__((always_inline)) {
        int pos[NU][2];
#pragma unroll
        for (int uu = 0; uu < NU; ++uu) {
            const int u = WU == 2 ? wu : uu;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ip = ps * 32 + u * 16 + 8 * lh + 4 * h + (L >> 2);
                const int pr = (int)fdiv((uint32_t)ip, a.fd_Q), pc = ip - pr * a.Q;
                pos[uu][h] = (ip < npx ? (pr * a.PWs + pc) * CPBF : 0) + choff;
            }
        }
        if constexpr (TC > 0) {
            // compile-time taps: the step's NU*TC (half, tap) products in one
            // sequence, B fragments read DIST products ahead of their MFMA
            // through a small register ring (the scheduling fences keep that
            // order; left alone, each read is sunk next to its MFMA)
            constexpr int DIST = 3, NRING = DIST + 1, SW = TC == 9 ? 3 : TC, NP = NU * TC;
            const int rowb = a.PWs * CPBF;
            auto rd = [&](int j) __attribute__((always_inline)) {
                typedef short i16x4 __attribute__((ext_vector_type(4)));
                typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
                const int uu = j / TC, t = j % TC;
                const int toff = (t / SW) * rowb + (t % SW) * CPBF;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(__attribute__((address_space(3))) char *)(patch + pos[uu][0] + toff));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(__attribute__((address_space(3))) char *)(patch + pos[uu][1] + toff));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                return u32x4{l2[0], l2[1], h2[0], h2[1]};
            };
            u32x4 ring[NRING];
            static_for<0, DIST>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                if constexpr (j < NP) ring[j] = rd(j);
            });
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, NP>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                if constexpr (j + DIST < NP) ring[(j + DIST) % NRING] = rd(j + DIST);
                acc[j % TC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, A[j / TC]),
                                                                      __builtin_bit_cast(bf16x8, ring[j % NRING]),
                                                                      acc[j % TC], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            });
            return;
        }
#pragma unroll
        for (int uu = 0; uu < NU; ++uu) {
#pragma unroll
            for (int t = 0; t < TMAX; ++t) {
                if (t < T) {  // predicated, not `break`: keeps acc[] indices compile-time
                    const int toff = toffs[t];
                    typedef short i16x4 __attribute__((ext_vector_type(4)));
                    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(__attribute__((address_space(3))) char *)(patch + pos[uu][0] + toff));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(__attribute__((address_space(3))) char *)(patch + pos[uu][1] + toff));
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                    const u32x4 fb = u32x4{l2[0], l2[1], h2[0], h2[1]};
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, A[uu]), __builtin_bit_cast(bf16x8, fb), acc[t], 0, 0, 0);
                }
            }
        }
    };

    if constexpr (PAIR) {
        for (int pb0 = b_begin; pb0 < b_end; pb0 += 2) {
            __syncthreads();   // zeroing done / the previous pair's patches are no longer read
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) {
                if (pb0 + bi >= b_end) continue;
                int n, p0, npx;
                band_geom(pb0 + bi, n, p0, npx);
                FillItem<VW> f0, f1;   // both items of a band in flight
                fill_load<VW>(rx, items[0], a.C, a.H, a.W, a.ph, n, p0, c0, f0);
                fill_load<VW>(rx, items[1], a.C, a.H, a.W, a.ph, n, p0, c0, f1);
                fill_store<VW, CPBF>(smem + bi * patch_bytes, items[0], a.PWs, a.pw, f0);
                fill_store<VW, CPBF>(smem + bi * patch_bytes, items[1], a.PWs, a.pw, f1);
            }
            __syncthreads();
            const int b = pb0 + wb;
            if (b < b_end) {
                int n, p0, npx;
                band_geom(b, n, p0, npx);
                const int nps = (npx + 31) / 32;
                // dy ring DA steps deep; steps past the band load zeros
#pragma unroll
                for (int j = 0; j < DA - 1; ++j) load_a(b, j, af[j]);
                int ps = 0;
                while (ps < nps) {
                    static_for<0, DA>([&](auto cur_c) __attribute__((always_inline)) {
                        constexpr int CUR = decltype(cur_c)::value;
                        if (ps < nps) {
                            mfma_step(smem + wb * patch_bytes, ps, npx, af[CUR]);
                            __builtin_amdgcn_sched_barrier(0);
                            load_a(b, ps + DA - 1, af[(CUR + DA - 1) % DA]);
                            ++ps;
                        }
                    });
                }
            }
        }
    } else {
        // prefetch cursor: band pb, step pps of pnps
        int pb = b_begin, pps = 0, pnps = 0;
        auto advance = [&]() __attribute__((always_inline)) {
            if (++pps >= pnps) {
                pps = 0;
                ++pb;
                if (pb < b_end) {
                    int n_, p0_, npx_;
                    band_geom(pb, n_, p0_, npx_);
                    pnps = (npx_ + 31) / 32;
                }
            }
        };
        if (b_begin < b_end) {
            {
                int n_, p0_, npx_;
                band_geom(pb, n_, p0_, npx_);
                pnps = (npx_ + 31) / 32;
            }
    #pragma unroll
            for (int j = 0; j < DA - 1; ++j) {
                load_a(pb, pps, af[j]);
                advance();
            }
            __syncthreads();  // zeroing done before the fill overwrites data columns
    #pragma unroll
            for (int k = 0; k < MAXI; ++k) {
                load_item(b_begin, k);
                store_item(0, k);
            }
            __syncthreads();
        }
        // steps run over (band, pixel step); CUR selects this step's dy registers and
        // the loop is unrolled by DA so register array indices are compile-time
        int b = b_begin, ps = 0, n = 0, p0 = 0, npx = 0;
        if (b < b_end) band_geom(b, n, p0, npx);
        auto body = [&](auto cur_c) __attribute__((always_inline)) {
            constexpr int CUR = decltype(cur_c)::value;
            const int nps = (npx + 31) / 32;
            const bool last = ps + 1 == nps;
            const int nb = last ? b + 1 : b;
            const int bi = (b - b_begin) & 1;
            // the next band's patch, one fill item in flight per thread: item 0's
            // global loads in step 0 of the band, its LDS store in step FD, item 1's
            // loads in step FD and its store in step 2*FD <= nps-1.  A store comes
            // before the step's own global loads, so the wait for its data covers
            // only loads issued steps earlier.  Bands of fewer than 3 steps fill the
            // next patch at their end.
            const int FD = (nps - 1) / 2;
            const bool fill_any = b + 1 < b_end && FD > 0;
            mfma_step(smem + bi * patch_bytes, ps, npx, af[CUR]);
            __builtin_amdgcn_sched_barrier(0);
            if (fill_any && (ps == FD || ps == 2 * FD))
                store_item(bi ^ 1, ps == FD ? 0 : 1);  // that buffer was last read in band b - 1
            load_a(pb, pps, af[(CUR + DA - 1) % DA]);
            advance();
            if (fill_any && (ps == 0 || ps == FD)) load_item(b + 1, ps == 0 ? 0 : 1);
            if (last) {
                if (FD == 0 && b + 1 < b_end) {
    #pragma unroll
                    for (int k = 0; k < MAXI; ++k) {
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
            static_for<0, DA>([&](auto cur_c) __attribute__((always_inline)) {
                if (b < b_end) body(cur_c);
            });
        }
    }

    // two waves per row block: the second adds its sums to the first through LDS
    const int wsplit = WU == 2 ? wu : wb;
    if (WU == 2 || WB == 2) {
        float *red = (float *)smem;  // WM waves x 16 floats x 64 lanes per tap
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t >= T) continue;
            __syncthreads();
            if (wsplit == 1)
#pragma unroll
                for (int v = 0; v < 16; ++v) red[(wm * 16 + v) * 64 + lane] = acc[t][v];
            __syncthreads();
            if (wsplit == 0)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[t][v] += red[(wm * 16 + v) * 64 + lane];
        }
    }

    // epilogue: partial sums [z][K][T][C] (or dW [K][C][T] with a single split)
    if ((WU == 2 || WB == 2) && wsplit != 0) return;
    const int c = c0 + lr;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t >= T) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int k = m0 + wm * 32 + acc_row(v, lh);
            if (k >= a.K) continue;
            if (a.direct)
                out_store(a.out, ((size_t)k * a.C + c) * T + t, acc[t][v], a.epi, a.has_epi);
            else
                a.out[(((size_t)z * a.K + k) * T + t) * a.C + c] = acc[t][v];
        }
    }
}

template <int BM, int VW, int AV, int TC, bool PAIR = false>
static hipError_t bwdf_go(const BFArgs &a, int grid, size_t lds, hipStream_t st) {
    auto k = bwdf_patch_kernel<BM, VW, AV, TC, PAIR>;
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int BM, int TC>
static hipError_t bwdf_vw_tc(const BFArgs &a, int vw, int av, int grid, size_t lds, hipStream_t st) {
    if (vw == 8) {
        if (av == 8) return bwdf_go<BM, 8, 8, TC>(a, grid, lds, st);
        if (av == 4) return bwdf_go<BM, 8, 4, TC>(a, grid, lds, st);
        return bwdf_go<BM, 8, 1, TC>(a, grid, lds, st);
    }
    if (vw == 4) {
        if (av == 8) return bwdf_go<BM, 4, 8, TC>(a, grid, lds, st);
        if (av == 4) return bwdf_go<BM, 4, 4, TC>(a, grid, lds, st);
        return bwdf_go<BM, 4, 1, TC>(a, grid, lds, st);
    }
    if (av == 8) return bwdf_go<BM, 2, 8, TC>(a, grid, lds, st);
    if (av == 4) return bwdf_go<BM, 2, 4, TC>(a, grid, lds, st);
    return bwdf_go<BM, 2, 1, TC>(a, grid, lds, st);
}

// 3x3 filters get the compile-time-tap form (TC = 9), other sizes the runtime one
// 64 filter rows, 3x3, two bands per split: the pair form
static hipError_t bwdf_pair(const BFArgs &a, int vw, int av, int grid, size_t lds, hipStream_t st) {
    if (vw == 8) return av == 8 ? bwdf_go<64, 8, 8, 9, true>(a, grid, lds, st) : (av == 4 ? bwdf_go<64, 8, 4, 9, true>(a, grid, lds, st) : bwdf_go<64, 8, 1, 9, true>(a, grid, lds, st));
    if (vw == 4) return av == 8 ? bwdf_go<64, 4, 8, 9, true>(a, grid, lds, st) : (av == 4 ? bwdf_go<64, 4, 4, 9, true>(a, grid, lds, st) : bwdf_go<64, 4, 1, 9, true>(a, grid, lds, st));
    return av == 8 ? bwdf_go<64, 2, 8, 9, true>(a, grid, lds, st) : (av == 4 ? bwdf_go<64, 2, 4, 9, true>(a, grid, lds, st) : bwdf_go<64, 2, 1, 9, true>(a, grid, lds, st));
}

template <int BM>
static hipError_t bwdf_vw(const BFArgs &a, int vw, int av, int grid, size_t lds, hipStream_t st) {
    if (a.R == 3 && a.S == 3) return bwdf_vw_tc<BM, 9>(a, vw, av, grid, lds, st);
    return bwdf_vw_tc<BM, 0>(a, vw, av, grid, lds, st);
}

int launch_bwdf_patch(const Plan &pl, const Problem &p, const void *x, const void *dy, float *dw, void *ws,
                      hipStream_t st, const Epi *epi) {
    if (pl.k16) return launch_bwdf16(pl, p, x, dy, dw, ws, st, epi);
    BFArgs a = {};
    if (epi) a.epi = *epi;
    a.has_epi = epi ? 1 : 0;
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
    a.fd_rb = make_fdiv((uint32_t)a.row_bands);
    float *part = pl.splits > 1 ? (float *)((char *)ws + pl.part_offset) : dw;
    a.out = part;
    size_t lds = 2 * (size_t)a.PR * a.PWs * 64;                         // two patch buffers
    if (lds < (size_t)2 * 16 * 64 * 4) lds = (size_t)2 * 16 * 64 * 4;  // epilogue reduction buffer
    const int grid = pl.m_tiles * pl.n_tiles * pl.splits;
    const int av = (p.P * p.Q) % 8 == 0 && (pl.tr * p.Q) % 8 == 0 ? 8 : ((p.P * p.Q) % 4 == 0 && (pl.tr * p.Q) % 4 == 0 ? 4 : 1);
    hipError_t e;
    if (pl.pair)
        e = bwdf_pair(a, pl.vw, av, grid, lds, st);
    else
        e = pl.bm == 64 ? bwdf_vw<64>(a, pl.vw, av, grid, lds, st) : bwdf_vw<128>(a, pl.vw, av, grid, lds, st);
    if (e != hipSuccess) return MICONV_ERR_HIP;
    if (pl.splits > 1) return launch_splitk_reduce(part, dw, p.K, p.C, p.R * p.S, pl.splits, st, epi);
    return MICONV_OK;
}

}  // namespace miconv
