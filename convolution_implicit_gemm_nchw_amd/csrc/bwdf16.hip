// bwdf16.hip -- stride-1 bf16 backward-filter for 3x3 filters on v_mfma_f32_16x16x32_bf16.
//
//   dW[k, c, t] = sum over output pixels (n, p, q) of dy[n, k, p, q] * x~(n, c, p - ph + r, q - pw + s),
//   t = r*3 + s.
//
// Work-group tile: BM filter rows (k) x 32 channels x all 9 taps, over a contiguous
// range of bands (whole output rows of one image, at most 224 pixels): one split
// of the pixel reduction.  Four waves: 2 row halves x 2 channel halves (16
// channels each); a wave keeps BM/32 row blocks x 9 taps of 16x16 accumulators.
//
// x: per band the input rows (band + 2 halo rows) are loaded once (16/8/4-byte
// row loads, 8x8 register transposes) into an LDS patch split into two
// 16-channel sub-patches, [half][row][col][16 channels], 32 bytes per position.
// The MFMA B fragment (8 pixels of one channel per lane) comes from two
// transposing reads (ds_read_b64_tr_b16: 16 lanes read 4 positions x 16 channels
// and receive 16 channels x 4 positions), so any tap shift is a plain address
// offset.  The 32 pixels of one reduction step are assigned to MFMA k-slots so
// that the two 16-lane groups of one read pass cover 8 consecutive positions of
// one sub-patch: lane group g holds pixels 4g..4g+3 and 16+4g..16+4g+3 of the
// step.  With 32-byte positions and a row stride congruent to Q (mod 8), 8
// consecutive pixels fall on 8 distinct 32-byte bank groups, row wraps included.
// Two patch buffers: the next band is filled while this one is in use.
//
// dy: staged through LDS one 32-pixel step at a time.  The work-group loads the
// BM rows x 32 pixels of a step as 8-byte pieces of 4 pixels, each wave 8 whole
// rows per load (each 64-lane load touches 8 rows, not 16 or 32 as
// fragment-shaped loads would, and no two waves load the same rows), NSTG steps
// ahead into registers (3 with 64 rows, 2 with 128 rows, for the register
// budget), and writes them NSTG - 1 steps later into one of two LDS slots.  A
// slot row is 80 bytes with the pieces reordered (piece p at byte
// 16*(p mod 4) + 8*(p / 4)), so the 8 pixels of one lane's MFMA A fragment
// (pixels 4g..4g+3 and 16+4g..16+4g+3) are one 16-byte read.  With 80-byte rows
// the fragment reads of consecutive rows, and the piece writes of the lane order
// chosen here (row = lane mod 8, piece bits from lanes 16, 32 and 8), fall on
// distinct banks in every group of lanes the LDS serves together.  Every wave
// reads its A fragments after the step's barrier.
//
// Schedule: bands of at most 7 steps, every step unrolled, so every load,
// store and wait sits at a compile-time position (the compiler's load-counter
// waits are exact).  A step's dy loads (for NSTG steps later) are issued before
// its MFMAs and written to LDS at the end of the next step.  The x fill of the
// next band loads item 0 in step 0 and stores
// it in step 3, loads item 1 in step 3 and stores it in step 6 (the last band
// refills the idle buffer); NSTG bands per loop iteration keep each step's
// staging set (global step mod NSTG) a compile-time constant.  A short band (the
// last rows of an image) skips the MFMAs of its missing steps but issues the
// same loads (zeros past its pixels).
//
// Output: partial sums [z][K][9][C] (split-K, reduced in a fixed order by the
// split-K reduce kernels), or dW [K][C][3][3] directly with one split.
#include "device.h"
#include "launch.h"
#include "patch_common.h"

namespace miconv {

namespace {

constexpr int kTaps = 9;
constexpr int kSteps = 7;     // steps of 32 pixels per band, at most
constexpr int kDyRow = 80;    // LDS bytes per staged dy row (64 data + 16 pad)

// Stores one fill item (8 channels x VW columns of one input row, transposed)
// into the split patch: octet o goes to sub-patch o/2, bytes (o%2)*16 of each
// 32-byte position.
template <int VW>
DEVI void fill_store_halves(char *patch, const ItemPos &q, int PWs, int pw, int half_bytes, const FillItem<VW> &f) {
    if (!q.ok) return;
    char *dst = patch + (q.o >> 1) * half_bytes + ((q.pr * PWs + pw + q.g * VW) * 32 + (q.o & 1) * 16);
#pragma unroll
    for (int i = 0; i < VW; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_amdgcn_perm(f.d[2 * e + 1][i >> 1], f.d[2 * e][i >> 1], sel);
        *(u32x4 *)(dst + i * 32) = v;
    }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

DEVI u32x2 tr_read(const char *p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(__attribute__((address_space(3))) char *)p);
    return __builtin_bit_cast(u32x2, v);
}

// The finished tile of a backward-filter work-group: the lane's accumulators acc[i][t][v]
// hold filter row k0 + 16i + v, tap t, channel c.  Partial sums go to [z][K][9][C]; with
// one split dW [K][C][3][3] is written through the output epilogue.  Element offsets are
// 32-bit (every buffer is below 2 GiB) and come from one product per lane plus uniform
// strides, not a 64-bit multiply per store.
template <int TMB, bool EPI>
DEVI void store_dw_tile(const BFArgs &a, const f32x4 (&acc)[TMB][kTaps], int z, int k0, int c) {
    constexpr int T = kTaps;
    if (a.direct) {
        const uint32_t base = (uint32_t)(k0 * a.C + c) * T, kstride = (uint32_t)a.C * T;
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int i = 0; i < TMB; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    if (k0 + 16 * i + v >= a.K) continue;
                    out_store(a.out, base + (uint32_t)(16 * i + v) * kstride + t, acc[i][t][v], a.epi, EPI);
                }
    } else {
        const uint32_t kstride = (uint32_t)T * a.C;
        const uint32_t base = ((uint32_t)z * a.K + k0) * kstride + c;
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int i = 0; i < TMB; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    if (k0 + 16 * i + v >= a.K) continue;
                    a.out[base + (uint32_t)(16 * i + v) * kstride + (uint32_t)(t * a.C)] = acc[i][t][v];
                }
    }
}

}  // namespace

// EPI: a direct (one-split) write goes through the output epilogue (a.epi).
template <int BM, int VW, bool EPI>
__global__ __launch_bounds__(256, 2) void bwdf16_kernel(BFArgs a) {
    constexpr int T = kTaps, BC = 32, NPS = kSteps, FD = (NPS - 1) / 2;
    constexpr int TMB = BM / 32;            // 16-row blocks per wave
    constexpr int NLD = BM / 32;            // 8-byte dy pieces per thread per step
    // dy staging sets (steps of load-to-LDS-write distance + 1) and bands per loop
    // iteration; the 128-row form keeps two to stay within 256 registers
    constexpr int NSTG = BM == 64 ? 3 : 2, DA = NSTG;
    constexpr bool EARLY = BM == 64 || VW == 2;   // dy loads issued before the step's MFMAs
    constexpr int SLOT = BM * kDyRow;       // bytes of one dy slot
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int L = lane & 15, g = lane >> 4;
    const int wk = wave & 1, wc = wave >> 1;   // row half, channel half

    const int tiles = a.m_tiles * a.c_tiles;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int z = logical / tiles, tile = logical - z * tiles;
    const int m0 = (tile % a.m_tiles) * BM, c0 = (tile / a.m_tiles) * BC;
    const int total_bands = a.N * a.row_bands;
    const int b_begin = z * a.bands_per_split, b_end = min(total_bands, b_begin + a.bands_per_split);
    const int half_bytes = a.PR * a.PWs * 32;
    const int patch_bytes = 2 * half_bytes;
    char *dys = smem + 2 * patch_bytes;   // two dy slots
    const rsrc_t rx = make_rsrc(a.X, a.x_bytes), rdy = make_rsrc(a.DY, a.dy_bytes);

    for (int o = tid * 16; o < 2 * patch_bytes; o += 256 * 16) *(u32x4 *)(smem + o) = u32x4{0, 0, 0, 0};

    auto band_geom = [&](int b, int &n, int &p0, int &npx) __attribute__((always_inline)) {
        n = (int)fdiv((uint32_t)b, a.fd_rb);
        p0 = (b - n * a.row_bands) * a.TR;
        npx = min(a.TR, a.P - p0) * a.Q;
    };

    // x patch fill
    const int nitems = 4 * a.PR * a.G;
    ItemPos items[MAXI];
#pragma unroll
    for (int k = 0; k < MAXI; ++k) items[k] = item_pos(tid + k * 256, nitems, a.G, a.PR);
    FillItem<VW> fi;   // one fill item in flight per thread
    auto load_item = [&](int b, int k) __attribute__((always_inline)) {
        int n, p0, npx;
        band_geom(b, n, p0, npx);
        fill_load<VW>(rx, k == 0 ? items[0] : items[1], a.C, a.H, a.W, a.ph, n, p0, c0, fi);
    };
    auto store_item = [&](int buf, int k) __attribute__((always_inline)) {
        fill_store_halves<VW>(smem + buf * patch_bytes, k == 0 ? items[0] : items[1], a.PWs, a.pw, half_bytes, fi);
    };

    // dy staging: piece j of this thread is row j*32 + srow, pixels 4*spiece .. +3 of the step;
    // wave w takes rows 8w .. 8w+7 (lane mod 8) and piece (lane/16 mod 4) + 4*(lane/8 mod 2)
    const int srow = ((tid >> 6) << 3) | (tid & 7), spiece = ((tid >> 4) & 3) | (((tid >> 3) & 1) << 2);
    u32x2 stg[NSTG][NLD];
    auto load_dy = [&](int b, int ps, u32x2 (&dst)[NLD]) __attribute__((always_inline)) {
        int n, p0, npx;
        const bool bok = b < b_end;
        band_geom(bok ? b : b_begin, n, p0, npx);
        const int px = ps * 32 + 4 * spiece;
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int krow = m0 + j * 32 + srow;
            const bool ok = bok && krow < a.K && px < npx;
            dst[j] = ld_b64(rdy, ok ? (uint32_t)((((n * a.K + krow) * a.P + p0) * a.Q + px) * 2) : kOOB);
        }
    };
    auto write_dy = [&](int slot, const u32x2 (&src)[NLD]) __attribute__((always_inline)) {
        char *base = dys + slot * SLOT + srow * kDyRow + (spiece & 3) * 16 + (spiece >> 2) * 8;
#pragma unroll
        for (int j = 0; j < NLD; ++j) *(u32x2 *)(base + j * 32 * kDyRow) = src[j];
    };
    // A fragment i: row wk*(BM/2) + 16i + L, pixels 4g..4g+3 (piece g) and 16+4g..+3 (piece 4+g),
    // stored next to each other at byte 16g of the row
    u32x4 A[TMB];
    auto read_a = [&](int slot) __attribute__((always_inline)) {
        const char *base = dys + slot * SLOT + (wk * (BM / 2) + L) * kDyRow + g * 16;
#pragma unroll
        for (int i = 0; i < TMB; ++i) A[i] = *(const u32x4 *)(base + 16 * i * kDyRow);
    };

    f32x4 acc[TMB][T];
#pragma unroll
    for (int i = 0; i < TMB; ++i)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][t][v] = 0.0f;

    const int choff = wc * half_bytes + 8 * (L & 3);
    const int rowb = a.PWs * 32;

    // One reduction step (32 pixels): 9 taps x TMB row blocks of MFMAs; the B
    // fragment of tap t + 2 is read while the MFMAs of tap t run (a small register
    // ring; the scheduling fences keep that order).
    auto mfma_step = [&](const char *patch, int ps, int npx) __attribute__((always_inline)) {
        int pos[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ip = ps * 32 + 4 * g + 16 * h + (L >> 2);
            const int pr = (int)fdiv((uint32_t)ip, a.fd_Q), pc = ip - pr * a.Q;
            pos[h] = (ip < npx ? (pr * a.PWs + pc) * 32 : 0) + choff;
        }
        constexpr int DIST = BM == 64 ? 2 : 1, NRING = DIST + 1;   // B reads this many taps ahead
        auto rd = [&](int t) __attribute__((always_inline)) {
            const int toff = (t / 3) * rowb + (t % 3) * 32;
            const u32x2 lo = tr_read(patch + pos[0] + toff), hi = tr_read(patch + pos[1] + toff);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        u32x4 ring[NRING];
        static_for<0, DIST>([&](auto tc) __attribute__((always_inline)) {
            constexpr int t = decltype(tc)::value;
            ring[t] = rd(t);
        });
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, T>([&](auto tc) __attribute__((always_inline)) {
            constexpr int t = decltype(tc)::value;
            if constexpr (t + DIST < T) ring[(t + DIST) % NRING] = rd(t + DIST);
#pragma unroll
            for (int i = 0; i < TMB; ++i)
                acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[i]),
                                                                   __builtin_bit_cast(bf16x8, ring[t % NRING]),
                                                                   acc[i][t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // prologue: steps 0 .. NSTG-1 into staging sets 0 .. NSTG-1, step 0 written to
    // slot 0, the first band's patch into buffer 0
    if (b_begin < b_end) {
#pragma unroll
        for (int j = 0; j < NSTG; ++j) load_dy(b_begin, j, stg[j]);
        __syncthreads();   // zeroing done before the fill overwrites data columns
        write_dy(0, stg[0]);
#pragma unroll
        for (int k = 0; k < MAXI; ++k) {
            load_item(b_begin, k);
            store_item(0, k);
        }
        __syncthreads();
    }
    // global step gs = (b - b_begin)*NPS + st: A from slot gs % 2; the staging set of
    // step gs + 1 (loaded NSTG - 1 steps ago) is written to slot (gs + 1) % 2, and the
    // set of step gs (written a step ago) is reloaded with step gs + NSTG
    for (int b0 = b_begin; b0 < b_end; b0 += DA) {
        static_for<0, DA>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const int b = b0 + j;
            if (b < b_end) {
                int n, p0, npx;
                band_geom(b, n, p0, npx);
                const int nps = (npx + 31) / 32;
                const int bi = (b - b_begin) & 1;
                const int bf = b + 1 < b_end ? b + 1 : b;   // the last band refills the idle buffer
                const int gs0 = (b - b_begin) * NPS;
                static_for<0, NPS>([&](auto sc) __attribute__((always_inline)) {
                    constexpr int st = decltype(sc)::value;
                    constexpr int WSET = (j * NPS + st + 1) % NSTG, LSET = (j * NPS + st) % NSTG;
                    constexpr int BO = (st + NSTG) / NPS, SS = (st + NSTG) % NPS;
                    const int gs = gs0 + st;
                    read_a(gs & 1);
                    // set LSET (step gs, already in LDS) is free: load step gs + NSTG into it
                    // before this step's MFMAs, so the loads have most of two steps to land
                    // (after them in the 128-row form with 4-column fill items, whose
                    // registers do not allow the longer lifetime)
                    if constexpr (EARLY) load_dy(b + BO, SS, stg[LSET]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (st < nps) mfma_step(smem + bi * patch_bytes, st, npx);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (st == FD) store_item(bi ^ 1, 0);
                    if constexpr (st == 2 * FD) store_item(bi ^ 1, 1);
                    write_dy((gs + 1) & 1, stg[WSET]);
                    if constexpr (!EARLY) load_dy(b + BO, SS, stg[LSET]);
                    if constexpr (st == 0) load_item(bf, 0);
                    if constexpr (st == FD) load_item(bf, 1);
                    __builtin_amdgcn_sched_barrier(0);
                    __syncthreads();   // step gs+1's dy visible, slot gs free; at a band end
                                       // also the next patch complete and this one free
                });
            }
        });
    }

    // epilogue: lane holds channel c0 + wc*16 + L and filter rows m0 + wk*BM/2 + 16i + 4g + v
    store_dw_tile<TMB, EPI>(a, acc, z, m0 + wk * (BM / 2) + 4 * g, c0 + wc * 16 + L);
}

// Stream form (bands are whole images): the split's images form one stream of
// pixels, consumed 32 per step whatever the image boundaries, so no step is
// padded at the end of an image (14x14 images: 196 steps per 32 images rather
// than 224).  A lane's 4-pixel group lies in one image (P*Q is a multiple of 4);
// its B reads address that image's patch buffer (image i of the split in buffer
// i mod 2).  The patch of image i + 2 is filled into the buffer of image i in the
// two steps after the last step that reads image i (one fill item per step,
// loaded and stored within the step); the host checks that every image's patch
// is complete two steps before its first step.  dy goes through three LDS slots:
// step s's loads are of step s + 3 and its slot write is of step s + 2, so the A
// fragments of step s + 1 are read during step s.  The B-read ring runs on
// across step boundaries (the next step's first taps are read during the last
// taps of this one).
template <int BM, int VW, bool EPI>
__global__ __launch_bounds__(256, 2) void bwdf16s_kernel(BFArgs a) {
    constexpr int T = kTaps, BC = 32;
    constexpr int TMB = BM / 32;            // 16-row blocks per wave
    constexpr int NLD = BM / 32;            // 8-byte dy pieces per thread per step
    constexpr int SLOT = BM * kDyRow;       // bytes of one dy slot
    constexpr int DIST = 2, NRING = 3;      // B reads this many taps ahead; T % NRING == 0
    static_assert(T % NRING == 0, "ring slots are tap-indexed");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int L = lane & 15, g = lane >> 4;
    const int wk = wave & 1, wc = wave >> 1;   // row half, channel half

    const int tiles = a.m_tiles * a.c_tiles;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int z = logical / tiles, tile = logical - z * tiles;
    const int m0 = (tile % a.m_tiles) * BM, c0 = (tile / a.m_tiles) * BC;
    const int n_begin = z * a.bands_per_split, nimg = min(a.N, n_begin + a.bands_per_split) - n_begin;
    const int PQ = a.P * a.Q;
    const int total = nimg * PQ, nsteps = (total + 31) / 32;
    const int half_bytes = a.PR * a.PWs * 32;
    const int patch_bytes = 2 * half_bytes;
    char *dys = smem + 2 * patch_bytes;   // three dy slots
    const rsrc_t rx = make_rsrc(a.X, a.x_bytes), rdy = make_rsrc(a.DY, a.dy_bytes);

    for (int o = tid * 16; o < 2 * patch_bytes; o += 256 * 16) *(u32x4 *)(smem + o) = u32x4{0, 0, 0, 0};

    // x patch fill: image i (of the split) into buffer i mod 2
    const int nitems = 4 * a.PR * a.G;
    ItemPos items[MAXI];
#pragma unroll
    for (int k = 0; k < MAXI; ++k) items[k] = item_pos(tid + k * 256, nitems, a.G, a.PR);
    FillItem<VW> fi;
    auto load_item = [&](int img, int k) __attribute__((always_inline)) {
        fill_load<VW>(rx, k == 0 ? items[0] : items[1], a.C, a.H, a.W, a.ph, n_begin + img, 0, c0, fi);
    };
    auto store_item = [&](int img, int k) __attribute__((always_inline)) {
        fill_store_halves<VW>(smem + (img & 1) * patch_bytes, k == 0 ? items[0] : items[1], a.PWs, a.pw,
                              half_bytes, fi);
    };

    // dy staging: piece j of this thread is row j*32 + srow, stream pixels 4*spiece .. +3 of the
    // step (one image: P*Q is a multiple of 4)
    const int srow = ((tid >> 6) << 3) | (tid & 7), spiece = ((tid >> 4) & 3) | (((tid >> 3) & 1) << 2);
    u32x2 stg[2][NLD];
    // The steps are loaded in order, 32 pixels apart, and an image holds more than 32 pixels
    // (the plan's fill schedule needs P*Q >= 96), so the next step's position follows from the
    // last with one wrap at most: sp (stream pixel), pix (its pixel in the image) and doff
    // (dy element of row m0 + srow there) advance by additions, not divisions.
    int sp = 4 * spiece, pix = sp;
    uint32_t doff = (uint32_t)(((n_begin * a.K + m0 + srow) * PQ) + sp);
    const uint32_t img_step = (uint32_t)((a.K - 1) * PQ);   // dy elements from one image's row to the next's
    auto load_dy = [&](u32x2 (&dst)[NLD]) __attribute__((always_inline)) {
        const bool pok = sp < total;
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const bool ok = pok && m0 + j * 32 + srow < a.K;
            dst[j] = ld_b64(rdy, ok ? (doff + (uint32_t)(j * 32 * PQ)) * 2 : kOOB);
        }
        sp += 32;
        pix += 32;
        doff += 32;
        if (pix >= PQ) {
            pix -= PQ;
            doff += img_step;
        }
    };
    auto write_dy = [&](int slot, const u32x2 (&src)[NLD]) __attribute__((always_inline)) {
        char *base = dys + slot * SLOT + srow * kDyRow + (spiece & 3) * 16 + (spiece >> 2) * 8;
#pragma unroll
        for (int j = 0; j < NLD; ++j) *(u32x2 *)(base + j * 32 * kDyRow) = src[j];
    };
    u32x4 A[2][TMB];
    auto read_a = [&](int slot, u32x4 (&dst)[TMB]) __attribute__((always_inline)) {
        const char *base = dys + slot * SLOT + (wk * (BM / 2) + L) * kDyRow + g * 16;
#pragma unroll
        for (int i = 0; i < TMB; ++i) dst[i] = *(const u32x4 *)(base + 16 * i * kDyRow);
    };

    f32x4 acc[TMB][T];
#pragma unroll
    for (int i = 0; i < TMB; ++i)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][t][v] = 0.0f;

    // B positions of a step: the two 4-pixel groups of this lane (pixels 4g + 16h + L/4).
    // Steps are taken in order and an image holds more than 32 pixels, so group 0 advances
    // 32 pixels per step, and group 1 lies 16 pixels after group 0, each with at most one
    // column wrap and one image wrap: ip (stream pixel), pr / pc (row, column) and core (its
    // patch byte offset, the image's buffer included) follow by additions.
    const int choff = wc * half_bytes + 8 * (L & 3);
    const int rowb = a.PWs * 32;
    const int d32 = 32 / a.Q, r32 = 32 % a.Q, d16 = 16 / a.Q, r16 = 16 % a.Q;
    const int wrap_col = (a.PWs - a.Q) * 32, img_rows = a.P * rowb;
    int ip = 4 * g + (L >> 2), pr = (int)fdiv((uint32_t)ip, a.fd_Q), pc = ip - pr * a.Q;
    int core = pr * rowb + pc * 32;
    auto positions = [&](int (&pos)[2]) __attribute__((always_inline)) {
        // group 1: 16 pixels on
        int pc1 = pc + r16, pr1 = pr + d16, core1 = core + d16 * rowb + r16 * 32;
        if (pc1 >= a.Q) {
            pc1 -= a.Q;
            ++pr1;
            core1 += wrap_col;
        }
        if (pr1 >= a.P) core1 += core >= patch_bytes ? -img_rows - patch_bytes : patch_bytes - img_rows;
        pos[0] = (ip < total ? core : 0) + choff;
        pos[1] = (ip + 16 < total ? core1 : 0) + choff;
        // group 0 of the next step
        ip += 32;
        pc += r32;
        pr += d32;
        core += d32 * rowb + r32 * 32;
        if (pc >= a.Q) {
            pc -= a.Q;
            ++pr;
            core += wrap_col;
        }
        if (pr >= a.P) {
            pr -= a.P;
            core += core >= patch_bytes ? -img_rows - patch_bytes : patch_bytes - img_rows;
        }
    };
    auto rd = [&](const int (&pos)[2], int t) __attribute__((always_inline)) {
        const int toff = (t / 3) * rowb + (t % 3) * 32;
        const u32x2 lo = tr_read(smem + pos[0] + toff), hi = tr_read(smem + pos[1] + toff);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };

    // first step at which image `img` may be filled: after the last step that reads image img - 2
    auto fill_from = [&](int img) __attribute__((always_inline)) { return ((img - 1) * PQ - 1) / 32 + 1; };

    // prologue: images 0 and 1 into buffers 0 and 1, dy steps 0 and 1 into slots 0 and 1,
    // step 2 into staging set 0, A of step 0 into set 0, the ring's first taps
    load_dy(stg[0]);
    load_dy(stg[1]);
    __syncthreads();   // zeroing done before the fill overwrites data columns
#pragma unroll
    for (int img = 0; img < 2; ++img)
#pragma unroll
        for (int k = 0; k < MAXI; ++k) {
            load_item(img, k);
            store_item(img, k);
        }
    write_dy(0, stg[0]);
    write_dy(1, stg[1]);
    load_dy(stg[0]);
    __syncthreads();
    read_a(0, A[0]);
    int pos[2], pos_n[2];
    positions(pos);
    u32x4 ring[NRING];
    ring[0] = rd(pos, 0);
    ring[1] = rd(pos, 1);
    int fimg = 2, fitem = 0, fstep = fill_from(2);

    // step s: loads of step s + 3 into staging set (s + 1) & 1, A of step s + 1 into set
    // (s + 1) & 1, MFMAs with A set s & 1, staging set s & 1 (step s + 2) to slot (s + 2) % 3
    auto step = [&](auto par_c, int s) __attribute__((always_inline)) {
        constexpr int P = decltype(par_c)::value;   // s & 1
        const bool fill = fimg < nimg && s >= fstep;
        if (fill) load_item(fimg, fitem);
        load_dy(stg[P ^ 1]);   // step s + 3
        read_a((s + 1) % 3, A[P ^ 1]);
        positions(pos_n);      // step s + 1
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, T>([&](auto tc) __attribute__((always_inline)) {
            constexpr int t = decltype(tc)::value;
            if constexpr (t + DIST < T)
                ring[(t + DIST) % NRING] = rd(pos, t + DIST);
            else
                ring[(t + DIST) % NRING] = rd(pos_n, t + DIST - T);
#pragma unroll
            for (int i = 0; i < TMB; ++i)
                acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[P][i]),
                                                                   __builtin_bit_cast(bf16x8, ring[t % NRING]),
                                                                   acc[i][t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
        if (fill) {
            store_item(fimg, fitem);
            if (++fitem == MAXI) {
                fitem = 0;
                ++fimg;
                fstep = fill_from(fimg);
            }
        }
        write_dy((s + 2) % 3, stg[P]);
        pos[0] = pos_n[0];
        pos[1] = pos_n[1];
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();   // step s + 1's A and next fills visible; slot s free
    };
    for (int s = 0; s < nsteps; s += 2) {
        step(std::integral_constant<int, 0>(), s);
        if (s + 1 < nsteps) step(std::integral_constant<int, 1>(), s + 1);
    }

    // epilogue: lane holds channel c0 + wc*16 + L and filter rows m0 + wk*BM/2 + 16i + 4g + v
    store_dw_tile<TMB, EPI>(a, acc, z, m0 + wk * (BM / 2) + 4 * g, c0 + wc * 16 + L);
}

template <int BM, int VW>
static hipError_t bwdf16_go(const BFArgs &a, int grid, size_t lds, hipStream_t st, bool stream) {
    const bool epi = a.has_epi && a.direct;
    auto k = epi ? bwdf16_kernel<BM, VW, true> : bwdf16_kernel<BM, VW, false>;
    if (stream) {
        // the 128-row stream form takes 4-byte fill loads only (register budget)
        if constexpr (BM == 128 && VW != 2) return hipErrorInvalidValue;
        else k = epi ? bwdf16s_kernel<BM, VW, true> : bwdf16s_kernel<BM, VW, false>;
    }
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int BM>
static hipError_t bwdf16_vw(const BFArgs &a, int vw, int grid, size_t lds, hipStream_t st, bool stream) {
    if (vw == 8) {   // the plan gives the 128-row form column groups of 4 or 2
        if constexpr (BM == 64) return bwdf16_go<BM, 8>(a, grid, lds, st, stream);
        return hipErrorInvalidValue;
    }
    if (vw == 4) return bwdf16_go<BM, 4>(a, grid, lds, st, stream);
    return bwdf16_go<BM, 2>(a, grid, lds, st, stream);
}

int launch_bwdf16(const Plan &pl, const Problem &p, const void *x, const void *dy, float *dw, void *ws,
                  hipStream_t st, const Epi *epi) {
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
    a.fd_PQ = make_fdiv((uint32_t)(p.P * p.Q));
    float *part = pl.splits > 1 ? (float *)((char *)ws + pl.part_offset) : dw;
    a.out = part;
    const bool stream = pl.stream != 0;
    if (stream && pl.tr != p.P) return MICONV_ERR_HIP;   // the stream form takes whole images
    const size_t lds = stream ? bwdf16s_lds_bytes(pl.bm, a.PR, a.PWs) : bwdf16_lds_bytes(pl.bm, a.PR, a.PWs);
    const int grid = pl.m_tiles * pl.n_tiles * pl.splits;
    hipError_t e = pl.bm == 64 ? bwdf16_vw<64>(a, pl.vw, grid, lds, st, stream)
                               : bwdf16_vw<128>(a, pl.vw, grid, lds, st, stream);
    if (e != hipSuccess) return MICONV_ERR_HIP;
    if (pl.splits > 1) return launch_splitk_reduce(part, dw, p.K, p.C, p.R * p.S, pl.splits, st, epi);
    return MICONV_OK;
}

}  // namespace miconv
