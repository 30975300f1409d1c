// pointwise.hip -- 1x1 bf16 convolution with zero padding 0 and stride s in {1, 2}:
// forward and backward-data as one GEMM per image, on v_mfma_f32_16x16x32_bf16.
//
//   forward        y[n,k,p,q]        = sum_c W[k,c] * x[n,c,s*p,s*q]
//   backward-data  dx[n,c,s*p,s*q]   = sum_k W[k,c] * dy[n,k,p,q],
//                  dx = 0 at every position whose row or column is not a multiple of s
//                  (H = s*P and W = s*Q here, so every dx position is one of the two kinds).
//
// Common form: out[n][m][pix] = sum_r A[m][r] * B[n][r][pix], where
//   forward:        A = W [K][C] (m = k, r = c), B = x subsampled by s, out = y;
//   backward-data:  A = W^T [C][K] (a transposed copy in the workspace), B = dy, out = dx
//                   written in whole rows with the zeros interleaved.
//
// Work-group tile: 256 output channels (m) x TR whole output rows of one image
// (NB blocks of 16 pixels, at most 8).  Four waves of 64 rows (four 16-row blocks)
// x all NB pixel blocks: each B fragment read from LDS feeds four MFMAs.  Tiles
// this tall make each B tile and each A chunk travel through L1 as few times as
// the 256-register budget allows (x is read by ceil(M/256) work-groups, the
// filter once per pixel tile).
// The reduction runs in chunks of 32 r-channels; both operands of a chunk are
// staged in LDS (two stages), and the loads run two chunks ahead through two
// register staging sets.  Every load has consecutive lanes on consecutive bytes
// of a row:
//   B: 16-byte (stride 2) or 8-byte (stride 1) row loads; the stride-2 columns are
//   picked by byte permutes and the pixels stored per channel ([32 ch][pixels],
//   288-byte rows).  The MFMA B fragment (8 channels of one pixel per lane) comes
//   from two transposing reads (ds_read_b64_tr_b16: 16 lanes read 4 channels x 16
//   pixels and receive 16 pixels x 4 channels).
//   A: the chunk's 256 rows x 32 channels, 16-byte loads, 80-byte LDS rows.
// MFMA k-slots: lane group g holds channels 4g..4g+3 and 16+4g..16+4g+3 of the
// chunk, so one read pass (two lane groups) touches 8 consecutive channel rows of
// B, which a 288-byte row stride spreads over 8 distinct 32-byte bank groups; the
// A reads of 16 rows at an 80-byte stride are conflict-free too.
// Output: the finished tile is staged in LDS and written row span by row span with
// 16-byte stores (a channel's rows of one tile are contiguous in memory); backward-
// data writes (value, 0, value, 0) on the even rows and zeros on the odd rows, so
// every byte of dx is written exactly once.
#include "device.h"
#include "launch.h"
#include "patch_common.h"

namespace miconv {

namespace {

constexpr int kRows = 256;        // output channels (m) per work-group tile
constexpr int kChunk = 32;        // reduction channels per chunk (one MFMA k-step)
constexpr int kRowStride = 288;   // LDS bytes per channel row of the B chunk (<= 128 pixels)
constexpr int kARow = 80;         // LDS bytes per row of the A chunk (32 channels + pad)
constexpr int kABytes = kRows * kARow, kBBytes = kChunk * kRowStride;
constexpr int kStageBytes = kABytes + kBBytes;   // one stage: A chunk then B chunk

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

DEVI u32x2 tr_read(const char *p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(__attribute__((address_space(3))) char *)p);
    return __builtin_bit_cast(u32x2, v);
}

// Transposed copy of a 1x1 filter: wt[c][k] = w[k][c] (bf16), through a 32 x 32 LDS tile.
__global__ __launch_bounds__(256) void pw_transpose(const uint16_t *__restrict__ w, uint16_t *__restrict__ wt, int K,
                                                    int C) {
    __shared__ uint16_t t[32][34];
    const int k0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int r = ty; r < 32; r += 8)
        if (k0 + r < K && c0 + tx < C) t[r][tx] = w[(size_t)(k0 + r) * C + c0 + tx];
    __syncthreads();
    for (int r = ty; r < 32; r += 8)
        if (c0 + r < C && k0 + tx < K) wt[(size_t)(c0 + r) * K + k0 + tx] = t[tx][r];
}

}  // namespace

struct PWArgs {
    const void *A;        // [M][Rc] bf16 row-major
    const void *B;        // [N][Rc][Hi][Wi] bf16
    float *O;             // forward: [N][M][Ho][Wo]; backward-data: [N][M][s*Ho][s*Wo]
    uint32_t a_bytes, b_bytes;
    int N, M, Rc, Hi, Wi, Ho, Wo, s;
    int TR, row_tiles, m_tiles;
    Epi epi;
};

// BWD: backward-data (zeros interleaved in the output); S: input subsampling stride
// of B (forward only); NB: 16-pixel blocks per tile; EPI: fused forward epilogue.
// Four consecutive outputs O[o .. o+3] of output row m (16-byte aligned; 8 bytes
// for bf16): stored as they are (EPI 0), or through the epilogue
// act(alpha * v + beta * old + bias[m]) as fp32 (EPI 1) or bf16 (EPI 2).  The
// old values are loaded only when beta != 0.
template <int EPI>
DEVI void store4(const PWArgs &a, size_t o, float4 v, int m) {
    if constexpr (EPI) {
        const float bias = a.epi.bias ? a.epi.bias[m] : 0.0f;
        float4 old = make_float4(0.f, 0.f, 0.f, 0.f);
        if (a.epi.beta != 0.0f) {
            if constexpr (EPI == 2) {
                const u32x2 h = *(const u32x2 *)((const uint16_t *)a.O + o);
                old = make_float4(bf16_to_f32(h[0] & 0xffffu), bf16_to_f32(h[0] >> 16), bf16_to_f32(h[1] & 0xffffu),
                                  bf16_to_f32(h[1] >> 16));
            } else {
                old = *(const float4 *)(a.O + o);
            }
        }
        v.x = epi_apply(a.epi, v.x, bias, old.x);
        v.y = epi_apply(a.epi, v.y, bias, old.y);
        v.z = epi_apply(a.epi, v.z, bias, old.z);
        v.w = epi_apply(a.epi, v.w, bias, old.w);
        if constexpr (EPI == 2) {
            *(u32x2 *)((uint16_t *)a.O + o) = u32x2{(uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16),
                                                    (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16)};
            return;
        }
    }
    *(float4 *)(a.O + o) = v;
}

template <bool BWD, int S, int NB, int EPI>
__global__ __launch_bounds__(256, 2) void pw_kernel(PWArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int L = lane & 15, g = lane >> 4;

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int mt = logical % a.m_tiles, rest = logical / a.m_tiles;
    const int rt = rest % a.row_tiles, n = rest / a.row_tiles;
    const int m0 = mt * kRows, p0 = rt * a.TR;
    const int rows = min(a.TR, a.Ho - p0);
    const int npx = rows * a.Wo;
    const int pieces_per_row = a.Wo / 4;
    const int nitems = kChunk * a.TR * pieces_per_row;   // B items per chunk (host: <= 4 per thread)
    const int nchunks = a.Rc / kChunk;
    const rsrc_t rb = make_rsrc(a.B, a.b_bytes), ra = make_rsrc(a.A, a.a_bytes);

    // B chunk load items (channel, output row of the tile, piece of 4 output pixels =
    // 4*S input pixels of one input row), fixed per work-group
    constexpr int MAXIT = 4;
    uint32_t goff[MAXIT];   // byte offset of the item in B for chunk 0 (kOOB when absent)
    int loff[MAXIT];        // LDS byte offset in a stage (-1 when absent)
#pragma unroll
    for (int j = 0; j < MAXIT; ++j) {
        const int it = tid + j * 256;
        goff[j] = kOOB;
        loff[j] = -1;
        if (it < nitems) {
            const int piece = it % pieces_per_row, r2 = it / pieces_per_row;
            const int orow = r2 % a.TR, ch = r2 / a.TR;
            if (orow < rows) {
                const int irow = (p0 + orow) * S, icol = piece * 4 * S;
                goff[j] = (uint32_t)((((size_t)n * a.Rc + ch) * a.Hi + irow) * a.Wi + icol) * 2;
            }
            loff[j] = kABytes + ch * kRowStride + (orow * a.Wo + piece * 4) * 2;
        }
    }
    const uint32_t chunk_stride = (uint32_t)kChunk * a.Hi * a.Wi * 2;   // bytes between chunks in B

    // two register staging sets: chunk c + 2 is loaded while chunk c is multiplied and
    // chunk c + 1 (loaded an iteration ago) is written to LDS
    typedef uint32_t piece_t __attribute__((ext_vector_type(2 * S)));
    piece_t bstg[2][MAXIT];
    u32x4 astg[2][4];   // A chunk: row m0 + (j*256 + tid)/4, 16-byte piece (j*256 + tid) % 4
    auto load_chunk = [&](int ci, piece_t (&bs)[MAXIT], u32x4 (&as)[4]) __attribute__((always_inline)) {
        const bool ok = ci < nchunks;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = j * 256 + tid, row = m0 + (idx >> 2);
            as[j] = ld_vec(ra, ok && row < a.M ? (uint32_t)(((size_t)row * a.Rc + ci * kChunk + (idx & 3) * 8) * 2)
                                               : kOOB);
        }
#pragma unroll
        for (int j = 0; j < MAXIT; ++j) {
            const uint32_t off = !ok || goff[j] == kOOB ? kOOB : goff[j] + (uint32_t)ci * chunk_stride;
            if constexpr (S == 2)
                bs[j] = ld_vec(rb, off);
            else
                bs[j] = ld_b64(rb, off);
        }
    };
    auto write_chunk = [&](int stage, const piece_t (&bs)[MAXIT], const u32x4 (&as)[4]) __attribute__((always_inline)) {
        char *base = smem + stage * kStageBytes;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = j * 256 + tid;
            *(u32x4 *)(base + (idx >> 2) * kARow + (idx & 3) * 16) = as[j];
        }
#pragma unroll
        for (int j = 0; j < MAXIT; ++j) {
            if (loff[j] < 0) continue;
            u32x2 v;
            if constexpr (S == 2) {   // bf16 elements 0, 2, 4, 6 of the 8 loaded
                v[0] = __builtin_amdgcn_perm(bs[j][1], bs[j][0], 0x05040100u);
                v[1] = __builtin_amdgcn_perm(bs[j][3], bs[j][2], 0x05040100u);
            } else {
                v[0] = bs[j][0];
                v[1] = bs[j][1];
            }
            *(u32x2 *)(base + loff[j]) = v;
        }
    };

    // wave w owns rows m0 + 64w .. +63 (A fragments i = 0..3); lane: row 16i + L,
    // r-channels 4g..4g+3 and 16+4g..16+4g+3 of the chunk
    f32x4 acc[4][NB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;

    auto compute = [&](int stage) __attribute__((always_inline)) {
        const char *base = smem + stage * kStageBytes;
        u32x4 af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const char *ar = base + (wave * 64 + 16 * i + L) * kARow + 8 * g;
            const u32x2 lo = *(const u32x2 *)ar, hi = *(const u32x2 *)(ar + 32);
            af[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        const char *bb = base + kABytes + (4 * g + (L >> 2)) * kRowStride + 8 * (L & 3);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const u32x2 lo = tr_read(bb + j * 32), hi = tr_read(bb + 16 * kRowStride + j * 32);
            const u32x4 bf = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                                   __builtin_bit_cast(bf16x8, bf), acc[i][j], 0, 0, 0);
        }
    };

    load_chunk(0, bstg[0], astg[0]);
    load_chunk(1, bstg[1], astg[1]);
    write_chunk(0, bstg[0], astg[0]);
    __syncthreads();
    // iteration c: load chunk c + 2 into set c % 2 (chunk c was written from it an
    // iteration ago), multiply chunk c in stage c % 2, write chunk c + 1 to stage
    // (c + 1) % 2 (last read for chunk c - 1, before the previous barrier)
    for (int c0 = 0; c0 < nchunks; c0 += 2) {
        static_for<0, 2>([&](auto pc) __attribute__((always_inline)) {
            constexpr int P = decltype(pc)::value;
            const int c = c0 + P;
            if (c < nchunks) {
                load_chunk(c + 2, bstg[P], astg[P]);
                compute(P);
                if (c + 1 < nchunks) write_chunk(P ^ 1, bstg[P ^ 1], astg[P ^ 1]);
                __syncthreads();
            }
        });
    }

    // epilogue: one wave's 64 rows at a time go through LDS ([64 rows][pixels], fp32,
    // 528-byte rows: the MFMA layout's 4 row groups x 16 pixels per store fall on
    // distinct banks); then every output row span of those rows -- contiguous in
    // memory -- is written by all threads with 16-byte stores, consecutive lanes on
    // consecutive bytes.  Lane holds pixel 16j + L and rows 64*wave + 16i + 4g + v.
    constexpr int SROW = 528;   // bytes per staged row (128 pixels + 4 words of pad)
    float *stile = (float *)smem;
    const int HoWo = a.Ho * a.Wo;
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int v = 0; v < 4; ++v) stile[(16 * i + 4 * g + v) * (SROW / 4) + 16 * j + L] = acc[i][j][v];
        }
        __syncthreads();
        const int r0 = m0 + 64 * w;
        const int mrows = min(64, a.M - r0);
        if constexpr (!BWD) {
            // y[n][r0 + r][p0*Wo .. p0*Wo + npx): npx/4 quads per row
            const int nq = npx / 4;
            const size_t base = ((size_t)n * a.M + r0) * HoWo + (size_t)p0 * a.Wo;
            for (int idx = tid; idx < mrows * nq; idx += 256) {
                const int r = idx / nq, q = idx - r * nq;
                float4 v = *(const float4 *)(stile + r * (SROW / 4) + 4 * q);
                store4<EPI>(a, base + (size_t)r * HoWo + 4 * q, v, r0 + r);
            }
        } else {
            // dx[n][r0 + r][s*p0 .. s*(p0 + rows)) whole rows: s*rows rows of s*Wo floats,
            // value (p, q) at (s*p, s*q), zeros elsewhere
            const int s = a.s, Wd = s * a.Wo, HWd = s * a.Ho * Wd;
            const int rq = Wd / 4;                 // quads per dx row
            const int nq = s * rows * rq;          // quads per channel of the tile
            const size_t base = ((size_t)n * a.M + r0) * HWd + (size_t)s * p0 * Wd;
            for (int idx = tid; idx < mrows * nq; idx += 256) {
                const int r = idx / nq, rem = idx - r * nq;
                const int dr = rem / rq, q = rem - dr * rq;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (s == 1) {
                    v = *(const float4 *)(stile + r * (SROW / 4) + dr * a.Wo + 4 * q);
                } else if ((dr & 1) == 0) {   // dx columns 4q .. 4q+3 = output columns 2q, 2q+1
                    const float2 u = *(const float2 *)(stile + r * (SROW / 4) + (dr >> 1) * a.Wo + 2 * q);
                    v = make_float4(u.x, 0.f, u.y, 0.f);
                }
                store4<EPI>(a, base + (size_t)r * HWd + (size_t)dr * Wd + 4 * q, v, r0 + r);
            }
        }
        __syncthreads();
    }
}

template <bool BWD, int S, int EPI>
static hipError_t pw_nb(const PWArgs &a, int nb, int grid, hipStream_t st) {
    const size_t lds = 2 * (size_t)kStageBytes;
    auto go = [&](auto kern) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, a);
        return hipGetLastError();
    };
    switch (nb) {
        case 1: return go(pw_kernel<BWD, S, 1, EPI>);
        case 2: return go(pw_kernel<BWD, S, 2, EPI>);
        case 3: return go(pw_kernel<BWD, S, 3, EPI>);
        case 4: return go(pw_kernel<BWD, S, 4, EPI>);
        case 5: return go(pw_kernel<BWD, S, 5, EPI>);
        case 6: return go(pw_kernel<BWD, S, 6, EPI>);
        case 7: return go(pw_kernel<BWD, S, 7, EPI>);
        default: return go(pw_kernel<BWD, S, 8, EPI>);
    }
}

// ------------------------------------------------------------------ backward-filter
// dW[k][c] = sum over output pixels (n, p, q) of dy[n][k][p][q] * x[n][c][s*p][s*q]: one
// GEMM (rows k, columns c) reducing over the flat pixel index f = (n*P + p)*Q + q.  The
// pixels are split into ranges of whole 64-pixel steps (split-K): partial sums
// [split][K][C] for the split-K reduce kernels (a fixed summation order), or dW written
// directly, through the output epilogue, with one split.
// Work-group tile: 128 k x 128 c; four waves of 64 x 64 (4 x 4 blocks of 16 x 16 on
// v_mfma_f32_16x16x32_bf16, two k32 sub-steps per step).  Per step both operands go to
// LDS as [row][64 pixels] (144-byte rows): dy as 16-byte pieces of 8 pixels of one row
// (P*Q % 8 == 0, so a piece never crosses an image), x as pieces of 4 output pixels of
// one output row (Q % 4 == 0): a 16-byte row load of 8 input columns whose even ones
// stride 2 keeps (byte permutes), or an 8-byte load at stride 1.  MFMA k-slots: lane
// group g holds pixels 8g..8g+7 of the sub-step, so every fragment is one 16-byte read;
// 16 rows 144 bytes apart fall on 16 distinct 16-byte bank groups.  Loads run three steps
// ahead through three register sets; two LDS stages.
namespace {
constexpr int kFT = 128;                      // tile rows (k) and columns (c)
constexpr int kFPix = 64;                     // pixels per step
constexpr int kFRow = 144;                    // LDS bytes per row of a step (128 data + 16 pad)
constexpr int kFStage = 2 * kFT * kFRow;      // dy rows, then x rows
}  // namespace

struct PWFArgs {
    const void *X, *DY;
    float *out;           // partial sums [splits][K][C], or dW [K][C] when direct
    uint32_t x_bytes, dy_bytes;
    int C, K, H, W, P, Q, PQ;
    int m_tiles, c_tiles, steps_per_split, total;   // total = N*P*Q pixels
    FDiv fd_PQ, fd_Q;
    int direct, has_epi;
    Epi epi;
};

template <int S>
__global__ __launch_bounds__(256, 2) void pwf_kernel(PWFArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int L = lane & 15, g = lane >> 4;
    const int wk = wave & 1, wc = wave >> 1;   // 64-row half, 64-column half
    const int tiles = a.m_tiles * a.c_tiles;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);   // a split's tiles on one XCD
    const int z = logical / tiles, tile = logical - z * tiles;
    const int m0 = (tile % a.m_tiles) * kFT, c0 = (tile / a.m_tiles) * kFT;
    const int s_begin = z * a.steps_per_split;
    const int nsteps = min(a.steps_per_split, (a.total + kFPix - 1) / kFPix - s_begin);   // >= 1 (host)
    const rsrc_t rx = make_rsrc(a.X, a.x_bytes), rdy = make_rsrc(a.DY, a.dy_bytes);

    // dy: 128 rows x 8 pieces of 8 pixels, 4 per thread: rows (tid >> 3) + 32j, piece tid & 7;
    // x: 128 channels x 16 pieces of 4 pixels, 8 per thread: channels (tid >> 4) + 16j, piece tid & 15.
    // A thread's pieces share one pixel position, which steps forward 64 pixels per step (the
    // steps are loaded in order); the plan guarantees at most one image wrap and one row wrap
    // per step, so the offsets advance by additions.  Offsets are elements of row / channel j = 0.
    typedef uint32_t xpiece_t __attribute__((ext_vector_type(2 * S)));
    u32x4 dstg[3][4];
    xpiece_t xstg[3][8];
    const int drow = tid >> 3, xch = tid >> 4;
    int df = s_begin * kFPix + (tid & 7) * 8;                       // dy pieces' stream pixel
    int dn = (int)fdiv((uint32_t)df, a.fd_PQ), dpix = df - dn * a.PQ;
    uint32_t doff = (uint32_t)((dn * a.K + m0 + drow) * a.PQ + dpix);
    const uint32_t d_img = (uint32_t)((a.K - 1) * a.PQ), d_j = (uint32_t)(32 * a.PQ);
    int xf = s_begin * kFPix + (tid & 15) * 4;                      // x pieces' stream pixel
    int xn = (int)fdiv((uint32_t)xf, a.fd_PQ), xpix = xf - xn * a.PQ;
    int xp = (int)fdiv((uint32_t)xpix, a.fd_Q), xq = xpix - xp * a.Q;
    uint32_t xoff = (uint32_t)(((xn * a.C + c0 + xch) * a.H + S * xp) * a.W + S * xq);
    const int d64 = kFPix / a.Q, r64 = kFPix % a.Q;
    const uint32_t x_adv = (uint32_t)(S * (d64 * a.W + r64)), x_row = (uint32_t)(S * (a.W - a.Q)),
                   x_img = (uint32_t)(a.C * a.H * a.W - S * a.P * a.W), x_j = (uint32_t)(16 * a.H * a.W);
    // rows / channels of the thread's pieces inside the tensor (fixed per work-group); an
    // absent piece's byte offset is kOOB plus a multiple of its stride (still out of range)
    bool dval[4], xval[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) dval[j] = m0 + drow + 32 * j < a.K;
#pragma unroll
    for (int j = 0; j < 8; ++j) xval[j] = c0 + xch + 16 * j < a.C;
    auto load_step = [&](int st, u32x4 (&ds)[4], xpiece_t (&xs)[8]) __attribute__((always_inline)) {
        const bool ok = st < nsteps;
        const uint32_t db = ok && df < a.total ? doff * 2 : kOOB, xb = ok && xf < a.total ? xoff * 2 : kOOB;
#pragma unroll
        for (int j = 0; j < 4; ++j) ds[j] = ld_vec(rdy, (dval[j] ? db : kOOB) + j * d_j * 2);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t off = (xval[j] ? xb : kOOB) + j * x_j * 2;
            if constexpr (S == 2)
                xs[j] = ld_vec(rx, off);
            else
                xs[j] = ld_b64(rx, off);
        }
        // 64 pixels on
        df += kFPix;
        dpix += kFPix;
        doff += kFPix;
        if (dpix >= a.PQ) {
            dpix -= a.PQ;
            doff += d_img;
        }
        xf += kFPix;
        xq += r64;
        xp += d64;
        xoff += x_adv;
        if (xq >= a.Q) {
            xq -= a.Q;
            ++xp;
            xoff += x_row;
        }
        if (xp >= a.P) {
            xp -= a.P;
            xoff += x_img;
        }
    };
    auto write_step = [&](int stage, const u32x4 (&ds)[4], const xpiece_t (&xs)[8]) __attribute__((always_inline)) {
        char *base = smem + stage * kFStage;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = j * 256 + tid;
            *(u32x4 *)(base + (idx >> 3) * kFRow + (idx & 7) * 16) = ds[j];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int idx = j * 256 + tid;
            u32x2 v;
            if constexpr (S == 2) {   // bf16 elements 0, 2, 4, 6 of the 8 loaded
                v[0] = __builtin_amdgcn_perm(xs[j][1], xs[j][0], 0x05040100u);
                v[1] = __builtin_amdgcn_perm(xs[j][3], xs[j][2], 0x05040100u);
            } else {
                v[0] = xs[j][0];
                v[1] = xs[j][1];
            }
            *(u32x2 *)(base + (kFT + (idx >> 4)) * kFRow + (idx & 15) * 8) = v;
        }
    };

    f32x4 acc[4][4];   // block (i, j): rows m0 + 64wk + 16i + 4g + v, column c0 + 64wc + 16j + L
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;
    auto compute = [&](int stage) __attribute__((always_inline)) {
        const char *base = smem + stage * kFStage;
#pragma unroll
        for (int h = 0; h < 2; ++h) {   // k32 sub-steps: pixels 32h + 8g .. +7
            u32x4 af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = *(const u32x4 *)(base + (wk * 64 + 16 * i + L) * kFRow + 64 * h + 16 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *(const u32x4 *)(base + (kFT + wc * 64 + 16 * j + L) * kFRow + 64 * h + 16 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bf[j]), acc[i][j], 0, 0, 0);
        }
    };

    // iteration s: load step s + 3 into register set s % 3 (step s was written from it an
    // iteration ago), multiply step s in LDS stage s % 2, write step s + 1 (set (s + 1) % 3)
    // to stage (s + 1) % 2 (last read for step s - 1, before the previous barrier).  Steps are
    // loaded in order; six iterations per loop turn keep every set and stage index constant.
    load_step(0, dstg[0], xstg[0]);
    load_step(1, dstg[1], xstg[1]);
    load_step(2, dstg[2], xstg[2]);
    write_step(0, dstg[0], xstg[0]);
    __syncthreads();
    for (int s0 = 0; s0 < nsteps; s0 += 6) {
        static_for<0, 6>([&](auto pc) __attribute__((always_inline)) {
            constexpr int P = decltype(pc)::value;
            constexpr int RS = P % 3, RN = (P + 1) % 3, ST = P % 2;
            const int st = s0 + P;
            if (st < nsteps) {
                load_step(st + 3, dstg[RS], xstg[RS]);
                compute(ST);
                if (st + 1 < nsteps) write_step(ST ^ 1, dstg[RN], xstg[RN]);
                __syncthreads();
            }
        });
    }

    // the tile: 32-bit element offsets from one product per lane plus uniform strides
    const int k0 = m0 + wk * 64 + 4 * g, cl = c0 + wc * 64 + L;
    const uint32_t base = (uint32_t)(a.direct ? 0 : z) * (uint32_t)a.K * a.C + (uint32_t)k0 * a.C + cl;
    if (!a.direct) {   // partial sums
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (k0 + 16 * i + v < a.K && cl + 16 * j < a.C)
                        a.out[base + (uint32_t)(16 * i + v) * a.C + 16 * j] = acc[i][j][v];
    } else {           // dW through the output epilogue
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (k0 + 16 * i + v < a.K && cl + 16 * j < a.C)
                        out_store(a.out, base + (uint32_t)(16 * i + v) * a.C + 16 * j, acc[i][j][v], a.epi,
                                  a.has_epi);
    }
}

static int launch_pointwise_bwdf(const Plan &pl, const Problem &p, const void *x, const void *dy, float *dw,
                                 void *ws, hipStream_t st, const Epi *epi) {
    PWFArgs a = {};
    a.X = x;
    a.DY = dy;
    a.x_bytes = (uint32_t)((size_t)p.N * p.C * p.H * p.W * 2);
    a.dy_bytes = (uint32_t)((size_t)p.N * p.K * p.P * p.Q * 2);
    a.C = p.C; a.K = p.K; a.H = p.H; a.W = p.W; a.P = p.P; a.Q = p.Q; a.PQ = p.P * p.Q;
    a.m_tiles = pl.m_tiles;
    a.c_tiles = pl.n_tiles;
    a.steps_per_split = pl.chunk / kFPix;
    a.total = p.N * p.P * p.Q;
    a.fd_PQ = make_fdiv((uint32_t)a.PQ);
    a.fd_Q = make_fdiv((uint32_t)p.Q);
    a.direct = pl.splits == 1;
    if (epi) a.epi = *epi;
    a.has_epi = epi ? 1 : 0;
    float *part = pl.splits > 1 ? (float *)((char *)ws + pl.part_offset) : dw;
    a.out = part;
    const size_t lds = 2 * (size_t)kFStage;
    auto k = p.sh == 2 ? pwf_kernel<2> : pwf_kernel<1>;
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return MICONV_ERR_HIP;
    hipLaunchKernelGGL(k, dim3(pl.m_tiles * pl.n_tiles * pl.splits), dim3(256), lds, st, a);
    if (hipGetLastError() != hipSuccess) return MICONV_ERR_HIP;
    if (pl.splits > 1) return launch_splitk_reduce(part, dw, p.K, p.C, 1, pl.splits, st, epi);
    return MICONV_OK;
}

int launch_pointwise(const Plan &pl, const Problem &p, const void *in0, const void *in1, float *out, void *ws,
                     hipStream_t st, const Epi *epi) {
    if (p.pass == BWD_FILTER) return launch_pointwise_bwdf(pl, p, in0, in1, out, ws, st, epi);
    PWArgs a = {};
    const bool bwd = p.pass == BWD_DATA;
    a.N = p.N;
    a.TR = pl.tr;
    a.s = p.sh;
    if (!bwd) {
        a.A = in1;   // W [K][C]
        a.B = in0;   // x
        a.M = p.K; a.Rc = p.C; a.Hi = p.H; a.Wi = p.W; a.Ho = p.P; a.Wo = p.Q;
    } else {
        uint16_t *wt = (uint16_t *)((char *)ws + pl.wt_offset);
        hipLaunchKernelGGL(pw_transpose, dim3((p.C + 31) / 32, (p.K + 31) / 32), dim3(256), 0, st,
                           (const uint16_t *)in1, wt, p.K, p.C);
        if (hipGetLastError() != hipSuccess) return MICONV_ERR_HIP;
        a.A = wt;    // W^T [C][K]
        a.B = in0;   // dy
        a.M = p.C; a.Rc = p.K; a.Hi = p.P; a.Wi = p.Q; a.Ho = p.P; a.Wo = p.Q;
    }
    a.O = out;
    a.a_bytes = (uint32_t)((size_t)a.M * a.Rc * 2);
    a.b_bytes = (uint32_t)((size_t)p.N * a.Rc * a.Hi * a.Wi * 2);
    a.row_tiles = (a.Ho + a.TR - 1) / a.TR;
    a.m_tiles = (a.M + kRows - 1) / kRows;
    const int nb = (a.TR * a.Wo + 15) / 16;
    const int grid = a.m_tiles * a.row_tiles * p.N;
    hipError_t e;
    const int em = epi ? (epi->out_bf16 ? 2 : 1) : 0;
    if (epi) a.epi = *epi;
    if (bwd) {
        e = em == 2 ? pw_nb<true, 1, 2>(a, nb, grid, st)
                    : (em == 1 ? pw_nb<true, 1, 1>(a, nb, grid, st) : pw_nb<true, 1, 0>(a, nb, grid, st));
    } else {
        if (p.sh == 2)
            e = em == 2 ? pw_nb<false, 2, 2>(a, nb, grid, st)
                        : (em == 1 ? pw_nb<false, 2, 1>(a, nb, grid, st) : pw_nb<false, 2, 0>(a, nb, grid, st));
        else
            e = em == 2 ? pw_nb<false, 1, 2>(a, nb, grid, st)
                        : (em == 1 ? pw_nb<false, 1, 1>(a, nb, grid, st) : pw_nb<false, 1, 0>(a, nb, grid, st));
    }
    return e == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
}

}  // namespace miconv
