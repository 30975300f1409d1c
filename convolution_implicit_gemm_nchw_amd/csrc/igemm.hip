// igemm.hip -- gfx950 implicit-GEMM kernels for NCHW / KCRS convolution.
//
// One MFMA main loop serves the three passes; each pass supplies the two
// operand gathers and the epilogue.  Nothing is materialised in HBM except an
// optional tap-major copy of the (small) filter and the backward-filter
// split-K partial sums.
//
// Work-group: 256 threads = 4 waves of 64.  Tile BM x BN of the GEMM output;
// each wave owns (BM/WM) x (BN/WN) and computes it in 32x32 MFMA blocks:
//   bf16: v_mfma_f32_32x32x16_bf16   fp32: v_mfma_f32_32x32x2_f32
// Accumulation is fp32 in both cases.
//
// LDS: both operands are stored reduction-contiguous ("K-major"): one LDS row
// of BKB bytes per GEMM row (A) or GEMM column (B), padded by 16 bytes so that
// the 16-byte fragment reads of 32 consecutive rows hit distinct banks.
// MFMA k-slots are paired identically for A and B: lane l reads row l%32 and
// the half (l/32) of the row's reduction slice, so every MFMA sums over
// matching reduction indices whatever the hardware's internal k order is.
// Two LDS stages; global loads for step k+1 are issued before the MFMAs of
// step k and written to LDS after them, one barrier per step.
//
// Gathers use raw buffer loads: an offset at or above the tensor's byte size
// returns 0, which is how zero padding, ragged tiles and out-of-range taps
// are produced without branches (tensors are < 2 GiB, so 0x80000000 is out of
// range for every tensor).
//
// Reduction order is tap-major: index = tap * channels + channel, so 16 bytes
// of consecutive reduction indices share one tap and one padding predicate
// whenever the channel count is a multiple of the vector width.
#include "device.h"
#include "launch.h"

namespace miconv {


// ------------------------------------------------------------------ forward
// rows = K (filter rows), cols = N*P*Q (output pixels), reduction (t, c): t = r*S + s.
// A: filter, tap-major copy [K][R*S][C] (or the original [K][C][R][S]).
// B: x gathered at (n, c, p*sh - ph + r, q*sw - pw + s), zero outside the image.
template <int DT, int BM, int BN, int BKB, bool CVEC, int EPI = 0>
struct FwdPass {
    static constexpr int ES = DT ? 2 : 4, VEC = 16 / ES, BK = BKB / ES, VPR = BKB / 16;
    static constexpr int NVA = (BM * VPR + 255) / 256, NVB = BN * VPR / 256;
    int m0, n0, nk, Kred, T, HW, PQ, NPQ;
    int ih0, iw0, xb;  // this thread's B column (output pixel)
    rsrc_t rx, rw;

    DEVI bool init(const KArgs &a, int logical, int tid) {
        const int tiles = a.m_tiles * a.n_tiles;
        if (logical >= tiles) return false;
        m0 = (logical % a.m_tiles) * BM;
        n0 = (logical / a.m_tiles) * BN;
        T = a.R * a.S;
        Kred = T * a.C;
        HW = a.H * a.W;
        PQ = a.P * a.Q;
        NPQ = a.N * PQ;
        nk = (Kred + BK - 1) / BK;
        rx = make_rsrc(a.a0, a.a0_bytes);
        rw = make_rsrc(a.a1, a.a1_bytes);
        const int gp = n0 + tid % BN;
        const int gq = gp < NPQ ? gp : 0;
        const int n = (int)fdiv((uint32_t)gq, a.fd_PQ);
        const int pq = gq - n * PQ;
        const int p = (int)fdiv((uint32_t)pq, a.fd_Q);
        const int q = pq - p * a.Q;
        ih0 = p * a.sh - a.ph;
        iw0 = q * a.sw - a.pw;
        xb = n * a.C * HW + ih0 * a.W + iw0;
        if (gp >= NPQ) ih0 = -(1 << 30);  // no tap row is ever inside the image
        return true;
    }

    DEVI void load_a(const KArgs &a, int kt, u32x4 *ra, int tid) const {
#pragma unroll
        for (int i = 0; i < NVA; ++i) {
            const int v = tid + i * 256;
            if (BM * VPR < 256 * (i + 1) && v >= BM * VPR) continue;
            const int row = v / VPR, kq = v % VPR;
            const int k = m0 + row, kk = kt * BK + kq * VEC;
            if (a.wt && CVEC) {
                const bool ok = k < a.K && kk < Kred;
                ra[i] = ld_vec(rw, ok ? (uint32_t)(k * Kred + kk) * ES : kOOB);
            } else {
                uint32_t e[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const int kr = kk + j;
                    uint32_t off = kOOB;
                    if (k < a.K && kr < Kred) {
                        if (a.wt) {
                            off = (uint32_t)(k * Kred + kr) * ES;
                        } else {
                            const int t = (int)fdiv((uint32_t)kr, a.fd_C), c = kr - t * a.C;
                            off = (uint32_t)((k * a.C + c) * T + t) * ES;
                        }
                    }
                    e[j] = ld_elem<ES>(rw, off);
                }
                ra[i] = pack<ES>(e);
            }
        }
    }

    DEVI void load_b(const KArgs &a, int kt, u32x4 *rb, int tid) const {
#pragma unroll
        for (int i = 0; i < NVB; ++i) {
            const int vq = uniform(tid / BN + i * (256 / BN));
            const int kb = kt * BK + vq * VEC;
            if (CVEC) {
                // VEC consecutive channels of one tap: one predicate, channel stride HW
                const int t = (int)fdiv((uint32_t)kb, a.fd_C), c0 = kb - t * a.C;
                const int r = (int)fdiv((uint32_t)t, a.fd_S), s = t - r * a.S;
                const bool ok = kb < Kred && (unsigned)(ih0 + r) < (unsigned)a.H &&
                                (unsigned)(iw0 + s) < (unsigned)a.W;
                const uint32_t base = ok ? (uint32_t)(xb + c0 * HW + r * a.W + s) * ES : kOOB;
                uint32_t e[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) e[j] = ld_elem<ES>(rx, base + (uint32_t)(j * HW * ES));
                rb[i] = pack<ES>(e);
            } else {
                uint32_t e[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const int kr = kb + j;
                    const int t = (int)fdiv((uint32_t)kr, a.fd_C), c = kr - t * a.C;
                    const int r = (int)fdiv((uint32_t)t, a.fd_S), s = t - r * a.S;
                    const bool ok = kr < Kred && (unsigned)(ih0 + r) < (unsigned)a.H &&
                                    (unsigned)(iw0 + s) < (unsigned)a.W;
                    e[j] = ld_elem<ES>(rx, ok ? (uint32_t)(xb + c * HW + r * a.W + s) * ES : kOOB);
                }
                rb[i] = pack<ES>(e);
            }
        }
    }

    template <int PITCH>
    DEVI void store_b(const u32x4 *rb, char *sb, int tid) const {
#pragma unroll
        for (int i = 0; i < NVB; ++i) {
            const int vq = tid / BN + i * (256 / BN);
            *(u32x4 *)(sb + (tid % BN) * PITCH + vq * 16) = rb[i];
        }
    }

    template <int WM, int TM, int TN>
    DEVI void epilogue(const KArgs &a, const f32x16 (&acc)[TM][TN], int wave, int lane, char *lds) const {
        constexpr int WN = 4 / WM, WTM = BM / WM, WTN = BN / WN;
        const int wm = wave % WM, wn = wave / WM, lr = lane & 31, lh = lane >> 5;
        // fused epilogue: the tile rows' bias values go to LDS (free once the main
        // loop is done) before any store, and each 32x32 block's previous outputs
        // are loaded before that block's stores
        float *bs = (float *)lds;
        if constexpr (EPI) {
            __syncthreads();   // every wave is done with the LDS stages
            for (int m = threadIdx.x; m < BM; m += 256) bs[m] = a.epi.bias && m0 + m < a.K ? a.epi.bias[m0 + m] : 0.0f;
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int gp = n0 + wn * WTN + j * 32 + lr;
            if (gp >= NPQ) continue;
            const int n = (int)fdiv((uint32_t)gp, a.fd_PQ);
            const size_t ob = (size_t)n * a.K * PQ + (gp - n * PQ);
            float *o = a.out + ob;
            uint16_t *o16 = (uint16_t *)a.out + ob;   // bf16 output (EPI == 2)
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if constexpr (EPI) {
                    float old[16];
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int k = m0 + wm * WTM + i * 32 + acc_row(v, lh);
                        const bool rd = a.epi.beta != 0.0f && k < a.K;
                        if constexpr (EPI == 2)
                            old[v] = rd ? bf16_to_f32(o16[(size_t)k * PQ]) : 0.0f;
                        else
                            old[v] = rd ? o[(size_t)k * PQ] : 0.0f;
                    }
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int mr = wm * WTM + i * 32 + acc_row(v, lh);
                        if (m0 + mr >= a.K) continue;
                        const float val = epi_apply(a.epi, acc[i][j][v], bs[mr], old[v]);
                        if constexpr (EPI == 2)
                            o16[(size_t)(m0 + mr) * PQ] = f32_to_bf16(val);
                        else
                            o[(size_t)(m0 + mr) * PQ] = val;
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int k = m0 + wm * WTM + i * 32 + acc_row(v, lh);
                        if (k < a.K) o[(size_t)k * PQ] = acc[i][j][v];
                    }
                }
            }
        }
    }
};

// ------------------------------------------------------------------ backward-data
// One stride phase per z: rows = C, cols = (n, a, b) over the phase's output
// positions i = i0h + sh*a, j = i0w + sw*b; reduction (t, k) over the phase's
// taps t = (u, v) -> r = fh + sh*u, s = fw + sw*v and output channels k.
// A: filter, tap-major copy [R*S][C][K] (or the original [K][C][R][S]).
// B: dy gathered at (n, k, baseh + a - u, basew + b - v), zero out of range.
template <int DT, int BM, int BN, int BKB, bool CVEC>
struct BwdDataPass {
    static constexpr int ES = DT ? 2 : 4, VEC = 16 / ES, BK = BKB / ES, VPR = BKB / 16;
    static constexpr int NVA = (BM * VPR + 255) / 256, NVB = BN * VPR / 256;
    int m0, n0, nk, Kred, PQ, ncols, fh, fw;
    PhaseDim dh, dw;
    FDiv fd_ab, fd_b, fd_nuw;
    int pb, qb, dyb;  // this thread's B column
    rsrc_t rdy, rw;

    DEVI bool init(const KArgs &a, int logical, int tid) {
        const int tiles = a.m_tiles * a.n_tiles;
        const int z = logical / tiles, tt = logical - z * tiles;
        if (z >= a.nz) return false;
        const int ph = a.use_map ? a.live_map[z] : z;
        fh = ph / a.sw;
        fw = ph - fh * a.sw;
        dh = phase_dim(fh, a.sh, a.ph, a.H, a.R);
        dw = phase_dim(fw, a.sw, a.pw, a.W, a.S);
        ncols = a.N * dh.na * dw.na;
        m0 = (tt % a.m_tiles) * BM;
        n0 = (tt / a.m_tiles) * BN;
        if (n0 >= ncols) return false;
        PQ = a.P * a.Q;
        Kred = dh.nu * dw.nu * a.K;
        nk = (Kred + BK - 1) / BK;
        fd_ab = make_fdiv((uint32_t)(dh.na * dw.na));
        fd_b = make_fdiv((uint32_t)dw.na);
        fd_nuw = make_fdiv((uint32_t)(dw.nu > 0 ? dw.nu : 1));
        rdy = make_rsrc(a.a0, a.a0_bytes);
        rw = make_rsrc(a.a1, a.a1_bytes);
        const int gc = n0 + tid % BN;
        const int gq = gc < ncols ? gc : 0;
        const int n = (int)fdiv((uint32_t)gq, fd_ab);
        const int rem = gq - n * dh.na * dw.na;
        const int aa = (int)fdiv((uint32_t)rem, fd_b);
        const int bb = rem - aa * dw.na;
        pb = dh.base + aa;
        qb = dw.base + bb;
        dyb = n * a.K * PQ + pb * a.Q + qb;
        if (gc >= ncols) pb = 1 << 30;  // every p = pb - u is out of range
        return true;
    }

    DEVI void load_a(const KArgs &a, int kt, u32x4 *ra, int tid) const {
#pragma unroll
        for (int i = 0; i < NVA; ++i) {
            const int v = tid + i * 256;
            if (BM * VPR < 256 * (i + 1) && v >= BM * VPR) continue;
            const int row = v / VPR, kq = v % VPR;
            const int c = m0 + row, kk = kt * BK + kq * VEC;
            if (a.wt && CVEC) {
                uint32_t off = kOOB;
                if (c < a.C && kk < Kred) {
                    const int t = (int)fdiv((uint32_t)kk, a.fd_K), k0 = kk - t * a.K;
                    const int u = (int)fdiv((uint32_t)t, fd_nuw), vv = t - u * dw.nu;
                    const int r = fh + a.sh * u, s = fw + a.sw * vv;
                    off = (uint32_t)(((r * a.S + s) * a.C + c) * a.K + k0) * ES;
                }
                ra[i] = ld_vec(rw, off);
            } else {
                uint32_t e[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const int kr = kk + j;
                    uint32_t off = kOOB;
                    if (c < a.C && kr < Kred) {
                        const int t = (int)fdiv((uint32_t)kr, a.fd_K), k = kr - t * a.K;
                        const int u = (int)fdiv((uint32_t)t, fd_nuw), vv = t - u * dw.nu;
                        const int r = fh + a.sh * u, s = fw + a.sw * vv;
                        off = a.wt ? (uint32_t)(((r * a.S + s) * a.C + c) * a.K + k) * ES
                                   : (uint32_t)(((k * a.C + c) * a.R + r) * a.S + s) * ES;
                    }
                    e[j] = ld_elem<ES>(rw, off);
                }
                ra[i] = pack<ES>(e);
            }
        }
    }

    DEVI void load_b(const KArgs &a, int kt, u32x4 *rb, int tid) const {
#pragma unroll
        for (int i = 0; i < NVB; ++i) {
            const int vq = uniform(tid / BN + i * (256 / BN));
            const int kb = kt * BK + vq * VEC;
            if (CVEC) {
                const int t = (int)fdiv((uint32_t)kb, a.fd_K), k0 = kb - t * a.K;
                const int u = (int)fdiv((uint32_t)t, fd_nuw), vv = t - u * dw.nu;
                const bool ok = kb < Kred && (unsigned)(pb - u) < (unsigned)a.P &&
                                (unsigned)(qb - vv) < (unsigned)a.Q;
                const uint32_t base = ok ? (uint32_t)(dyb + k0 * PQ - u * a.Q - vv) * ES : kOOB;
                uint32_t e[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) e[j] = ld_elem<ES>(rdy, base + (uint32_t)(j * PQ * ES));
                rb[i] = pack<ES>(e);
            } else {
                uint32_t e[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const int kr = kb + j;
                    const int t = (int)fdiv((uint32_t)kr, a.fd_K), k = kr - t * a.K;
                    const int u = (int)fdiv((uint32_t)t, fd_nuw), vv = t - u * dw.nu;
                    const bool ok = kr < Kred && (unsigned)(pb - u) < (unsigned)a.P &&
                                    (unsigned)(qb - vv) < (unsigned)a.Q;
                    e[j] = ld_elem<ES>(rdy, ok ? (uint32_t)(dyb + k * PQ - u * a.Q - vv) * ES : kOOB);
                }
                rb[i] = pack<ES>(e);
            }
        }
    }

    template <int PITCH>
    DEVI void store_b(const u32x4 *rb, char *sb, int tid) const {
#pragma unroll
        for (int i = 0; i < NVB; ++i) {
            const int vq = tid / BN + i * (256 / BN);
            *(u32x4 *)(sb + (tid % BN) * PITCH + vq * 16) = rb[i];
        }
    }

    template <int WM, int TM, int TN>
    DEVI void epilogue(const KArgs &a, const f32x16 (&acc)[TM][TN], int wave, int lane, char *lds) const {
        constexpr int WN = 4 / WM, WTM = BM / WM, WTN = BN / WN;
        const int wm = wave % WM, wn = wave / WM, lr = lane & 31, lh = lane >> 5;
        const int HW = a.H * a.W;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int gc = n0 + wn * WTN + j * 32 + lr;
            if (gc >= ncols) continue;
            const int n = (int)fdiv((uint32_t)gc, fd_ab);
            const int rem = gc - n * dh.na * dw.na;
            const int aa = (int)fdiv((uint32_t)rem, fd_b);
            const int bb = rem - aa * dw.na;
            const int ii = dh.i0 + a.sh * aa, jj = dw.i0 + a.sw * bb;
            const size_t o = (size_t)n * a.C * HW + ii * a.W + jj;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int c = m0 + wm * WTM + i * 32 + acc_row(v, lh);
                    if (c < a.C)
                        out_store(a.out, o + (size_t)c * HW, acc[i][j][v], a.epi, a.has_epi,
                                  a.epi.bias ? a.epi.bias[c] : 0.0f);
                }
        }
    }
};

// ------------------------------------------------------------------ backward-filter
// rows = K, cols = (t, c) with t = r*S + s, reduction = output pixels (n, p, q),
// split into nz contiguous chunks of `chunk` pixels (one per z).
// A: dy [N][K][P*Q] rows k, pixel-contiguous.
// B: x gathered at (n, c, p*sh - ph + r, q*sw - pw + s); lanes run along
//    pixels (coalesced), each thread holds VEC columns of one pixel and writes
//    them to LDS one element at a time (transposing into pixel-contiguous rows).
template <int DT, int BM, int BN, int BKB, bool CVEC, bool PQVEC>
struct BwdFilterPass {
    static constexpr int ES = DT ? 2 : 4, VEC = 16 / ES, BK = BKB / ES, VPR = BKB / 16;
    static constexpr int NVA = (BM * VPR + 255) / 256, NVB = BN * VPR / 256;
    static_assert(BK == 64, "one wave covers the 64 pixels of a reduction step");
    int m0, n0, nk, z, pbeg, pend, T, TC, HW, PQ;
    rsrc_t rx, rdy;

    DEVI bool init(const KArgs &a, int logical, int tid) {
        const int tiles = a.m_tiles * a.n_tiles;
        z = logical / tiles;
        const int tt = logical - z * tiles;
        if (z >= a.nz) return false;
        m0 = (tt % a.m_tiles) * BM;
        n0 = (tt / a.m_tiles) * BN;
        T = a.R * a.S;
        TC = T * a.C;
        HW = a.H * a.W;
        PQ = a.P * a.Q;
        const int npq = a.N * PQ;
        pbeg = z * a.chunk;
        pend = min(npq, pbeg + a.chunk);
        nk = pend > pbeg ? (pend - pbeg + BK - 1) / BK : 0;
        rx = make_rsrc(a.a0, a.a0_bytes);
        rdy = make_rsrc(a.a1, a.a1_bytes);
        (void)tid;
        return true;
    }

    DEVI void load_a(const KArgs &a, int kt, u32x4 *ra, int tid) const {
#pragma unroll
        for (int i = 0; i < NVA; ++i) {
            const int v = tid + i * 256;
            if (BM * VPR < 256 * (i + 1) && v >= BM * VPR) continue;
            const int row = v / VPR, kq = v % VPR;
            const int k = m0 + row, px0 = pbeg + kt * BK + kq * VEC;
            if (PQVEC) {
                // P*Q % VEC == 0: the vector lies inside one image and is 16-byte aligned
                uint32_t off = kOOB;
                if (k < a.K && px0 < pend) {
                    const int n = (int)fdiv((uint32_t)px0, a.fd_PQ);
                    off = (uint32_t)((n * a.K + k) * PQ + (px0 - n * PQ)) * ES;
                }
                ra[i] = ld_vec(rdy, off);
            } else {
                uint32_t e[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const int px = px0 + j;
                    uint32_t off = kOOB;
                    if (k < a.K && px < pend) {
                        const int n = (int)fdiv((uint32_t)px, a.fd_PQ);
                        off = (uint32_t)((n * a.K + k) * PQ + (px - n * PQ)) * ES;
                    }
                    e[j] = ld_elem<ES>(rdy, off);
                }
                ra[i] = pack<ES>(e);
            }
        }
    }

    DEVI void load_b(const KArgs &a, int kt, u32x4 *rb, int tid) const {
        const int px = pbeg + kt * BK + (tid & 63);
        const int pxq = px < pend ? px : pbeg;
        const int n = (int)fdiv((uint32_t)pxq, a.fd_PQ);
        const int pq = pxq - n * PQ;
        const int p = (int)fdiv((uint32_t)pq, a.fd_Q);
        const int q = pq - p * a.Q;
        int ih0 = p * a.sh - a.ph;
        const int iw0 = q * a.sw - a.pw;
        const int xb = n * a.C * HW + ih0 * a.W + iw0;
        if (px >= pend) ih0 = -(1 << 30);  // past the split's last pixel: contributes 0
#pragma unroll
        for (int i = 0; i < NVB; ++i) {
            const int col0 = n0 + uniform((tid >> 6) + 4 * i) * VEC;
            if (CVEC) {
                const int t = (int)fdiv((uint32_t)col0, a.fd_C), c0 = col0 - t * a.C;
                const int r = (int)fdiv((uint32_t)t, a.fd_S), s = t - r * a.S;
                const bool ok = col0 < TC && (unsigned)(ih0 + r) < (unsigned)a.H &&
                                (unsigned)(iw0 + s) < (unsigned)a.W;
                const uint32_t base = ok ? (uint32_t)(xb + c0 * HW + r * a.W + s) * ES : kOOB;
                uint32_t e[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) e[j] = ld_elem<ES>(rx, base + (uint32_t)(j * HW * ES));
                rb[i] = pack<ES>(e);
            } else {
                uint32_t e[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const int col = col0 + j;
                    const int t = (int)fdiv((uint32_t)col, a.fd_C), c = col - t * a.C;
                    const int r = (int)fdiv((uint32_t)t, a.fd_S), s = t - r * a.S;
                    const bool ok = col < TC && (unsigned)(ih0 + r) < (unsigned)a.H &&
                                    (unsigned)(iw0 + s) < (unsigned)a.W;
                    e[j] = ld_elem<ES>(rx, ok ? (uint32_t)(xb + c * HW + r * a.W + s) * ES : kOOB);
                }
                rb[i] = pack<ES>(e);
            }
        }
    }

    template <int PITCH>
    DEVI void store_b(const u32x4 *rb, char *sb, int tid) const {
        const int kidx = tid & 63;
#pragma unroll
        for (int i = 0; i < NVB; ++i) {
            char *p = sb + (((tid >> 6) + 4 * i) * VEC) * PITCH + kidx * ES;
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                if constexpr (ES == 4) {
                    *(uint32_t *)(p + j * PITCH) = rb[i][j];
                } else {
                    *(uint16_t *)(p + j * PITCH) = (uint16_t)(rb[i][j >> 1] >> (16 * (j & 1)));
                }
            }
        }
    }

    template <int WM, int TM, int TN>
    DEVI void epilogue(const KArgs &a, const f32x16 (&acc)[TM][TN], int wave, int lane, char *lds) const {
        constexpr int WN = 4 / WM, WTM = BM / WM, WTN = BN / WN;
        const int wm = wave % WM, wn = wave / WM, lr = lane & 31, lh = lane >> 5;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * WTN + j * 32 + lr;
            if (col >= TC) continue;
            const int t = (int)fdiv((uint32_t)col, a.fd_C), c = col - t * a.C;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int k = m0 + wm * WTM + i * 32 + acc_row(v, lh);
                    if (k >= a.K) continue;
                    if (a.direct)
                        out_store(a.out, ((size_t)k * a.C + c) * T + t, acc[i][j][v], a.epi, a.has_epi);
                    else
                        a.out[((size_t)z * a.K + k) * TC + col] = acc[i][j][v];
                }
        }
    }
};

// ------------------------------------------------------------------ main loop
template <int DT, int BM, int BN, int WM, int BKB, class Pass>
__global__ __launch_bounds__(256) void igemm_kernel(KArgs a) {
    constexpr int PITCH = BKB + 16, WN = 4 / WM, WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32, NPC = BKB / 32, VPR = BKB / 16;
    constexpr int STAGE = (BM + BN) * PITCH;
    __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    Pass pass;
    if (!pass.init(a, logical, tid)) return;

    u32x4 ra[Pass::NVA], rb[Pass::NVB];
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    auto store_a = [&](char *sa) {
#pragma unroll
        for (int i = 0; i < Pass::NVA; ++i) {
            const int v = tid + i * 256;
            if (BM * VPR < 256 * (i + 1) && v >= BM * VPR) continue;
            *(u32x4 *)(sa + (v / VPR) * PITCH + (v % VPR) * 16) = ra[i];
        }
    };

    const int nk = pass.nk;
    if (nk > 0) {
        pass.load_a(a, 0, ra, tid);
        pass.load_b(a, 0, rb, tid);
        store_a(lds);
        pass.template store_b<PITCH>(rb, lds + BM * PITCH, tid);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        char *cur = lds + (kt & 1) * STAGE;
        const bool more = kt + 1 < nk;
        if (more) {
            pass.load_a(a, kt + 1, ra, tid);
            pass.load_b(a, kt + 1, rb, tid);
        }
        mma_stage<DT, TM, TN, NPC, PITCH>(cur + (wave % WM) * WTM * PITCH,
                                          cur + BM * PITCH + (wave / WM) * WTN * PITCH, acc, lane);
        if (more) {
            char *nxt = lds + ((kt + 1) & 1) * STAGE;
            store_a(nxt);
            pass.template store_b<PITCH>(rb, nxt + BM * PITCH, tid);
        }
        __syncthreads();
    }
    pass.template epilogue<WM, TM, TN>(a, acc, wave, lane, lds);
}

// ------------------------------------------------------------------ small kernels
template <typename E>
__global__ __launch_bounds__(256) void filter_to_tck(const E *__restrict__ w, E *__restrict__ wt, int K,
                                                     int C, int T) {
    const long long total = (long long)K * C * T;
    for (long long e = blockIdx.x * 256LL + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
        const int t = (int)(e / ((long long)C * K));
        const int rem = (int)(e - (long long)t * C * K), c = rem / K, k = rem - c * K;
        wt[e] = w[((long long)k * C + c) * T + t];
    }
}

// Second stage of split-K: dW[k][c][t] = sum over splits z of part[z][k][t*C + c].
// A block covers 64 consecutive partial-sum positions with ZG waves (ZG =
// min(16, splits)); wave g sums the splits z = g, g + ZG, g + 2*ZG, ... in
// increasing order (eight independent loads in flight, added in that order),
// then the ZG wave sums are added in the fixed order g = 0, 1, ..., ZG-1.  The
// result does not depend on timing, so repeated calls are bitwise identical.
constexpr int kReduceGroups = 16;

__global__ __launch_bounds__(1024) void splitk_reduce(const float *__restrict__ part, float *__restrict__ dw,
                                                      int K, int C, int T, int splits, Epi ep, int has) {
    __shared__ float red[kReduceGroups][64];
    const int ZG = blockDim.x >> 6;
    const int TC = T * C;
    const long long total = (long long)K * TC;
    const int g = threadIdx.x >> 6, l = threadIdx.x & 63;
    const long long e = blockIdx.x * 64LL + l;
    float s = 0.0f;
    if (e < total) {
        const float *p = part + e;
        int z = g;
        for (; z + 7 * ZG < splits; z += 8 * ZG) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = p[(long long)(z + u * ZG) * total];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; z < splits; z += ZG) s += p[(long long)z * total];
    }
    red[g][l] = s;
    __syncthreads();
    if (g == 0 && e < total) {
        float v = red[0][l];
        for (int i = 1; i < ZG; ++i) v += red[i][l];
        const int k = (int)(e / TC), col = (int)(e - (long long)k * TC);
        const int t = col / C, c = col - t * C;
        out_store(dw, ((size_t)k * C + c) * T + t, v, ep, has);
    }
}

// The same order with 16-byte lanes: a block of 256 threads covers 64
// consecutive positions (16 lanes x 4); thread (g, l) sums splits g, g + 16,
// ... of its 4 positions in increasing order, sixteen loads in flight including
// the last partial batch (one batch for up to 256 splits), then thread j < 64
// adds the 16 group sums of position j in the order g = 0, 1, ..., 15 and
// writes it.  With at most 16 splits a group holds one split or none.
__global__ __launch_bounds__(256) void splitk_reduce_v4(const float4 *__restrict__ part, float *__restrict__ dw,
                                                        int K, int C, int T, int splits, Epi ep, int has) {
    constexpr int U = 16;
    __shared__ float red[kReduceGroups][64 + 4];
    const int TC = T * C;
    const long long total4 = (long long)K * TC / 4;
    const int g = threadIdx.x >> 4, l = threadIdx.x & 15;
    const long long e4 = blockIdx.x * 16LL + l;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (e4 < total4) {
        const float4 *p = part + e4;
        for (int z = g; z < splits; z += U * kReduceGroups) {
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = z + u * kReduceGroups < splits ? p[(long long)(z + u * kReduceGroups) * total4]
                                                      : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (z + u * kReduceGroups < splits) {
                    s.x += v[u].x;
                    s.y += v[u].y;
                    s.z += v[u].z;
                    s.w += v[u].w;
                }
        }
    }
    red[g][4 * l + 0] = s.x;
    red[g][4 * l + 1] = s.y;
    red[g][4 * l + 2] = s.z;
    red[g][4 * l + 3] = s.w;
    __syncthreads();
    const int j = threadIdx.x;
    const long long e = blockIdx.x * 64LL + j;
    if (j < 64 && e < total4 * 4) {
        const int ng = splits < kReduceGroups ? splits : kReduceGroups;
        float v = red[0][j];
        for (int i = 1; i < ng; ++i) v += red[i][j];
        const int k = (int)(e / TC), col = (int)(e - (long long)k * TC);
        const int t = col / C, c = col - t * C;
        out_store(dw, ((size_t)k * C + c) * T + t, v, ep, has);
    }
}

// Few splits: a thread adds 4 consecutive positions (one 16-byte load per
// split, all in flight) over z = 0, 1, ..., splits-1 in order.
__global__ __launch_bounds__(256) void splitk_reduce4(const float *__restrict__ part, float *__restrict__ dw, int K,
                                                      int C, int T, int splits, Epi ep, int has) {
    const int TC = T * C;
    const long long total = (long long)K * TC;
    const long long e = (blockIdx.x * 256LL + threadIdx.x) * 4;
    if (e >= total) return;
    const float4 *p = (const float4 *)(part + e);
    const long long zs = total / 4;
    float4 s = p[0];
#pragma unroll 8
    for (int z = 1; z < splits; ++z) {
        const float4 v = p[z * zs];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const long long ei = e + i;
        const int k = (int)(ei / TC), col = (int)(ei - (long long)k * TC);
        const int t = col / C, c = col - t * C;
        out_store(dw, ((size_t)k * C + c) * T + t, sv[i], ep, has);
    }
}

// Few splits, one filter row k per work-group: the row's partial sums
// [T][C] (C contiguous) are summed over z = 0, 1, ..., splits-1 in order with
// 16-byte loads, staged in LDS with a padded row stride, and written out as
// dW[k][C][T] (T contiguous) with consecutive lanes on consecutive addresses.
// Same additions in the same order as splitk_reduce4, so the same bits.
__global__ __launch_bounds__(256) void splitk_reduce_rows(const float4 *__restrict__ part, float *__restrict__ dw,
                                                          int K, int C, int T, int splits, Epi ep, int has) {
    extern __shared__ float slab[];   // [T][C + 1]
    const int k = blockIdx.x;
    const int TC4 = T * C / 4;
    const long long zs = (long long)K * TC4;   // float4s per split
    const float4 *p = part + (long long)k * TC4;
    for (int v = threadIdx.x; v < TC4; v += 256) {
        float4 acc = p[v];
        for (int z = 1; z < splits; ++z) {
            const float4 o = p[z * zs + v];
            acc.x += o.x;
            acc.y += o.y;
            acc.z += o.z;
            acc.w += o.w;
        }
        const int e = v * 4, t = e / C, c = e - t * C;   // C % 4 == 0: the 4 values share t
        float *row = slab + t * (C + 1) + c;
        row[0] = acc.x;
        row[1] = acc.y;
        row[2] = acc.z;
        row[3] = acc.w;
    }
    __syncthreads();
    const size_t row = (size_t)k * C * T;
    for (int o = threadIdx.x; o < C * T; o += 256) {
        const int c = o / T, t = o - c * T;
        out_store(dw, row + o, slab[t * (C + 1) + c], ep, has);
    }
}

int launch_splitk_reduce(const float *part, float *dw, int K, int C, int T, int splits, hipStream_t st,
                         const Epi *epi) {
    const long long total = (long long)K * C * T;
    Epi ep = {};
    if (epi) ep = *epi;
    const int has = epi ? 1 : 0;
    const size_t slab = (size_t)T * (C + 1) * sizeof(float);
    if (splits <= kReduceGroups && C % 4 == 0 && slab <= 64 * 1024 && ((uintptr_t)part & 15) == 0) {
        hipLaunchKernelGGL(splitk_reduce_rows, dim3((unsigned)K), dim3(256), slab, st, (const float4 *)part, dw, K,
                           C, T, splits, ep, has);
        return hipGetLastError() == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
    }
    if (splits <= kReduceGroups && total % 4 == 0 && ((uintptr_t)part & 15) == 0) {
        hipLaunchKernelGGL(splitk_reduce4, dim3((unsigned)((total / 4 + 255) / 256)), dim3(256), 0, st, part, dw, K, C,
                           T, splits, ep, has);
        return hipGetLastError() == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
    }
    const int zg = splits < kReduceGroups ? splits : kReduceGroups;
    if (total % 4 == 0 && ((uintptr_t)part & 15) == 0) {
        hipLaunchKernelGGL(splitk_reduce_v4, dim3((unsigned)((total / 4 + 15) / 16)), dim3(256), 0, st,
                           (const float4 *)part, dw, K, C, T, splits, ep, has);
        return hipGetLastError() == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
    }
    hipLaunchKernelGGL(splitk_reduce, dim3((unsigned)((total + 63) / 64)), dim3(64 * zg), 0, st, part, dw, K, C, T,
                       splits, ep, has);
    return hipGetLastError() == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
}

// ------------------------------------------------------------------ launch
template <int DT, int BM, int BN, int WM, int BKB, class Pass>
static hipError_t go(const KArgs &a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((igemm_kernel<DT, BM, BN, WM, BKB, Pass>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int DT, bool CV, int EPI>
static hipError_t fwd_tile(const Plan &pl, const KArgs &a, int grid, hipStream_t st) {
    if (pl.bm == 32) return go<DT, 32, 256, 1, 64, FwdPass<DT, 32, 256, 64, CV, EPI>>(a, grid, st);
    if (pl.bm == 64) return go<DT, 64, 256, 1, 64, FwdPass<DT, 64, 256, 64, CV, EPI>>(a, grid, st);
    return go<DT, 128, 128, 2, 64, FwdPass<DT, 128, 128, 64, CV, EPI>>(a, grid, st);
}

template <int DT, bool CV>
static hipError_t bwdd_tile(const Plan &pl, const KArgs &a, int grid, hipStream_t st) {
    if (pl.bm == 32) return go<DT, 32, 256, 1, 64, BwdDataPass<DT, 32, 256, 64, CV>>(a, grid, st);
    if (pl.bm == 64) return go<DT, 64, 256, 1, 64, BwdDataPass<DT, 64, 256, 64, CV>>(a, grid, st);
    return go<DT, 128, 128, 2, 64, BwdDataPass<DT, 128, 128, 64, CV>>(a, grid, st);
}

template <int DT, bool CV, bool PV>
static hipError_t bwdf_tile(const Plan &pl, const KArgs &a, int grid, hipStream_t st) {
    constexpr int BKB = DT ? 128 : 256;
    if (pl.bm == 64) return go<DT, 64, 128, 2, BKB, BwdFilterPass<DT, 64, 128, BKB, CV, PV>>(a, grid, st);
    return go<DT, 128, 128, 2, BKB, BwdFilterPass<DT, 128, 128, BKB, CV, PV>>(a, grid, st);
}

template <int DT>
static hipError_t run_gemm(const Plan &pl, const KArgs &a, int grid, hipStream_t st, int epi) {
    if (pl.pass == FWD) {
        if (epi == 2) return pl.cvec ? fwd_tile<DT, true, 2>(pl, a, grid, st) : fwd_tile<DT, false, 2>(pl, a, grid, st);
        if (epi == 1) return pl.cvec ? fwd_tile<DT, true, 1>(pl, a, grid, st) : fwd_tile<DT, false, 1>(pl, a, grid, st);
        return pl.cvec ? fwd_tile<DT, true, 0>(pl, a, grid, st) : fwd_tile<DT, false, 0>(pl, a, grid, st);
    }
    if (pl.pass == BWD_DATA)
        return pl.cvec ? bwdd_tile<DT, true>(pl, a, grid, st) : bwdd_tile<DT, false>(pl, a, grid, st);
    if (pl.cvec)
        return pl.pqvec ? bwdf_tile<DT, true, true>(pl, a, grid, st) : bwdf_tile<DT, true, false>(pl, a, grid, st);
    return pl.pqvec ? bwdf_tile<DT, false, true>(pl, a, grid, st) : bwdf_tile<DT, false, false>(pl, a, grid, st);
}

// Zeroes n floats (16-byte aligned start): one 16-byte store per thread.
__global__ __launch_bounds__(256) void fill_zero(float *__restrict__ p, long long n) {
    const long long i = (blockIdx.x * 256LL + threadIdx.x) * 4;
    if (i + 4 <= n) {
        *(float4 *)(p + i) = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
        for (long long j = i; j < n; ++j) p[j] = 0.f;
    }
}

// Output epilogue applied to a result of 0 at every dx element of a stride
// phase that no filter tap reaches (phase bit fh of live_h clear, or bit fw of
// live_w clear; the phase of row i is (i + ph) mod sh); the live phases are
// left to the GEMM, so every element is written exactly once.
__global__ __launch_bounds__(256) void fill_dead_phases(float *__restrict__ dx, Epi ep, int C, int H, int W, int ph,
                                                        int pw, int sh, int sw, unsigned live_h, unsigned live_w,
                                                        long long n) {
    for (long long e = blockIdx.x * 256LL + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
        const long long img = e / W;
        const int j = (int)(e - img * W);
        const long long ch = img / H;
        const int i = (int)(img - ch * H);
        const int c = (int)(ch % C);
        if (((live_h >> ((i + ph) % sh)) & 1u) && ((live_w >> ((j + pw) % sw)) & 1u)) continue;
        out_store(dx, (size_t)e, 0.0f, ep, 1, ep.bias ? ep.bias[c] : 0.0f);
    }
}

static int blocks_for(long long n) {
    long long b = (n + 255) / 256;
    return (int)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

int launch_plan(const Plan &pl, const Problem &p, const void *in0, const void *in1, float *out, void *ws,
                hipStream_t st, const Epi *epi) {
    const int es = p.dtype ? 2 : 4;
    const int T = p.R * p.S;
    KArgs a = {};
    a.a0 = in0;
    a.a1 = in1;
    a.out = out;
    a.N = p.N; a.C = p.C; a.H = p.H; a.W = p.W; a.K = p.K; a.R = p.R; a.S = p.S;
    a.ph = p.ph; a.pw = p.pw; a.sh = p.sh; a.sw = p.sw; a.P = p.P; a.Q = p.Q;
    a.m_tiles = pl.m_tiles;
    a.n_tiles = pl.n_tiles;
    a.nz = pl.nz;
    a.wt = pl.wt;
    a.fd_PQ = make_fdiv((uint32_t)(p.P * p.Q));
    a.fd_Q = make_fdiv((uint32_t)p.Q);
    a.fd_C = make_fdiv((uint32_t)p.C);
    a.fd_S = make_fdiv((uint32_t)p.S);
    a.fd_K = make_fdiv((uint32_t)p.K);
    if (epi) a.epi = *epi;
    a.has_epi = epi ? 1 : 0;
    // the forward selects its epilogue kernels at compile time; the backward
    // passes apply theirs per element at the store (out_store)
    const int epi_mode = epi && p.pass == FWD ? (epi->out_bf16 ? 2 : 1) : 0;
    const size_t nchw = (size_t)p.N * p.C * p.H * p.W, nkpq = (size_t)p.N * p.K * p.P * p.Q;
    const size_t kcrs = (size_t)p.K * p.C * T;
    hipError_t e = hipSuccess;

    if (pl.algo == ALGO_PATCH)
        return p.pass == BWD_FILTER ? launch_bwdf_patch(pl, p, in0, in1, out, ws, st, epi)
                                    : launch_patch(pl, p, in0, in1, out, ws, st, epi);
    if (pl.algo == ALGO_TINYC)
        return p.pass == BWD_FILTER ? launch_tinyc_bwdf(pl, p, in0, in1, out, ws, st, epi)
               : p.pass == FWD      ? launch_tinyc_fwd(pl, p, in0, in1, out, st, epi)
                                    : launch_tinyc(pl, p, in0, in1, out, st, epi);
    if (pl.algo == ALGO_POINTWISE) return launch_pointwise(pl, p, in0, in1, out, ws, st, epi);
    if (p.pass == FWD || p.pass == BWD_DATA) {
        a.a0_bytes = (uint32_t)((p.pass == FWD ? nchw : nkpq) * es);
        a.a1_bytes = (uint32_t)(kcrs * es);
        if (pl.wt && pl.wt_bytes > 0) {
            void *wt = (char *)ws + pl.wt_offset;
            const int blocks = blocks_for((long long)kcrs);
            if (p.pass == FWD) {
                if (es == 2)
                    hipLaunchKernelGGL(filter_to_ktc<uint16_t>, dim3(blocks), dim3(256), 0, st,
                                       (const uint16_t *)in1, (uint16_t *)wt, p.K, p.C, T);
                else
                    hipLaunchKernelGGL(filter_to_ktc<uint32_t>, dim3(blocks), dim3(256), 0, st,
                                       (const uint32_t *)in1, (uint32_t *)wt, p.K, p.C, T);
            } else {
                if (es == 2)
                    hipLaunchKernelGGL(filter_to_tck<uint16_t>, dim3(blocks), dim3(256), 0, st,
                                       (const uint16_t *)in1, (uint16_t *)wt, p.K, p.C, T);
                else
                    hipLaunchKernelGGL(filter_to_tck<uint32_t>, dim3(blocks), dim3(256), 0, st,
                                       (const uint32_t *)in1, (uint32_t *)wt, p.K, p.C, T);
            }
            if ((e = hipGetLastError()) != hipSuccess) return MICONV_ERR_HIP;
            a.a1 = wt;
        }
        if (p.pass == BWD_DATA && p.sh * p.sw <= 16) {
            // Phases that no filter tap reaches hold zeros only: zero all of dx with
            // coalesced stores and run the GEMM over the phases with taps.
            int live = 0;
            unsigned live_h = 0, live_w = 0;
            for (int fh = 0; fh < p.sh; ++fh)
                if (phase_dim(fh, p.sh, p.ph, p.H, p.R).nu > 0) live_h |= 1u << fh;
            for (int fw = 0; fw < p.sw; ++fw)
                if (phase_dim(fw, p.sw, p.pw, p.W, p.S).nu > 0) live_w |= 1u << fw;
            for (int fh = 0; fh < p.sh; ++fh)
                for (int fw = 0; fw < p.sw; ++fw)
                    if (((live_h >> fh) & 1u) && ((live_w >> fw) & 1u)) a.live_map[live++] = fh * p.sw + fw;
            if (live < p.sh * p.sw) {
                const long long n = (long long)nchw;
                if (epi)
                    hipLaunchKernelGGL(fill_dead_phases, dim3((unsigned)blocks_for(n)), dim3(256), 0, st, out, *epi,
                                       p.C, p.H, p.W, p.ph, p.pw, p.sh, p.sw, live_h, live_w, n);
                else
                    hipLaunchKernelGGL(fill_zero, dim3((unsigned)((n / 4 + 1 + 255) / 256)), dim3(256), 0, st, out,
                                       n);
                if ((e = hipGetLastError()) != hipSuccess) return MICONV_ERR_HIP;
                a.use_map = 1;
                a.nz = live;
                if (live == 0) return MICONV_OK;
            }
        }
        const int grid = pl.m_tiles * pl.n_tiles * a.nz;
        e = p.dtype ? run_gemm<1>(pl, a, grid, st, epi_mode) : run_gemm<0>(pl, a, grid, st, epi_mode);
        return e == hipSuccess ? MICONV_OK : MICONV_ERR_HIP;
    }

    // backward-filter
    a.a0_bytes = (uint32_t)(nchw * es);
    a.a1_bytes = (uint32_t)(nkpq * es);
    a.chunk = pl.chunk;
    a.direct = pl.splits == 1;
    float *part = pl.splits > 1 ? (float *)((char *)ws + pl.part_offset) : out;
    a.out = part;
    const int grid = pl.m_tiles * pl.n_tiles * pl.nz;
    e = p.dtype ? run_gemm<1>(pl, a, grid, st, epi_mode) : run_gemm<0>(pl, a, grid, st, epi_mode);
    if (e != hipSuccess) return MICONV_ERR_HIP;
    if (pl.splits > 1) return launch_splitk_reduce(part, out, p.K, p.C, T, pl.splits, st, epi);
    return MICONV_OK;
}

}  // namespace miconv
