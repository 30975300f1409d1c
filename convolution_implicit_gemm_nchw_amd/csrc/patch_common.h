// patch_common.h -- pieces shared by the stride-1 LDS-patch kernels: the patch
// fill (global row loads, 8x8 register transposes, LDS stores), the output tile
// descriptor and a compile-time loop helper.
#pragma once
#include <type_traits>

#include "device.h"

namespace miconv {

namespace patchfill {

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

// The octet is the fastest index: the 4 lanes of one column group store the 4
// 16-byte quarters of the same positions, which spreads a store instruction
// over more LDS banks than a column-group-fastest order.
DEVI ItemPos item_pos(int it, int nitems, int G, int PR) {
    ItemPos q;
    q.ok = it < nitems;
    const int itq = q.ok ? it : 0;
    q.o = itq & 3;
    const int rest = itq >> 2;
    q.g = rest % G;
    q.pr = rest / G;
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

}  // namespace patchfill
using namespace patchfill;

// One output tile: filter rows m0 .. m0+BM-1, output rows p0 .. p0+TR-1 of image n
// (npx = valid pixels; the last row band of an image may be short).
struct Tile {
    int n, p0, m0, npx;
    int ph;   // stride phase (backward-data by phases), else 0
};

template <int I, int N, typename F>
DEVI void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>());
        static_for<I + 1, N>(f);
    }
}

}  // namespace miconv
