// device.h -- device-side helpers shared by the HIP kernels (buffer loads,
// MFMA fragment types, work-group to XCD mapping).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MICONV_DEVICE_CODE 1
#include "common.h"

namespace miconv {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

#define DEVI __device__ __forceinline__

static constexpr uint32_t kOOB = 0x80000000u;

DEVI rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

template <int ES>
DEVI uint32_t ld_elem(rsrc_t r, uint32_t off);
template <>
DEVI uint32_t ld_elem<4>(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
template <>
DEVI uint32_t ld_elem<2>(rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
DEVI u32x2 ld_b64(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
DEVI u32x4 ld_vec(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
// 16-byte load at voff + soff (soff work-group-uniform; it takes no part in the
// range check, so only for addresses known to be in range)
DEVI u32x4 ld_vec_s(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

// Packs VEC loaded elements (low bits) into one 16-byte vector.
template <int ES>
DEVI u32x4 pack(const uint32_t *e);
template <>
DEVI u32x4 pack<4>(const uint32_t *e) {
    return u32x4{e[0], e[1], e[2], e[3]};
}
template <>
DEVI u32x4 pack<2>(const uint32_t *e) {
    return u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
}

DEVI uint32_t fdiv(uint32_t n, const FDiv &f) { return f.m == 0 ? n : (__umulhi(n, f.m) >> f.s); }

DEVI int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Work-groups are dispatched to the 8 XCDs round-robin; give each XCD one
// contiguous range of tiles so neighbouring tiles (which share an operand
// panel) share that XCD's L2.
DEVI int xcd_remap(int h, int total) {
    const int full = total & ~7;
    if (h >= full) return h;
    return (h & 7) * (full >> 3) + (h >> 3);
}

// ------------------------------------------------------------------ MFMA tile
template <int DT, int TM, int TN, int NPC, int PITCH>
DEVI void mma_stage(const char *sa, const char *sb, f32x16 (&acc)[TM][TN], int lane) {
    const int lr = lane & 31, lh = lane >> 5;
    const char *pa = sa + lr * PITCH + lh * (NPC * 16);
    const char *pb = sb + lr * PITCH + lh * (NPC * 16);
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc) {
        u32x4 fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = *(const u32x4 *)(pa + i * 32 * PITCH + pc * 16);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = *(const u32x4 *)(pb + j * 32 * PITCH + pc * 16);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (DT == 1) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, fa[i]), __builtin_bit_cast(bf16x8, fb[j]), acc[i][j], 0, 0, 0);
                } else {
                    // cast whole vectors: a bit_cast of one subscripted element was lowered
                    // to element 0 for every subscript
                    const f32x4 af = __builtin_bit_cast(f32x4, fa[i]), bf = __builtin_bit_cast(f32x4, fb[j]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], bf[e], acc[i][j], 0, 0, 0);
                }
            }
    }
}

// Fused forward epilogue of one output: `bias` is the row's bias (0 without
// one), `old` the previous output, used only when beta != 0.  The callers load
// both before issuing any of the tile's stores: loads and stores share the
// in-order vector memory counter, so a load issued after a store could only be
// waited for once that store had completed.
DEVI float epi_apply(const Epi &e, float acc, float bias, float old) {
    float v = e.alpha * acc;
    if (e.beta != 0.0f) v += e.beta * old;
    v += bias;
    return e.relu ? fmaxf(v, 0.0f) : v;
}

// fp32 -> bf16 with round to nearest, ties to even (the upper 16 bits after
// adding 0x7fff plus the lowest kept bit); NaN stays a quiet NaN.
DEVI uint16_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
DEVI float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// One-element output epilogue at element i of `out` (the backward passes and
// the deconvolution forward): out[i] = act(alpha * v + beta * out[i] + bias),
// out[i] read only when beta != 0, stored as fp32 or, with e.out_bf16, as bf16
// rounded to nearest even.  Without an epilogue (has == 0) v is stored as it is.
DEVI void out_store(void *out, size_t i, float v, const Epi &e, int has, float bias = 0.0f) {
    if (!has) {
        ((float *)out)[i] = v;
        return;
    }
    if (e.out_bf16) {
        uint16_t *o = (uint16_t *)out;
        const float old = e.beta != 0.0f ? bf16_to_f32(o[i]) : 0.0f;
        o[i] = f32_to_bf16(epi_apply(e, v, bias, old));
    } else {
        float *o = (float *)out;
        const float old = e.beta != 0.0f ? o[i] : 0.0f;
        o[i] = epi_apply(e, v, bias, old);
    }
}

// Row (within the 32x32 block) held by accumulator register v of a lane in half lh.
DEVI int acc_row(int v, int lh) { return (v >> 2) * 8 + lh * 4 + (v & 3); }

// Tap-major filter copies.  fwd: wt[k][t][c] = w[k][c][t]; bwd-data: wt[t][c][k] = w[k][c][t].
template <typename E>
__global__ __launch_bounds__(256) void filter_to_ktc(const E *__restrict__ w, E *__restrict__ wt, int K,
                                                     int C, int T) {
    const long long total = (long long)K * C * T;
    for (long long e = blockIdx.x * 256LL + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
        const long long k = e / ((long long)T * C);
        const int rem = (int)(e - k * T * C), t = rem / C, c = rem - t * C;
        wt[e] = w[(k * C + c) * T + t];
    }
}

}  // namespace miconv
