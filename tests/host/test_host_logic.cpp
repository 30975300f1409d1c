// Host-only checks of the library's index helpers and plan selection, built
// with g++ and sanitizers by tests/test_abi_cpu.py (no HIP, no device code).
#include <stdio.h>
#include <stdlib.h>

#include <random>

#include "common.h"
#include "plan.h"

static int fails = 0;
#define CHECK(c)                                                    \
    do {                                                            \
        if (!(c)) {                                                 \
            if (fails < 20) printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); \
            ++fails;                                                \
        }                                                           \
    } while (0)

static void check_fdiv() {
    std::mt19937_64 g(1234);
    const uint32_t top = 0x7fffffffu;
    for (uint32_t d = 1; d < 70000; d += (d < 4096 ? 1 : 97)) {
        FDiv f = make_fdiv(d);
        uint32_t ns[] = {0, 1, d - 1, d, d + 1, 2 * d - 1, top, top - 1, top - d};
        for (uint32_t n : ns)
            if (n <= top) CHECK(fdiv_host(n, f) == n / d);
        for (int i = 0; i < 200; ++i) {
            uint32_t n = (uint32_t)(g() & top);
            CHECK(fdiv_host(n, f) == n / d);
        }
    }
    for (int i = 0; i < 20000; ++i) {
        uint32_t d = (uint32_t)(g() % top) + 1, n = (uint32_t)(g() & top);
        CHECK(fdiv_host(n, make_fdiv(d)) == n / d);
    }
}

// Stride-phase geometry against brute force: every input row i is in exactly one
// phase, and for each tap r the output row p = (i + pad - r) / stride is visited
// iff the division is exact, through p = base + a - u.
static void check_phases() {
    for (int stride = 1; stride <= 4; ++stride)
        for (int pad = 0; pad <= 4; ++pad)
            for (int filt = 1; filt <= 7; ++filt)
                for (int in = 1; in <= 12; ++in) {
                    int seen[64] = {0};
                    for (int f = 0; f < stride; ++f) {
                        PhaseDim d = phase_dim(f, stride, pad, in, filt);
                        for (int a = 0; a < d.na; ++a) {
                            int i = d.i0 + stride * a;
                            CHECK(i >= 0 && i < in);
                            CHECK((i + pad) % stride == f);
                            seen[i]++;
                            int taps = 0;
                            for (int u = 0; u < d.nu; ++u) {
                                int r = f + stride * u;
                                CHECK(r < filt);
                                CHECK(d.base + a - u == (i + pad - r) / stride);
                                CHECK((i + pad - r) % stride == 0 || i + pad - r < 0);
                                ++taps;
                            }
                            int brute = 0;
                            for (int r = 0; r < filt; ++r)
                                if ((i + pad - r) % stride == 0 || (i + pad - r < 0 && (r - i - pad) % stride == 0))
                                    ++brute;
                            CHECK(taps == brute);
                        }
                    }
                    for (int i = 0; i < in; ++i) CHECK(seen[i] == 1);
                }
}

static void check_plans() {
    using namespace miconv;
    int shapes[][13] = {
        {2, 3, 8, 8, 4, 3, 3, 1, 1, 1, 1, 8, 8},
        {64, 64, 56, 56, 64, 3, 3, 1, 1, 1, 1, 56, 56},
        {64, 256, 56, 56, 512, 1, 1, 0, 0, 2, 2, 28, 28},
        {32, 3, 224, 224, 64, 7, 7, 3, 3, 2, 2, 112, 112},
        {32, 128, 32, 32, 256, 4, 4, 1, 1, 2, 2, 16, 16},
        {256, 512, 14, 14, 512, 3, 3, 1, 1, 1, 1, 14, 14},
        {1, 1, 2060, 300, 500, 5, 300, 0, 0, 1, 1, 2056, 1},
    };
    size_t budgets[] = {0, 1000, 1 << 20, 64u << 20, (size_t)4 << 30};
    for (auto &s : shapes)
        for (int pass = 0; pass < 3; ++pass)
            for (int dt = 0; dt < 2; ++dt)
                for (size_t b : budgets) {
                    Problem p = {pass, dt, s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7], s[8], s[9], s[10], s[11], s[12]};
                    CHECK(validate_problem(p) == 0);
                    Plan pl;
                    make_plan(p, b, &pl);
                    size_t cap = b < 1000000000ull ? b : 1000000000ull;
                    CHECK(pl.ws_used <= cap);
                    CHECK((long long)pl.m_tiles * pl.bm >= pl.rows);
                    if (pass == 2 && pl.algo == ALGO_PATCH) {
                        // a work-group covers bn channels x all taps; split-K over bands of tr output rows
                        CHECK((long long)pl.n_tiles * pl.bn == p.C);
                        CHECK(pl.tr >= 1 && pl.tr <= p.P);
                        long long bands = (long long)p.N * ((p.P + pl.tr - 1) / pl.tr);
                        CHECK(pl.chunk > 0);
                        CHECK((long long)pl.splits * pl.chunk >= bands);
                        CHECK((long long)(pl.splits - 1) * pl.chunk < bands);
                        CHECK(pl.splits == 1 || pl.part_bytes == (size_t)pl.splits * pl.rows * pl.cols * 4);
                    } else if (pass == 2) {
                        CHECK((long long)pl.n_tiles * pl.bn >= pl.cols);
                        CHECK(pl.chunk % 64 == 0 && pl.chunk > 0);
                        CHECK((long long)pl.splits * pl.chunk >= pl.red);
                        CHECK((long long)(pl.splits - 1) * pl.chunk < pl.red);
                        CHECK(pl.splits == 1 || pl.part_bytes == (size_t)pl.splits * pl.rows * pl.cols * 4);
                    } else {
                        CHECK((long long)pl.n_tiles * pl.bn >= pl.cols);
                    }
                }
    // wrong P/Q and bad sizes
    Problem bad = {0, 0, 2, 3, 8, 8, 4, 3, 3, 1, 1, 1, 1, 7, 8};
    CHECK(validate_problem(bad) == 3);
    bad.P = 8; bad.R = 11;
    CHECK(validate_problem(bad) == 2);
}

int main() {
    check_fdiv();
    check_phases();
    check_plans();
    printf("%s (%d failures)\n", fails ? "FAILED" : "OK", fails);
    return fails ? 1 : 0;
}
