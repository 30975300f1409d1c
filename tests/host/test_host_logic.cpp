// Host-only checks of the library's index helpers and plan selection, built
// with g++ and sanitizers by tests/test_abi_cpu.py (no HIP, no device code).
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <thread>
#include <vector>

#include "common.h"
#include "nd.h"
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

// Tiling invariants every plan (default or candidate) must satisfy.
static void check_plan_invariants(const miconv::Problem &p, const miconv::Plan &pl, size_t b) {
    using namespace miconv;
    size_t cap = b < 1000000000ull ? b : 1000000000ull;
    CHECK(pl.ws_used <= cap);
    CHECK((long long)pl.m_tiles * pl.bm >= pl.rows);
    if (p.pass == 2 && pl.algo == ALGO_PATCH) {
        // a work-group covers bn channels x all taps; split-K over bands of tr output rows
        CHECK((long long)pl.n_tiles * pl.bn == p.C);
        CHECK(pl.tr >= 1 && pl.tr <= p.P);
        long long bands = (long long)p.N * ((p.P + pl.tr - 1) / pl.tr);
        CHECK(pl.chunk > 0);
        CHECK((long long)pl.splits * pl.chunk >= bands);
        CHECK((long long)(pl.splits - 1) * pl.chunk < bands);
        CHECK(pl.splits == 1 || pl.part_bytes == (size_t)pl.splits * pl.rows * pl.cols * 4);
        if (pl.k16) CHECK((long long)p.P * p.Q % 4 == 0 && (long long)pl.tr * p.Q % 4 == 0 && p.R == 3 && p.S == 3);
        if (pl.stream) {
            // whole images; LDS of two work-groups per CU; the 128-row form with 4-byte fill loads
            CHECK(pl.k16 && pl.tr == p.P && !pl.pair);
            CHECK(bwdf16s_lds_bytes(pl.bm, pl.tr + p.R - 1, pl.pws) <= 78 * 1024);
            CHECK(pl.bm == 64 || pl.vw == 2);
            // fill schedule, event by event: image i's two fill steps start after the last
            // step reading image i - 2 and after image i - 1's fill; its second step must
            // precede the first step reading image i by at least two steps
            const long long PQ = (long long)p.P * p.Q;
            long long prev_end = -1;
            for (long long i = 2; i < 70 && i < pl.chunk; ++i) {
                const long long last_prev2 = ((i - 1) * PQ - 1) / 32;
                long long start = last_prev2 + 1;
                if (start <= prev_end) start = prev_end + 1;
                const long long end = start + 1;
                CHECK(end + 2 <= (i * PQ) / 32);
                prev_end = end;
            }
        }
    } else if (p.pass == 2 && pl.algo == ALGO_TINYC) {
        // few-channel MFMA kernel: runs of tc_rows output rows, one split each
        CHECK(p.dtype == 0 && p.K == 64 && p.C <= 4 && p.R == 7 && p.sw == 2 && p.C * p.R * p.S <= 160);
        CHECK(p.Q % 4 == 0 && p.Q <= 4 * kTcQT && 2 * (4 * kTcQT - 1) + p.S <= kTcXWP);
        const long long orows = (long long)p.N * p.P;
        CHECK(pl.tc_rows >= 1);
        CHECK((long long)pl.splits * pl.tc_rows >= orows);
        CHECK((long long)(pl.splits - 1) * pl.tc_rows < orows);
        CHECK(pl.splits == 1 || pl.part_bytes == (size_t)pl.splits * p.K * p.C * p.R * p.S * 4);
    } else if (p.pass == 2) {
        CHECK((long long)pl.n_tiles * pl.bn >= pl.cols);
        CHECK(pl.chunk % 64 == 0 && pl.chunk > 0);
        CHECK((long long)pl.splits * pl.chunk >= pl.red);
        CHECK((long long)(pl.splits - 1) * pl.chunk < pl.red);
        CHECK(pl.splits == 1 || pl.part_bytes == (size_t)pl.splits * pl.rows * pl.cols * 4);
        CHECK(pl.bm == 64 || pl.bm == 128);
    } else {
        CHECK((long long)pl.n_tiles * pl.bn >= pl.cols);
        if (pl.algo == ALGO_TINYC && p.pass == 0) {
            // forward MFMA form: runs of tc_rows output rows
            CHECK(p.dtype == 0 && p.K == 64 && p.C <= 4 && p.R == 7 && p.S >= 4 && p.sw == 2);
            CHECK(p.C * p.R * p.S <= 4 * kTcFwdSteps && p.Q <= 4 * kTcQT && 2 * (4 * kTcQT - 1) + p.S <= kTcXWP);
            CHECK(pl.tc_rows >= 1 && pl.ws_used == 0);
        }
        if (pl.tc_pairs) {
            // backward-data MFMA form: K of 32 or 64, the ring offsets stay below 2^32
            CHECK(pl.algo == ALGO_TINYC && p.pass == 1 && p.dtype == 0 && p.sh == 2 && p.sw == 2 && p.R == 7);
            CHECK(p.C * p.S <= 32 && p.Q <= 128 && (p.K == 32 || p.K == 64) && 124LL * p.P * p.Q < (1LL << 31));
            CHECK(pl.tc_pairs >= 1 && pl.tc_pairs <= (p.H + 1) / 2);
        }
        if (pl.algo == ALGO_IGEMM) CHECK((pl.bm == 32 && pl.bn == 256) || (pl.bm == 64 && pl.bn == 256) ||
                                         (pl.bm == 128 && pl.bn == 128));
        if (pl.algo == ALGO_PATCH) {
            const int Wi = p.pass == 0 ? p.W : p.Q;
            CHECK(pl.tr >= 1 && Wi % pl.vw == 0);
            CHECK(4LL * (pl.tr + p.R - 1) * (Wi / pl.vw) <= 512);
            if (pl.bm == 128 && !(p.R == 3 && p.S == 3)) CHECK(pl.vw <= 4);
        }
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
                    check_plan_invariants(p, pl, b);
                    // candidates: the default first, pairwise distinct, each a valid plan
                    Plan c[kMaxCandidates];
                    const int n = enumerate_plans(p, b, c, kMaxCandidates);
                    CHECK(n >= 1 && n <= kMaxCandidates);
                    CHECK(same_plan(c[0], pl));
                    for (int i = 0; i < n; ++i) {
                        check_plan_invariants(p, c[i], b);
                        for (int j = 0; j < i; ++j) CHECK(!same_plan(c[i], c[j]));
                    }
                }
    // wrong P/Q and bad sizes
    Problem bad = {0, 0, 2, 3, 8, 8, 4, 3, 3, 1, 1, 1, 1, 7, 8};
    CHECK(validate_problem(bad) == 3);
    bad.P = 8; bad.R = 11;
    CHECK(validate_problem(bad) == 2);
}

// The plan cache: default plans per budget, an installed plan used only where it
// fits the budget, removal and clearing; concurrent use from several threads.
static void check_plan_cache() {
    using namespace miconv;
    clear_plan_cache();
    Problem p = {2, 1, 256, 512, 14, 14, 512, 3, 3, 1, 1, 1, 1, 14, 14};
    Plan def, got, c[kMaxCandidates];
    make_plan(p, 1000000000ull, &def);
    cached_plan(p, (size_t)4 << 30, &got);   // budget capped at 1e9
    CHECK(same_plan(got, def));
    const int n = enumerate_plans(p, 1000000000ull, c, kMaxCandidates);
    CHECK(n >= 4);
    int pick = -1;   // a candidate that needs workspace and differs from the default
    for (int i = 1; i < n && pick < 0; ++i)
        if (c[i].ws_used > 0) pick = i;
    CHECK(pick > 0);
    if (pick > 0) {
        set_tuned_plan(p, c[pick]);
        cached_plan(p, 1000000000ull, &got);
        CHECK(same_plan(got, c[pick]));
        Plan small;
        make_plan(p, c[pick].ws_used - 1, &small);
        cached_plan(p, c[pick].ws_used - 1, &got);   // does not fit: the default for that budget
        CHECK(same_plan(got, small));
        int tuned = 0, total = 0;
        plan_cache_counts(&tuned, &total);
        CHECK(tuned == 1 && total >= 3);
        drop_tuned_plan(p);
        cached_plan(p, 1000000000ull, &got);
        CHECK(same_plan(got, def));
    }
    clear_plan_cache();
    int tuned = -1, total = -1;
    plan_cache_counts(&tuned, &total);
    CHECK(tuned == 0 && total == 0);
    // several threads planning, installing and clearing at once
    std::vector<std::thread> th;
    for (int t = 0; t < 8; ++t)
        th.emplace_back([t]() {
            for (int i = 0; i < 300; ++i) {
                Problem q = {i % 3, (i + t) % 2, 1 + (i % 5), 32, 14, 14, 64, 3, 3, 1, 1, 1, 1, 14, 14};
                Plan a, b;
                cached_plan(q, (size_t)(i % 7) << 20, &a);
                make_plan(q, (size_t)(i % 7) << 20, &b);
                if (t == 0 && i % 50 == 0) clear_plan_cache();
                if (t == 1 && i % 10 == 0) set_tuned_plan(q, b);
                if (t != 1) CHECK(same_plan(a, b) || a.ws_used <= ((size_t)(i % 7) << 20));
            }
        });
    for (auto &x : th) x.join();
    clear_plan_cache();
}

// Generalised problems: the output-size rule against brute force (count the window
// positions that fit), validation, the plan's split-K cover, and the 2-D mapping.
static void check_nd() {
    using namespace miconv;
    for (int in = 1; in <= 12; ++in)
        for (int f = 1; f <= 5; ++f)
            for (int lo = 0; lo <= 3; ++lo)
                for (int hi = 0; hi <= 3; ++hi)
                    for (int st = 1; st <= 3; ++st)
                        for (int dil = 1; dil <= 3; ++dil) {
                            int count = 0;   // windows o with every tap inside the padded extent
                            for (int o = 0; o * st + dil * (f - 1) < in + lo + hi; ++o) ++count;
                            CHECK(nd_out_dim(in, f, lo, hi, st, dil) == count);
                        }
    const int in[3] = {6, 9, 10}, f[3] = {3, 3, 2}, lo[3] = {1, 0, 1}, hi[3] = {1, 1, 0}, st[3] = {2, 1, 2},
              dil[3] = {1, 2, 1};
    int out[3];
    for (int d = 0; d < 3; ++d) out[d] = nd_out_dim(in[d], f[d], lo[d], hi[d], st[d], dil[d]);
    size_t budgets[] = {0, 1 << 16, 1 << 24, (size_t)4 << 30};
    for (int pass = 0; pass < 3; ++pass)
        for (int ndim = 1; ndim <= 3; ++ndim)
            for (int G : {1, 2, 4})
                for (size_t b : budgets) {
                    NdProblem p;
                    const int o = 3 - ndim;
                    CHECK(nd_from_desc(pass, 1, ndim, 3, 8, 12, G, in + o, f + o, out + o, lo + o, hi + o, st + o,
                                       dil + o, &p) == 0);
                    CHECK(validate_nd(p) == 0);
                    for (int d = 0; d < 3 - ndim; ++d) CHECK(p.in[d] == 1 && p.f[d] == 1 && p.out[d] == 1);
                    NdPlan pl;
                    make_nd_plan(p, b, &pl);
                    size_t cap = b < 1000000000ull ? b : 1000000000ull;
                    CHECK(pl.ws_used <= cap);
                    CHECK((long long)pl.m_tiles * pl.bm >= pl.rows && (long long)pl.n_tiles * pl.bn >= pl.cols);
                    CHECK(pl.chunk % pl.bk == 0 && pl.chunk > 0);
                    CHECK((long long)pl.splits * pl.chunk >= pl.red && (long long)(pl.splits - 1) * pl.chunk < pl.red);
                    CHECK(pl.splits == 1 || pass == 2);
                    CHECK(pl.splits == 1 || pl.part_bytes == (size_t)pl.splits * 12 * pl.cols * 4);
                    Problem q;
                    CHECK(!nd_as_2d(p, &q) || (G == 1 && ndim == 1));
                }
    // bad groups, wrong output size, plain 2-D mapping
    NdProblem p;
    int i2[2] = {7, 8}, f2[2] = {3, 3}, o2[2] = {7, 8}, l2[2] = {1, 1}, s2[2] = {1, 1}, d2[2] = {1, 1};
    CHECK(nd_from_desc(0, 0, 2, 2, 6, 4, 4, i2, f2, o2, l2, l2, s2, d2, &p) == 0 && validate_nd(p) == 2);
    CHECK(nd_from_desc(0, 0, 2, 2, 6, 4, 2, i2, f2, o2, l2, l2, s2, d2, &p) == 0 && validate_nd(p) == 0);
    o2[1] = 9;
    CHECK(nd_from_desc(0, 0, 2, 2, 6, 4, 2, i2, f2, o2, l2, l2, s2, d2, &p) == 0 && validate_nd(p) == 3);
    o2[1] = 8;
    CHECK(nd_from_desc(0, 0, 4, 2, 6, 4, 1, i2, f2, o2, l2, l2, s2, d2, &p) == 2);
    Problem q;
    CHECK(nd_from_desc(1, 1, 2, 2, 6, 4, 1, i2, f2, o2, l2, l2, s2, d2, &p) == 0 && nd_as_2d(p, &q));
    CHECK(q.pass == 1 && q.N == 2 && q.C == 6 && q.K == 4 && q.H == 7 && q.W == 8 && q.R == 3 && q.S == 3 &&
          q.ph == 1 && q.pw == 1 && q.P == 7 && q.Q == 8 && validate_problem(q) == 0);
    d2[0] = 2;
    o2[0] = 5;
    CHECK(nd_from_desc(1, 1, 2, 2, 6, 4, 1, i2, f2, o2, l2, l2, s2, d2, &p) == 0 && !nd_as_2d(p, &q));
    // padding modes
    int plo, phi, po;
    nd_padding(1, 13, 4, 2, 1, &plo, &phi, &po);
    CHECK(po == 7 && plo + phi == 3 && plo == 1 && nd_out_dim(13, 4, plo, phi, 2, 1) == 7);
    nd_padding(0, 13, 4, 2, 1, &plo, &phi, &po);
    CHECK(plo == 0 && phi == 0 && po == 5);
}

int main() {
    check_fdiv();
    check_phases();
    check_plans();
    check_plan_cache();
    check_nd();
    printf("%s (%d failures)\n", fails ? "FAILED" : "OK", fails);
    return fails ? 1 : 0;
}
