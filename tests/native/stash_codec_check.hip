// Host-side check of the BCJR stash codec and the normaliser rounding (bcjr.hpp), built
// for the CPU by the test suite: the same inline functions the kernels call.
//   - next_up(x) is the next binary32 above x (no float in between), for x of both signs,
//     zero, subnormals and the largest finite values;
//   - to_fix codes, read as unsigned: fixed point (0 .. 2^31) exactly for v in [-1024, 0],
//     equal to their definition 2^31 + rint(v 2^21) (ties to even, exact halves included),
//     tail codes (above 2^31) below; to_fix(0) = kFixZero;
//   - round trip: |from_fix(to_fix(v)) - v| <= 2^-22 in the fixed range and
//     <= 2^-24 (-1024 - v) (binary32 rounding of the distance) below it;
//   - the kernels' decode from_fix_shifted is the value plus kStashShift (exactly in the
//     fixed range, to one fp64 rounding in the tail);
//   - from_fix(to_fix(.)) is non-decreasing across the boundary at -1024.
// Prints "ok" and exits 0, or prints the first failure and exits 1.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "bcjr.hpp"

using qtcq::from_fix;
using qtcq::next_up;
using qtcq::to_fix;

static int fail(const char* what, double v, double a, double b)
{
    std::printf("FAIL %s: v=%.17g got=%.17g bound/other=%.17g\n", what, v, a, b);
    return 1;
}

int main()
{
    // next_up
    const float xs[] = {0.0f, -0.0f, 1e-45f, -1e-45f, 1.0f, -1.0f, 1024.0f, -1024.0f,
                        3.4e38f, -3.4e38f, 12345.678f, -98765.4f, 1.17549435e-38f};
    for (float x : xs) {
        const float u = next_up(x);
        if (!(u > x)) return fail("next_up above", x, u, x);
        if (std::nextafter(x, INFINITY) != u) return fail("next_up adjacent", x, u, std::nextafter(x, INFINITY));
    }
    if (next_up(INFINITY) != INFINITY) return fail("next_up inf", INFINITY, next_up(INFINITY), INFINITY);

    std::mt19937_64 rng(7);
    std::vector<double> vs = {0.0, -0.0, -1e-300, -2.3841857910156250e-07, -1.0, -1023.9999999,
                              -1024.0, -1024.0000000001, -1024.5, -1100.0, -2048.0, -1e5,
                              -3.3e9, -1e12, -1e30};
    // exact halves of the fixed-point unit: the ties of the rounding
    for (int k = 0; k < 4096; ++k) vs.push_back(-(k + 0.5) * 0x1p-21);
    for (int k = 0; k < 4096; ++k) vs.push_back(-1024.0 + (k + 0.5) * 0x1p-21);
    for (int i = 0; i < 200000; ++i) {
        const double mag = std::ldexp(1.0, (int)(rng() % 44)) * (double)(rng() >> 11) * 0x1p-53;
        vs.push_back(-mag);
        vs.push_back(-1024.0 - std::ldexp(1.0, -(int)(rng() % 40)) * (double)(rng() >> 11) * 0x1p-53);
        vs.push_back(-1024.0 + std::ldexp(1.0, -(int)(rng() % 40)) * (double)(rng() >> 11) * 0x1p-53);
    }
    if (to_fix(0.0) != qtcq::kFixZero || from_fix(qtcq::kFixZero) != 0.0)
        return fail("zero", 0.0, from_fix(qtcq::kFixZero), 0.0);
    for (double v : vs) {
        const int q = to_fix(v);
        const uint32_t u = (uint32_t)q;
        const double r = from_fix(q);
        const double rs = qtcq::from_fix_shifted(q);
        if (v >= -1024.0) {
            // the code is its definition: 2^31 + rint(v 2^21), ties to even
            const uint32_t def = 0x80000000u + (uint32_t)(int)std::nearbyint(v * 2097152.0);
            if (u != def) return fail("fixed code definition", v, u, def);
            if (u > 0x80000000u) return fail("fixed code range", v, u, 0x80000000u);
            if (std::fabs(r - v) > 0x1p-22) return fail("fixed round trip", v, r, 0x1p-22);
            if (rs - qtcq::kStashShift != r) return fail("fixed shifted decode", v, rs, r);
        } else {
            if (u <= 0x80000000u) return fail("tail code range", v, u, 0x80000000u);
            const double bound = 0x1p-24 * (-1024.0 - v);
            if (std::fabs(r - v) > bound) return fail("tail round trip", v, r, bound);
            if (std::fabs((rs - qtcq::kStashShift) - r) > 0x1p-52 * std::fabs(v))
                return fail("tail shifted decode", v, rs, r);
        }
    }
    // monotone across the boundary
    double prev = -1e300;
    for (double v = -1024.01; v <= -1023.99; v += 1.0 / 65536.0) {
        const double r = from_fix(to_fix(v));
        if (r < prev) return fail("monotone", v, r, prev);
        prev = r;
    }
    std::printf("ok\n");
    return 0;
}
