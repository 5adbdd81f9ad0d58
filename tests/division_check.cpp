// division_check.cpp -- CPU check of the kernels' exact division steps.
//
// Compiles int4_quantization_amd/csrc/dq_div.h, the header the kernels use,
// on the host and compares it with IEEE division (aclnnDynamicQuantV2,
// Formula: every "/" is a correctly rounded binary32 division):
//   A. div_by_const(a, D, RN(1/D)) == RN(a / D) for every binary32 a in
//      [2^-100, FLT_MAX] and D in {7, 15, 127, 255} (all ~1.9e9 values each);
//   B. div_by_row(v, d, RN(1/d)) == RN(v / d) for d in [2^-60, 2^60] and
//      |v / d| >= 2^-40, on >= 1e8 pairs: divisors with random, all-ones and
//      near-all-ones mantissas, the range edges, quotients log-uniform in
//      [2^-45, 2^9] and quotients placed a few ulps around k + 1/2 and k;
//      below 2^-40 the rounded code (what the kernels use) must agree;
//   C. div_by(x, div_magic(d)) == x / d for x < 2^31: every d < 2^16 at the
//      multiples of d and their neighbours, and random larger d.
// Prints one line per part and exits nonzero on any mismatch.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "dq_div.h"

namespace {

inline float bits2f(uint32_t u)
{
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}
inline uint32_t f2bits(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
}

struct Rng {  // splitmix64
    uint64_t s;
    uint64_t next()
    {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    double unit() { return (next() >> 11) * 0x1p-53; }
};

template <typename F>
uint64_t parallel(int threads, uint64_t n, F body)
{
    std::vector<std::thread> pool;
    std::vector<uint64_t> bad(threads, 0);
    for (int t = 0; t < threads; ++t)
        pool.emplace_back([&, t] {
            const uint64_t lo = n * t / threads, hi = n * (t + 1) / threads;
            bad[t] = body(t, lo, hi);
        });
    for (auto& th : pool)
        th.join();
    uint64_t total = 0;
    for (uint64_t b : bad)
        total += b;
    return total;
}

// A: every binary32 a in [2^-100, FLT_MAX].
uint64_t part_a(int threads, uint64_t* checked, uint64_t* recip_differs)
{
    const uint32_t lo = f2bits(0x1p-100f), hi = 0x7F7FFFFFu;
    const float Ds[4] = {7.0f, 15.0f, 127.0f, 255.0f};
    uint64_t bad = 0;
    for (float D : Ds) {
        const float rD = 1.0f / D;
        bad += parallel(threads, uint64_t(hi - lo) + 1, [&](int, uint64_t b, uint64_t e) {
            uint64_t nb = 0;
            for (uint64_t i = b; i < e; ++i) {
                const float a = bits2f(static_cast<uint32_t>(lo + i));
                nb += f2bits(dq::div_by_const(a, D, rD)) != f2bits(a / D);
            }
            return nb;
        });
        // The same values expose a plain reciprocal product (sampled).
        for (uint64_t i = 0; i < (uint64_t{1} << 24); ++i) {
            const float a = bits2f(static_cast<uint32_t>(lo + i * 113));
            *recip_differs += f2bits(a * rD) != f2bits(a / D);
        }
        *checked += uint64_t(hi - lo) + 1;
    }
    return bad;
}

// B: per-row divisors.
uint64_t part_b(int threads, uint64_t pairs, uint64_t* checked, uint64_t* tiny_checked, uint64_t* recip_differs)
{
    std::vector<uint64_t> small(threads, 0), rdiff(threads, 0);
    const uint64_t bad = parallel(threads, pairs, [&](int t, uint64_t b, uint64_t e) {
        Rng g{0x5eed0000ull + 977 * t};
        uint64_t nb = 0;
        for (uint64_t i = b; i < e;) {
            // divisor: mantissa class by i, exponent uniform in [-60, 59]
            uint32_t mant;
            switch (g.next() % 6) {
            case 0: mant = 0x7FFFFFu; break;                             // all ones
            case 1: mant = 0x7FFFFFu - static_cast<uint32_t>(g.next() % 64); break;  // near all ones
            case 2: mant = static_cast<uint32_t>(g.next() % 64); break;  // near a power of two
            default: mant = static_cast<uint32_t>(g.next()) & 0x7FFFFFu;
            }
            const int ex = -60 + static_cast<int>(g.next() % 120);
            float d = std::ldexp(bits2f(0x3F800000u | mant), ex);
            const uint64_t edge = g.next() % 64;
            if (edge == 0)
                d = 0x1p-60f;
            else if (edge == 1)
                d = 0x1p60f;
            else if (edge == 2)
                d = std::nextafter(0x1p60f, 0.0f);
            else if (edge == 3)
                d = std::nextafter(0x1p-60f, 1.0f);
            if (!dq::row_divisor_in_range(d))
                continue;
            const float r = 1.0f / d;
            // 64 dividends per divisor
            for (int j = 0; j < 64 && i < e; ++j, ++i) {
                float v;
                const uint64_t kind = g.next() % 4;
                if (kind == 0) {  // quotient log-uniform in [2^-45, 2^9]
                    v = static_cast<float>(std::ldexp(1.0 + g.unit(), -45 + static_cast<int>(g.next() % 54)) * d);
                } else if (kind == 1 || kind == 2) {  // a few ulps around (k + 1/2) * d or k * d
                    const double k = static_cast<double>(g.next() % 300) + (kind == 1 ? 0.5 : 0.0);
                    const float c = static_cast<float>(k * d);
                    const int steps = static_cast<int>(g.next() % 9) - 4;
                    v = bits2f(static_cast<uint32_t>(static_cast<int64_t>(f2bits(c)) + steps));
                } else {  // arbitrary binary32 with |v / d| <= 2^9
                    v = static_cast<float>(g.unit() * 512.0 * d);
                }
                if (g.next() & 1)
                    v = -v;
                if (!std::isfinite(v))
                    continue;
                const float want = v / d;
                const float got = dq::div_by_row(v, d, r);
                if (std::fabs(want) >= 0x1p-40f) {
                    nb += f2bits(got) != f2bits(want);
                    rdiff[t] += f2bits(v * r) != f2bits(want);
                } else {
                    ++small[t];
                    nb += std::nearbyint(got) != std::nearbyint(want);
                }
            }
        }
        return nb;
    });
    *checked += pairs;
    for (uint64_t s : small)
        *tiny_checked += s;
    for (uint64_t s : rdiff)
        *recip_differs += s;
    return bad;
}

// C: integer division by a launch constant.
uint64_t part_c(int threads, uint64_t* checked)
{
    std::vector<uint64_t> cnt(threads, 0);
    const uint64_t nd = 65535;
    uint64_t bad = parallel(threads, nd, [&](int t, uint64_t b, uint64_t e) {
        uint64_t nb = 0;
        for (uint64_t d = b + 1; d <= e; ++d) {
            const dq::DivMagic m = dq::div_magic(d);
            const uint64_t kmax = (uint64_t{1} << 31) / d;
            const uint64_t step = kmax / 2000 + 1;
            for (uint64_t k = 0; k <= kmax + 1; k += step) {
                for (int64_t off = -2; off <= 2; ++off) {
                    const int64_t x = static_cast<int64_t>(k * d) + off;
                    if (x < 0 || x >= (int64_t{1} << 31))
                        continue;
                    ++cnt[t];
                    nb += dq::div_by(static_cast<uint32_t>(x), m) != static_cast<uint64_t>(x) / d;
                }
            }
            const uint32_t top = 0x7FFFFFFFu;
            ++cnt[t];
            nb += dq::div_by(top, m) != top / d;
        }
        return nb;
    });
    bad += parallel(threads, 1u << 22, [&](int t, uint64_t b, uint64_t e) {
        Rng g{0xd1d0000ull + 131 * t};
        uint64_t nb = 0;
        for (uint64_t i = b; i < e; ++i) {
            const uint64_t d = 1 + g.next() % (uint64_t{1} << (16 + g.next() % 17));
            const dq::DivMagic m = dq::div_magic(d);
            for (int j = 0; j < 8; ++j) {
                uint64_t x = g.next() & 0x7FFFFFFFu;
                if (j == 0)
                    x = 0x7FFFFFFFu;
                else if (j == 1 && d <= 0x7FFFFFFFu)
                    x = (0x7FFFFFFFu / d) * d - 1;
                ++cnt[t];
                nb += dq::div_by(static_cast<uint32_t>(x), m) != x / d;
            }
        }
        return nb;
    });
    for (uint64_t c : cnt)
        *checked += c;
    return bad;
}

}  // namespace

int main(int argc, char** argv)
{
    int threads = static_cast<int>(std::thread::hardware_concurrency());
    threads = threads < 1 ? 1 : threads > 16 ? 16 : threads;
    const uint64_t pairs = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 120000000ull;
    uint64_t ca = 0, cb = 0, cbt = 0, cc = 0, ra = 0, rb = 0;
    const uint64_t ba = part_a(threads, &ca, &ra);
    std::printf("A div_by_const: %llu values, %llu mismatches (reciprocal product alone: %llu of 2^26 sampled differ)\n",
                (unsigned long long)ca, (unsigned long long)ba, (unsigned long long)ra);
    const uint64_t bb = part_b(threads, pairs, &cb, &cbt, &rb);
    std::printf("B div_by_row: %llu pairs (%llu with |q| < 2^-40), %llu mismatches (reciprocal product alone: %llu differ)\n",
                (unsigned long long)cb, (unsigned long long)cbt, (unsigned long long)bb, (unsigned long long)rb);
    const uint64_t bc = part_c(threads, &cc);
    std::printf("C div_magic: %llu divisions, %llu mismatches\n", (unsigned long long)cc, (unsigned long long)bc);
    // Inputs that never exposed the uncorrected product would prove nothing.
    return (ba || bb || bc || ra == 0 || rb == 0) ? 1 : 0;
}
