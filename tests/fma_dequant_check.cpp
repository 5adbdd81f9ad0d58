// Host check of wq_fma.h: wherever wq_fma_exact accepts (o, s), the one-FMA
// dequantization equals the formula's steps in binary32, bit for bit (a zero
// may change sign), for every code of the width.
//   RN(RN(code + o) * s)  against  fma(d, s_eff, RN(o * s))
// with d = 16 code and s_eff = s / 16 for int4 (the decode kernel's form),
// d = code and s_eff = s for int8.
// Usage: fma_dequant_check <int4|int8> <bf16|fp16> <floor scale: 1 or 0.5>
// Sweeps every finite o of T with scales at a stride through every finite s
// of T, then every finite s with offsets at a stride; prints
// "<accepted pairs> accepted, <mismatching pairs> mismatches".
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "wq_fma.h"

static float from_bits(uint32_t u)
{
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}
static uint32_t to_bits(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
}
// Exact value of a T bit pattern as binary32 (both fit).
static float t_value(uint16_t h, bool bf16)
{
    if (bf16)
        return from_bits(static_cast<uint32_t>(h) << 16);
    const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    float v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = std::ldexp(static_cast<float>(m), -24);
    else
        v = std::ldexp(static_cast<float>(1024 + m), e - 25);
    return sign ? -v : v;
}

struct Tally {
    uint64_t accepted = 0, mismatches = 0;
};

static void check_pair(float o, float s, bool int4, float lo, Tally& t)
{
    volatile float os_v = o * s;
    const float os = os_v;
    if (!dq::wq_fma_exact(o, s, os, lo))
        return;
    ++t.accepted;
    const int cmin = int4 ? -8 : -128, cmax = int4 ? 7 : 127;
    const float s_eff = int4 ? s * 0.0625f : s;
    for (int c = cmin; c <= cmax; ++c) {
        volatile float u = static_cast<float>(c) + o;  // RN(code + o)
        volatile float ref = u * s;                     // RN(RN(code + o) * s)
        const float d = int4 ? static_cast<float>(16 * c) : static_cast<float>(c);
        const float got = std::fmaf(d, s_eff, os);
        const uint32_t a = to_bits(ref), b = to_bits(got);
        const bool both_zero = ((a | b) & 0x7FFFFFFFu) == 0;
        const bool both_nan = std::isnan(static_cast<float>(ref)) && std::isnan(got);
        if (a != b && !both_zero && !both_nan) {
            ++t.mismatches;
            if (t.mismatches <= 3)
                std::fprintf(stderr, "mismatch o=%a s=%a c=%d ref=%a fma=%a\n", o, static_cast<float>(s), c,
                             static_cast<float>(ref), got);
            return;
        }
    }
}

int main(int argc, char** argv)
{
    if (argc != 4)
        return 2;
    const bool int4 = std::strcmp(argv[1], "int4") == 0;
    const bool bf16 = std::strcmp(argv[2], "bf16") == 0;
    const float lo = dq::wq_fma_offset_floor(int4, bf16) * static_cast<float>(std::atof(argv[3]));
    // int8 runs 256 codes per pair: a coarser stride keeps the sweep short.
    const int stride = int4 ? 61 : 509;
    const unsigned nthreads = std::thread::hardware_concurrency() ? std::thread::hardware_concurrency() : 4;
    std::vector<Tally> tallies(nthreads);
    std::vector<std::thread> pool;
    for (unsigned w = 0; w < nthreads; ++w) {
        pool.emplace_back([&, w] {
            Tally& t = tallies[w];
            for (uint32_t a = w; a < 65536; a += nthreads) {
                const float va = t_value(static_cast<uint16_t>(a), bf16);
                if (!std::isfinite(va))
                    continue;
                for (uint32_t b = a % stride; b < 65536; b += stride) {
                    const float vb = t_value(static_cast<uint16_t>(b), bf16);
                    if (!std::isfinite(vb))
                        continue;
                    check_pair(va, vb, int4, lo, t);  // every o, strided s
                    check_pair(vb, va, int4, lo, t);  // every s, strided o
                }
            }
        });
    }
    for (auto& th : pool)
        th.join();
    Tally all;
    for (const Tally& t : tallies) {
        all.accepted += t.accepted;
        all.mismatches += t.mismatches;
    }
    std::printf("%llu accepted, %llu mismatches\n", static_cast<unsigned long long>(all.accepted),
                static_cast<unsigned long long>(all.mismatches));
    return all.mismatches == 0 ? 0 : 1;
}
