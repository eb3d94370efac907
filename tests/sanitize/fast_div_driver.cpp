// The kernels divide tile indices by launch constants with the multiply and
// shift of attn::make_fast_div; this checks that quotient against plain
// division for every divisor up to 5000 and a spread of larger ones, on all
// numerators below 20000, on each divisor's largest multiples below 2^31 and
// their neighbours, and on a sample across [0, 2^31).  It also checks the
// host's rule for the chained sweep (attn::fwd_chained) on launches at and
// around each of its limits.
#include <cstdint>
#include <cstdio>

#include "attn_params.h"

int main() {
    unsigned long long checked = 0, bad = 0;
    for (uint32_t d = 1; d <= 70000; d = d < 5000 ? d + 1 : d * 3 / 2 + 1) {
        const attn::FastDiv f = attn::make_fast_div(d);
        auto quot = [&](uint32_t n) {
            const uint32_t hi = (uint32_t)(((unsigned long long)n * f.mul) >> 32);
            return (hi + n) >> f.shift;
        };
        auto check = [&](uint32_t n) {
            ++checked;
            if (quot(n) != n / d && bad++ < 5) std::printf("d %u n %u: %u\n", d, n, quot(n));
        };
        for (uint32_t n = 0; n < 20000; ++n) check(n);
        for (unsigned long long j = 1; j < 2000; ++j) check((uint32_t)(j * 1000003ull * d % 2147483648ull));
        const uint32_t top = 2147483647u / d;
        for (uint32_t m = top; m > 0 && m + 50 > top; --m) {
            check(m * d);
            check(m * d - 1);
            if ((unsigned long long)m * d + d - 1 < 2147483648ull) check(m * d + d - 1);
        }
        check(2147483647u);
    }
    std::printf("checked %llu quotients, %llu wrong\n", checked, bad);
    if (bad == 0) std::printf("all quotients exact\n");

    // the chained-sweep rule: (causal, d_qk, d_v, Lk, tiles, grid, splits, split output)
    struct Case {
        bool causal;
        int dqk, dv, Lk, units, n_m, grid, n_split, part;
        bool want;
    };
    const Case cases[] = {
        {false, 128, 128, 2048, 256, 8, 256, 1, 0, true},     // mha_l2k: 32 blocks
        {true, 128, 128, 2048, 256, 8, 256, 1, 0, false},     // causal
        {false, 192, 128, 2048, 256, 8, 256, 1, 0, false},    // unequal head dims
        {false, 128, 128, 1152, 256, 8, 256, 1, 0, true},     // 18 blocks, the fewest at d = 128
        {false, 128, 128, 1088, 256, 8, 256, 1, 0, false},    // 17 blocks
        {false, 128, 128, 1090, 256, 8, 256, 1, 0, true},     // 18 blocks, the last with 2 keys
        {false, 128, 128, 1216, 256, 8, 256, 1, 0, false},    // 19 blocks: odd
        {false, 64, 64, 640, 256, 8, 256, 1, 0, true},        // 10 blocks, the fewest at d = 64
        {false, 64, 64, 576, 256, 8, 256, 1, 0, false},       // 9 blocks
        {false, 128, 128, 2048, 256, 8, 256, 4, 1, false},    // key splits into fp32 states
        {false, 128, 128, 2048, 256, 8, 256, 1, 1, false},    // one split, fp32 state output
        {false, 64, 64, 1 << 23, 1 << 20, 1, 256, 1, 0, false},  // the sweep's count past 2^29
        {false, 64, 64, 1 << 16, 1 << 12, 1, 256, 1, 0, true},   // 17 tiles x 1024 blocks
    };
    int rule_bad = 0;
    for (const Case& c : cases) {
        attn::FwdParams p{};
        p.Lk = c.Lk;
        p.units = c.units;
        p.n_m = c.n_m;
        p.grid = c.grid;
        p.n_split = c.n_split;
        float part = 0.0f;
        p.o_part = c.part ? &part : nullptr;
        const bool got = attn::fwd_chained(p, c.dqk, c.dv, c.causal);
        if (got != c.want) {
            ++rule_bad;
            std::printf("fwd_chained(causal %d, d %d/%d, Lk %d, units %d) = %d\n", c.causal, c.dqk,
                        c.dv, c.Lk, c.units, got);
        }
    }
    if (rule_bad == 0) std::printf("chained-sweep rule as stated\n");
    return bad != 0 || rule_bad != 0;
}
