// The kernels divide tile indices by launch constants with the multiply and
// shift of attn::make_fast_div; this checks that quotient against plain
// division for every divisor up to 5000 and a spread of larger ones, on all
// numerators below 20000, on each divisor's largest multiples below 2^31 and
// their neighbours, and on a sample across [0, 2^31).
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
    return bad != 0;
}
