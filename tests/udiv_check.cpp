// Host check of the launch-time division (exact_io_aware_07_amd/csrc/attn_udiv.h):
// udiv_apply(n, udiv_make(d)) must equal n / d for every divisor and dividend
// the forward kernel can meet (0 <= n < 2^31).  Exhaustive over small d and n,
// every power of two and its neighbours, and a fixed pseudo-random sample of
// large pairs.  Prints the number of mismatches; exit status 1 if any.
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "attn_udiv.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next31() {  // xorshift64*, top 31 bits
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 33);
}

static long bad = 0;
static void check(uint32_t n, uint32_t d) {
    const uint32_t got = attn::udiv_apply(n, attn::udiv_make(d));
    if (got != n / d) {
        if (bad < 10) printf("n=%u d=%u: got %u, want %u\n", n, d, got, n / d);
        ++bad;
    }
}

int main() {
    for (uint32_t d = 1; d <= 2048; ++d)
        for (uint32_t n = 0; n < 8192; ++n) check(n, d);
    for (uint32_t k = 0; k < 31; ++k) {
        const uint32_t p = 1u << k;
        for (uint32_t d : {p - 1, p, p + 1}) {
            if (d == 0) continue;
            for (uint32_t n : {0u, 1u, d - 1, d, d + 1, 0x7fffffffu, 0x7ffffffeu, 0x40000000u})
                if (n < 0x80000000u) check(n, d);
        }
    }
    for (int i = 0; i < 2000000; ++i) {
        const uint32_t d = 1 + next31() % (1u << (1 + next31() % 30));
        check(next31(), d);
        check(next31() % (64u * d + 1), d);
    }
    printf("mismatches %ld\n", bad);
    return bad ? 1 : 0;
}
