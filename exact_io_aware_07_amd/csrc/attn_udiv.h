// Integer division by a divisor fixed at launch time (internal to libattn.so).
//
// The forward kernel maps its workgroup index to (query tile, sequence, head)
// with a few divisions by launch constants.  Done in the kernel, each one is a
// float-reciprocal sequence with a vector-to-scalar round trip; here the host
// computes a multiplier once and the kernel takes a multiply-high, an add and
// a shift.  Round-up method with a 33-bit multiplier 2^32 + m (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// for d >= 1 let l = ceil(log2 d) and m' = floor(2^(32+l) / d) + 1; then
// m'd - 2^(32+l) lies in (0, d], which is at most 2^l, and that makes
// floor(n m' / 2^(32+l)) equal floor(n / d) for every 0 <= n < 2^32.  With
// m = m' - 2^32 (it fits in 32 bits) the quotient is
// (mulhi(n, m) + n) >> l, and for n < 2^31 the sum cannot overflow.
//
// Plain C++ (no HIP headers): the device code and the host-side check in the
// tests compile the same functions.
#pragma once

#include <stdint.h>

namespace attn {

struct UDiv {
    uint32_t m = 0;  // multiplier minus 2^32
    uint32_t l = 0;  // ceil(log2 d)
};

// Multiplier and shift for divisor d, 1 <= d < 2^31 (the launchers pass head
// and sequence counts).  Values outside are clamped into that range so that
// the shifts below stay defined; a launch that could use them is refused
// before it starts.
inline UDiv udiv_make(uint32_t d) {
    if (d == 0) d = 1;
    if (d > 0x7fffffffu) d = 0x7fffffffu;
    uint32_t l = 0;
    while ((uint64_t{1} << l) < d) ++l;
    const uint64_t mp = ((uint64_t{1} << (32 + l)) / d) + 1;
    return UDiv{(uint32_t)(mp - (uint64_t{1} << 32)), l};
}

// floor(n / d) for 0 <= n < 2^31.
constexpr uint32_t udiv_apply(uint32_t n, UDiv q) {
    return (uint32_t)((((uint64_t)n * q.m) >> 32) + n) >> q.l;
}

}  // namespace attn
