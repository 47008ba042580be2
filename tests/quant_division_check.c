/* Exhaustive check of the division scheme the FP8 quantiser's finite-block
 * path uses (DeepEP notes ch.7, s7.1: per-128-channel FP8 scales).  For every
 * finite bf16 block maximum amax (bit patterns 0 .. 0x7F7F), with
 * s = RN(max(amax, 1e-12) / 448) and y = RN(1 / s), and for every bf16 x of
 * either sign with |x| <= amax:
 *   q0 = RN(x * y), n = RN(q0 * s - x), q = RN(q0 - n * y)
 * (fused multiply-adds; n is the negated remainder, so that x = -0 gives
 * q = -0 without a sign fix) must equal the correctly rounded quotient
 * RN(x / s) bit for bit, unless both lie below 2^-11 in magnitude with the
 * same sign (the E4M3 code is then the signed zero either way).  The UE8M0 form,
 * x * 2^-k for the rounded-up power of two 2^k >= s, must equal x / 2^k
 * exactly.  Prints the number of pairs and of failures of each kind.
 * Plain C with IEEE binary32 arithmetic (no flush to zero, no contraction). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) {
    float v;
    memcpy(&v, &u, 4);
    return v;
}

static uint32_t to_bits(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    return u;
}

int main(void) {
    long long pairs = 0, bad_rcp = 0, bad_pow2 = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad_rcp, bad_pow2)
    for (int am = 0; am <= 0x7F7F; ++am) {
        const float amax = from_bits((uint32_t)am << 16);
        const float s = (amax > 1e-12f ? amax : 1e-12f) / 448.0f;
        const float y = 1.0f / s;
        uint32_t e = (to_bits(s) >> 23) & 0xFFu;
        if (to_bits(s) & 0x7FFFFFu)
            ++e;
        const float div2 = from_bits(e << 23), mul2 = from_bits((254u - e) << 23);
        for (uint32_t xb = 0; xb <= (uint32_t)am; ++xb) {
            for (uint32_t sign = 0; sign < 2; ++sign) {
                const float x = from_bits((xb | sign << 15) << 16);
                const float q = x / s;
                const float q0 = x * y;
                const float n = fmaf(q0, s, -x);
                const float q1 = fmaf(-n, y, q0);
                ++pairs;
                if (to_bits(q1) != to_bits(q) &&
                    !(fabsf(q) < 0x1p-11f && fabsf(q1) < 0x1p-11f && signbit(q) == signbit(q1)))
                    ++bad_rcp;
                if (to_bits(x * mul2) != to_bits(x / div2))
                    ++bad_pow2;
            }
        }
    }
    printf("%lld %lld %lld\n", pairs, bad_rcp, bad_pow2);
    return 0;
}
