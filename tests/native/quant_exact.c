/*
 * Exactness checks of the fast fp32 quantiser of the HIP library's append
 * and tier kernels, on the CPU in IEEE single precision (no contraction, no
 * flush to zero), with the same operation sequence as the device code.
 *
 *  scale   s = fma(fma(-s0, qmax, r), C, s0), s0 = r * C, C = RN(1/qmax),
 *          must equal the correctly rounded r / qmax for every finite r >= 0
 *          (every fp32 bit pattern 0 .. 0x7F7FFFFF) at qmax 15 and 63.
 *  quotient q0 = x * rc, q1 = fma(fma(-q0, s, x), rc, q0) with rc within two
 *          ulps of 1 / s; when |q1 - rint(q1)| <= 0.5 - 2^-16 (the lane is not
 *          sent to correctly rounded division), rint(q1) must equal
 *          rint(RN(x / s)).  Checked on random scales and quotients, and on
 *          quotients placed at half-integers and a few ulps around them.
 *
 * Usage: quant_exact scale <qmax> <first> <count> [plain]   (bit patterns)
 *        quant_exact quotient <seed> <samples> [guard]
 * "plain" drops the fma correction (s = s0); a guard replaces the 0.5 -
 * 2^-16 bound, and a negative guard also drops the quotient's correction
 * (q1 = q0, no lane deferred): they exist to show that the checks catch a
 * mistake.
 * Prints "ok <checked>" or the first counterexample; exit status 0 / 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static int check_scale(int qmax, uint64_t first, uint64_t count, int plain)
{
    const float C = qmax == 63 ? 0x1.041042p-6f : 0x1.111112p-4f;
    const float fq = (float)qmax;
    if (C != (float)(1.0 / qmax)) { printf("C is not RN(1/qmax)\n"); return 1; }
    long bad = -1;
#pragma omp parallel for schedule(dynamic, 1 << 20) reduction(max : bad)
    for (int64_t i = 0; i < (int64_t)count; i++) {
        const uint32_t u = (uint32_t)(first + (uint64_t)i);
        if (u > 0x7F7FFFFFu) continue;
        const float r = from_bits(u);
        const float s0 = r * C;
        const float s = plain ? s0 : fmaf(fmaf(-s0, fq, r), C, s0);
        const float want = r / fq;
        if (bits_of(s) != bits_of(want) && (long)u > bad) bad = (long)u;
    }
    if (bad >= 0) {
        const float r = from_bits((uint32_t)bad);
        printf("scale mismatch at qmax %d, r = %a\n", qmax, r);
        return 1;
    }
    printf("ok %llu\n", (unsigned long long)count);
    return 0;
}

/* splitmix64 */
static uint64_t mix(uint64_t* x)
{
    uint64_t z = (*x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static float nudge(float x, int ulps)
{
    for (; ulps > 0; ulps--) x = nextafterf(x, INFINITY);
    for (; ulps < 0; ulps++) x = nextafterf(x, -INFINITY);
    return x;
}

static int check_quotient(uint64_t seed, int64_t samples, float guard)
{
    long fails = 0;
    int64_t checked = 0;
#pragma omp parallel for schedule(static) reduction(+ : fails, checked)
    for (int64_t i = 0; i < samples; i++) {
        uint64_t st = seed * 0x100000001B3ull + (uint64_t)i;
        const uint64_t a = mix(&st), b = mix(&st);
        /* a normal scale: exponent in [-100, 100], random mantissa */
        const float s = ldexpf(1.0f + (float)(a & 0x7FFFFF) / 8388608.0f, (int)((a >> 23) % 201) - 100);
        /* a quotient target in (-128, 128): either random, or a half-integer
           moved by a few ulps, where rounding is decided */
        float t;
        if (b & 1) {
            t = ((float)((b >> 1) & 0xFFFFFF) / 16777216.0f) * 255.0f - 127.5f;
        } else {
            const int k = (int)((b >> 1) % 255) - 127;
            t = nudge((float)k + 0.5f, (int)((b >> 9) % 9) - 4);
        }
        const float x = nudge(t * s, (int)((b >> 13) % 5) - 2);
        if (!isfinite(x)) continue;
        const float want = rintf(x / s);
        for (int e = -2; e <= 2; e++) {
            const float rc = nudge(1.0f / s, e);
            const float q0 = x * rc;
            const float q1 = guard < 0.0f ? q0 : fmaf(fmaf(-q0, s, x), rc, q0);
            const float r = rintf(q1);
            const int slow = guard < 0.0f ? 0 : !(fabsf(q1 - r) <= guard);
            checked++;
            if (!slow && r != want) fails++;
        }
    }
    if (fails) {
        printf("quotient: %ld wrong fast results\n", fails);
        return 1;
    }
    printf("ok %lld\n", (long long)checked);
    return 0;
}

int main(int argc, char** argv)
{
    if ((argc == 5 || argc == 6) && !strcmp(argv[1], "scale"))
        return check_scale(atoi(argv[2]), strtoull(argv[3], 0, 0), strtoull(argv[4], 0, 0),
                           argc == 6 && !strcmp(argv[5], "plain"));
    if ((argc == 4 || argc == 5) && !strcmp(argv[1], "quotient"))
        return check_quotient(strtoull(argv[2], 0, 0), strtoll(argv[3], 0, 0),
                              argc == 5 ? strtof(argv[4], 0) : 0.5f - 0x1p-16f);
    fprintf(stderr, "usage: quant_exact scale <qmax> <first> <count> | quotient <seed> <samples>\n");
    return 2;
}
