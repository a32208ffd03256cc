/* Exhaustive check of the oracle's binary32 -> bfloat16 rounding against an
 * independent nearest-neighbour selector evaluated in double precision.
 * For every one of the 2^32 bit patterns:
 *   - NaN must map to a quiet NaN of the same sign;
 *   - otherwise the result must be the nearer of the two bfloat16 values that
 *     bracket |x| (the truncation and the next value away from zero, the
 *     value after the largest finite one standing for 2^128, i.e. overflow to
 *     infinity), with a tie going to the one whose last mantissa bit is 0.
 * Prints the number of mismatches and exits non-zero if there is any. */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint16_t oracle_bf16_rne(uint32_t u);

static double bf16_mag_value(uint32_t mag16) {
    /* magnitude bits (no sign) of a bfloat16 -> double; 0x7F80 stands for 2^128 */
    if (mag16 == 0x7F80u) return ldexp(1.0, 128);
    uint32_t u = mag16 << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static uint16_t select_nearest(uint32_t u) {
    uint32_t sign = u & 0x80000000u;
    uint32_t mag = u & 0x7FFFFFFFu;
    if (mag >= 0x7F800000u) return (uint16_t)((sign >> 16) | 0x7F80u); /* +-Inf */
    float f;
    memcpy(&f, &mag, 4);
    double x = (double)f;
    uint32_t lo = mag >> 16;
    uint32_t hi = lo + 1;
    double dlo = x - bf16_mag_value(lo);
    double dhi = bf16_mag_value(hi) - x;
    uint32_t pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = (lo & 1u) ? hi : lo;
    return (uint16_t)((sign >> 16) | pick);
}

typedef struct {
    uint64_t start, end, bad;
} span;

static void *worker(void *arg) {
    span *s = (span *)arg;
    for (uint64_t v = s->start; v < s->end; ++v) {
        uint32_t u = (uint32_t)v;
        uint16_t got = oracle_bf16_rne(u);
        int isnan_in = (u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu);
        if (isnan_in) {
            int ok = (got & 0x7F80u) == 0x7F80u && (got & 0x0040u) && ((got ^ (u >> 16)) & 0x8000u) == 0;
            if (!ok) s->bad++;
        } else if (got != select_nearest(u)) {
            s->bad++;
        }
    }
    return NULL;
}

int main(void) {
    enum { T = 8 };
    pthread_t th[T];
    span sp[T];
    uint64_t total = 1ull << 32;
    for (int i = 0; i < T; ++i) {
        sp[i].start = total * i / T;
        sp[i].end = total * (i + 1) / T;
        sp[i].bad = 0;
        pthread_create(&th[i], NULL, worker, &sp[i]);
    }
    uint64_t bad = 0;
    for (int i = 0; i < T; ++i) {
        pthread_join(th[i], NULL);
        bad += sp[i].bad;
    }
    printf("mismatches %llu\n", (unsigned long long)bad);
    return bad ? 1 : 0;
}
