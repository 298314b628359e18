/* Host check of the residue method the MOD_LT predicate uses on the GPU
 * (x mod m < s, the non-negative residue of an int32 x, modulus m >= 1):
 *   inv = 1/m, half = inv/2 and thr = s/m, each rounded once,
 *   t = fma(x, inv, half),  f = t - floor(t)  (v_fract_f64),
 *   keep iff f < thr, which the flag masks read as the sign bit of f - thr,
 * compared with the residue computed in 64-bit integers. t is (x + 1/2)/m to
 * within 2^-21/m, so f is (r + 1/2)/m to within that: below s/m iff r < s,
 * with 1/(2m) to spare. C's fma, floor and subtraction are the IEEE
 * operations the kernels perform. Both forms of the final test are checked.
 * Usage: residue_fp64 quick | full. Exit status 1 on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int method(int32_t x, int32_t m, int32_t s) {
    const double inv = 1.0 / (double)m, half = 0.5 * inv, thr = (double)s / (double)m;
    const double t = fma((double)x, inv, half);
    const double f = t - floor(t);
    const int by_compare = f < thr;
    const int by_sign = signbit(f - thr) != 0;
    return by_compare == by_sign ? by_compare : -1;
}

static int residue(int32_t x, int32_t m, int32_t s) {
    int64_t r = (int64_t)x % m;
    if (r < 0) r += m;
    return r < (int64_t)s;
}

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}

static long long sweep(int32_t m, int32_t s, int64_t lo, int64_t hi) {
    long long bad = 0;
    for (int64_t x = lo; x <= hi; ++x)
        if (method((int32_t)x, m, s) != residue((int32_t)x, m, s)) ++bad;
    return bad;
}

int main(int argc, char **argv) {
    const int full = argc > 1 && strcmp(argv[1], "full") == 0;
    long long bad = 0;
    /* small, prime, power-of-two-adjacent and the largest moduli */
    const int32_t ms[] = {1, 2, 3, 100, 65537, 699049, 1048577, 1000000007, 2147483646, 2147483647};
    for (unsigned i = 0; i < sizeof(ms) / sizeof(ms[0]); ++i) {
        const int32_t m = ms[i];
        /* bounds in the middle, at the ends, and outside [1, m - 1] */
        const int32_t ss[] = {m / 2 + 1, 1, m - 1, 0, m};
        for (unsigned k = 0; k < (full ? 3u : 5u); ++k) {
            const int32_t s = ss[k];
            if (full) {
                bad += sweep(m, s, INT32_MIN, INT32_MAX);
            } else {
                /* the ends and the middle of the int32 range, 2^22 values each */
                bad += sweep(m, s, INT32_MIN, (int64_t)INT32_MIN + (1 << 22));
                bad += sweep(m, s, -(1 << 21), 1 << 21);
                bad += sweep(m, s, (int64_t)INT32_MAX - (1 << 22), INT32_MAX);
            }
        }
    }
    const int64_t triples = full ? 400000000LL : 50000000LL;
    for (int64_t t = 0; t < triples; ++t) {
        int32_t m = (int32_t)(next() % 2147483647u) + 1;
        if (t & 1) m = (int32_t)(next() % 5000) + 1;
        const int32_t s = (int32_t)((int64_t)(next() % ((uint64_t)m + 3)) - 1);
        const int32_t x = (int32_t)next();
        if (method(x, m, s) != residue(x, m, s)) ++bad;
    }
    printf("%lld mismatches\n", bad);
    return bad != 0;
}
