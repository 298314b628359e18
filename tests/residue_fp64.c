/* Host check of the residue method the MOD_LT predicate uses on the GPU
 * (x mod m < s, the non-negative residue of an int32 x, modulus m >= 1):
 *   q = floor(fma(x, inv, 2^-20)) with inv = 1/m rounded once,
 *   r = fma(-q, m, x),  keep iff (0 <= r < s) or r < s - m,
 * compared with the residue computed in 64-bit integers. C's fma and floor
 * are the IEEE operations the kernel's v_fma_f64 and v_floor_f64 perform.
 * Usage: residue_fp64 quick | full. Exit status 1 on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int method(int32_t x, int32_t m, int32_t s) {
    const double inv = 1.0 / (double)m, md = m, sd = s, smm = (double)s - (double)m;
    const double xd = (double)x;
    const double q = floor(fma(xd, inv, 0x1p-20));
    const double r = fma(-q, md, xd);
    return (r >= 0.0 && r < sd) || r < smm;
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
    /* moduli on both sides of 699,050, where q = floor(x/m) + 1 first becomes
       possible, plus the extremes */
    const int32_t ms[] = {1, 3, 100, 699049, 699051, 1000000007, 2147483647};
    for (unsigned i = 0; i < sizeof(ms) / sizeof(ms[0]); ++i) {
        const int32_t m = ms[i];
        if (full) {
            bad += sweep(m, m / 2 + 1, INT32_MIN, INT32_MAX);
        } else {
            /* the ends and the middle of the int32 range, 2^24 values each */
            bad += sweep(m, m / 2 + 1, INT32_MIN, (int64_t)INT32_MIN + (1 << 24));
            bad += sweep(m, m / 2 + 1, -(1 << 23), 1 << 23);
            bad += sweep(m, m / 2 + 1, (int64_t)INT32_MAX - (1 << 24), INT32_MAX);
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
