/* Drives every function of oracle/oracle.c over edge sizes and every
 * predicate with valid arguments, for builds with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers_cpu.py). Each buffer is
 * allocated at exactly the size the function may touch, so a read or write
 * one element out of bounds, a signed overflow, an out-of-range shift or a
 * misaligned access stops the run. Cross-checks between the functions (the
 * counts agree, partition's kept count, sorted output) catch gross
 * breakage; the value checks proper are the oracle pins.
 * Exit status 0 and "ok <calls>" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_pred_id(int which);
int orc_pred_args_ok(int pred, int32_t pa, int32_t pb);
int orc_pred(int32_t x, int pred, int32_t pa, int32_t pb);
int orc_pred_f32(float x, int pred, float a, float b);
int64_t orc_compact_f32(const float *in, float *out, int64_t n, int pred, float a, float b);
int64_t orc_partition_f32(const float *in, float *out, int64_t n, int pred, float a, float b);
int64_t orc_select_index_f32(const float *in, int32_t *idx, int64_t n, int pred, float a, float b);
void orc_flags(const int32_t *in, int32_t *flags, int64_t n, int pred, int32_t pa, int32_t pb);
void orc_exclusive_scan_i32(const int32_t *in, int32_t *out, int64_t n, int32_t *total);
void orc_exclusive_scan_f32(const float *in, double *out, int64_t n, double *total);
void orc_inclusive_scan_i32(const int32_t *in, int32_t *out, int64_t n);
void orc_inclusive_scan_f32(const float *in, double *out, int64_t n);
int64_t orc_count(const int32_t *in, int64_t n, int pred, int32_t pa, int32_t pb);
int64_t orc_compact_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa,
                        int32_t pb, int32_t *ranks);
int64_t orc_select_index_i32(const int32_t *in, int32_t *idx, int64_t n, int pred, int32_t pa,
                             int32_t pb);
int64_t orc_partition_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa,
                          int32_t pb);
void orc_radix_sort_u32(const uint32_t *in, uint32_t *out, uint32_t *tmp, int64_t n, int passes);
int64_t orc_compact_flags_b32(const uint32_t *in, const uint8_t *flags, uint32_t *out, int64_t n);
int64_t orc_select_flags(const uint8_t *flags, int32_t *idx, int64_t n);
int64_t orc_compact_kv_i32(const int32_t *keys, const uint32_t *vals, int32_t *okeys,
                           uint32_t *ovals, int64_t n, int pred, int32_t pa, int32_t pb);
int64_t orc_compact_kv_f32(const float *keys, const uint32_t *vals, float *okeys, uint32_t *ovals,
                           int64_t n, int pred, float a, float b);
int orc_pred_args_ok_i64(int pred, int32_t pa);
int orc_pred_i64(int64_t x, int pred, int32_t pa);
int64_t orc_compact_i64(const int64_t *in, int64_t *out, int64_t n, int pred, int32_t pa);
int64_t orc_select_index_i64(const int64_t *in, int32_t *idx, int64_t n, int pred, int32_t pa);

static uint64_t state = 0x2545F4914F6CDD1Dull;
static uint32_t rnd(void) {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 11);
}

static long calls = 0;

static void fail(const char *what, int64_t n) {
    printf("FAIL %s n=%lld\n", what, (long long)n);
    exit(1);
}

/* exactly n elements of size sz (one byte when n == 0, never dereferenced) */
static void *alloc(int64_t n, size_t sz) { return malloc(n ? (size_t)n * sz : 1); }

static void int_preds(const int32_t *x, int64_t n) {
    static const int32_t args[][3] = {
        {0, 0, 0}, {1, 0, 0}, {2, 0, 0}, {3, 0, 0}, {3, 31, 0}, {4, 0, 0}, {4, 31, 0},
        {5, 1, 0}, {5, 1, 1}, {5, 100, 1}, {5, 100, 50}, {5, 100, 99}, {5, 7, -1}, {5, 7, 8},
        {5, 2147483647, 5}, {5, 2147483647, 2147483647},
    };
    for (size_t a = 0; a < sizeof args / sizeof args[0]; ++a) {
        const int p = args[a][0];
        const int32_t pa = args[a][1], pb = args[a][2];
        if (!orc_pred_args_ok(p, pa, pb)) fail("args rejected", n);
        int32_t *out = alloc(n, 4), *ranks = alloc(n, 4), *idx = alloc(n, 4), *fl = alloc(n, 4);
        int32_t *part = alloc(n, 4), *ko = alloc(n, 4);
        uint32_t *vals = alloc(n, 4), *vo = alloc(n, 4);
        for (int64_t i = 0; i < n; ++i) vals[i] = rnd();
        const int64_t m = orc_compact_i32(x, out, n, p, pa, pb, ranks);
        const int64_t c = orc_count(x, n, p, pa, pb);
        const int64_t s = orc_select_index_i32(x, idx, n, p, pa, pb);
        const int64_t k = orc_partition_i32(x, part, n, p, pa, pb);
        const int64_t kv = orc_compact_kv_i32(x, vals, ko, vo, n, p, pa, pb);
        orc_flags(x, fl, n, p, pa, pb);
        calls += 6;
        if (m != c || s != m || k != m || kv != m) fail("counts differ", n);
        int64_t f = 0;
        for (int64_t i = 0; i < n; ++i) f += fl[i];
        if (f != m) fail("flags sum", n);
        free(out), free(ranks), free(idx), free(fl), free(part), free(ko), free(vals), free(vo);
    }
}

static void f32_preds(const float *x, int64_t n) {
    static const float args[][3] = {
        {6, 0.0f, 0.0f}, {7, 0.5f, 0.0f}, {8, 0.5f, 0.0f}, {9, 0.25f, 0.75f}, {9, 0.0f, 0.0f},
        {7, NAN, 0.0f}, {9, -INFINITY, INFINITY},
    };
    for (size_t a = 0; a < sizeof args / sizeof args[0]; ++a) {
        const int p = (int)args[a][0];
        float *out = alloc(n, 4), *part = alloc(n, 4), *ko = alloc(n, 4);
        int32_t *idx = alloc(n, 4);
        uint32_t *vals = alloc(n, 4), *vo = alloc(n, 4);
        for (int64_t i = 0; i < n; ++i) vals[i] = rnd();
        const int64_t m = orc_compact_f32(x, out, n, p, args[a][1], args[a][2]);
        const int64_t k = orc_partition_f32(x, part, n, p, args[a][1], args[a][2]);
        const int64_t s = orc_select_index_f32(x, idx, n, p, args[a][1], args[a][2]);
        const int64_t kv = orc_compact_kv_f32(x, vals, ko, vo, n, p, args[a][1], args[a][2]);
        calls += 4;
        if (k != m || s != m || kv != m) fail("f32 counts differ", n);
        free(out), free(part), free(ko), free(idx), free(vals), free(vo);
    }
}

static void i64_preds(const int64_t *x, int64_t n) {
    static const int32_t args[][2] = {{0, 0}, {1, 0}, {2, 0}, {3, 0}, {3, 63}, {4, 40}, {4, 63}};
    for (size_t a = 0; a < sizeof args / sizeof args[0]; ++a) {
        if (!orc_pred_args_ok_i64(args[a][0], args[a][1])) fail("i64 args rejected", n);
        int64_t *out = alloc(n, 8);
        int32_t *idx = alloc(n, 4);
        const int64_t m = orc_compact_i64(x, out, n, args[a][0], args[a][1]);
        const int64_t s = orc_select_index_i64(x, idx, n, args[a][0], args[a][1]);
        calls += 2;
        if (s != m) fail("i64 counts differ", n);
        free(out), free(idx);
    }
}

static void scans_and_sort(const int32_t *x, const float *f, int64_t n) {
    int32_t *o = alloc(n, 4), tot = 0;
    double *d = alloc(n, 8), dt = 0.0;
    orc_exclusive_scan_i32(x, o, n, &tot);
    orc_inclusive_scan_i32(x, o, n);
    orc_exclusive_scan_f32(f, d, n, &dt);
    orc_inclusive_scan_f32(f, d, n);
    calls += 4;
    uint32_t *so = alloc(n, 4), *st = alloc(n, 4);
    for (int passes = 1; passes <= 32; passes *= 2) {
        orc_radix_sort_u32((const uint32_t *)x, so, st, n, passes);
        ++calls;
    }
    for (int64_t i = 1; i < n; ++i)
        if (so[i - 1] > so[i]) fail("sort order", n);
    uint8_t *fl = alloc(n, 1);
    for (int64_t i = 0; i < n; ++i) fl[i] = (uint8_t)(rnd() % 3 == 0 ? 0 : rnd());
    int32_t *idx = alloc(n, 4);
    const int64_t m = orc_compact_flags_b32((const uint32_t *)x, fl, so, n);
    const int64_t s = orc_select_flags(fl, idx, n);
    calls += 2;
    if (m != s) fail("flag counts differ", n);
    free(o), free(d), free(so), free(st), free(fl), free(idx);
}

int main(void) {
    static const int64_t sizes[] = {0, 1, 2, 3, 31, 32, 33, 63, 64, 65, 1000, 4097, 30721};
    for (int w = 0; w < 6; ++w) orc_pred_id(w);
    for (size_t t = 0; t < sizeof sizes / sizeof sizes[0]; ++t) {
        const int64_t n = sizes[t];
        int32_t *x = alloc(n, 4);
        float *f = alloc(n, 4);
        int64_t *y = alloc(n, 8);
        for (int64_t i = 0; i < n; ++i) {
            const uint32_t r = rnd();
            x[i] = (i % 7 == 0) ? (i % 14 == 0 ? INT32_MIN : INT32_MAX) : (int32_t)r;
            f[i] = (float)(rnd() & 0xFFFFFF) / 16777216.0f;
            y[i] = (int64_t)(((uint64_t)rnd() << 32) | rnd());
        }
        if (n > 2) f[n / 2] = NAN, f[1] = -0.0f;
        int_preds(x, n);
        f32_preds(f, n);
        i64_preds(y, n);
        scans_and_sort(x, f, n);
        free(x), free(f), free(y);
    }
    printf("ok %ld\n", calls);
    return 0;
}
