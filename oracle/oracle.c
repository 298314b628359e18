/*
 * Sequential CPU oracle for scan, stream compaction, stable partition and
 * the chained-partition radix sort.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link or
 * call this file; only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it. It shares no source, header, table or constant
 * generator with the HIP library: the predicate numbering below is written
 * out again here, and a test checks that both sides agree on it.
 *
 * Every function is the plain definition of what it computes, one loop at a
 * time, in input order, with no blocking or reordering. Sources:
 *   - "Day 33 compaction.cu" (stream compaction and partition): the header
 *     comment states the three steps (flag, exclusive scan of the flags,
 *     scatter to out[rank]), that the count is the top of the scan, and that
 *     i - rank[i] addresses the second half of a partition; compactCpu and
 *     partitionCpu give the sequential host forms followed here.
 *   - "CUDA Handbook ch. 13, Stream Compaction": compaction is an exclusive
 *     scan of 0/1 predicate flags whose values are output indices; the odd
 *     predicate is x & 1 (Listing 13-17).
 *   - "Day 32 scan_2.cu", scanExclusiveCpu: exclusive scan with a double
 *     accumulator (partial sums are kept in double precision).
 *   - "Day 31 scan.cu", scanInclusiveCpu: the inclusive form of the scan,
 *     out[i] = in[0] + ... + in[i] (whole array here, not restarted per tile).
 *   - "CIS 565 Project 2: Stream Compaction": the printed exclusive-scan and
 *     compaction transcripts fix the exclusive convention and the order.
 *
 * Readings where the pages leave a step open (each one is also listed with
 * its reason in the design notes of this repository):
 *   - int32 scan overflow wraps modulo 2^32; the sum is taken in uint32_t.
 *   - Partition puts the predicate-true elements first, both halves in
 *     input order (partitionCpu puts the flagged evens first).
 *   - MOD_LT uses the non-negative (Euclidean) residue for negative x.
 *   - ODD/EVEN test bit 0 of the two's-complement value, so -3 is odd.
 *   - The radix sort is 32 stable partitions, bit 0 first, keys whose bit is
 *     clear first, which leaves the keys ascending as unsigned integers.
 *   - n == 0 gives a count / total of 0.
 *   - fp32 arrays ("CUDA Handbook ch. 13": the compaction kernel is a
 *     template over the element type) take comparison predicates with IEEE
 *     semantics: NaN compares false (so NaN is nonzero but never above,
 *     below or inside a range) and -0.0 equals 0.0.
 *   - 64-bit elements (the same template) take the bit predicates on all 64
 *     bits of the two's-complement value: nonzero, odd, even, bit b set or
 *     clear for 0 <= b <= 63. The residue predicate is not defined for them.
 *   - A caller's own predicate ("Day 33 compaction.cu": the predicate is the
 *     only part that changes, everything after it reads an array of ones and
 *     zeros) arrives as one flag byte per element; any nonzero byte keeps
 *     the element.
 *   - Key-value compaction: the predicate is taken on the key and each value
 *     travels with its key, so both outputs hold the same positions.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>

/* Predicate kinds. Numbering mirrors the public C ABI; a test compares them. */
enum {
    ORC_PRED_NONZERO = 0,   /* x != 0                      */
    ORC_PRED_ODD = 1,       /* (x & 1) == 1                */
    ORC_PRED_EVEN = 2,      /* (x & 1) == 0                */
    ORC_PRED_BIT_SET = 3,   /* bit pa of x is 1, 0<=pa<=31 */
    ORC_PRED_BIT_CLEAR = 4, /* bit pa of x is 0            */
    ORC_PRED_MOD_LT = 5     /* mod(x, pa) < pb, pa >= 1    */
};

/* Predicates on fp32 elements (comparison semantics of IEEE 754). */
enum {
    ORC_PRED_F32_NONZERO = 6, /* x != 0                       */
    ORC_PRED_F32_GT = 7,      /* x > a                        */
    ORC_PRED_F32_LT = 8,      /* x < a                        */
    ORC_PRED_F32_IN = 9       /* a <= x && x < b              */
};

int orc_pred_id(int which) {
    switch (which) {
    case 0: return ORC_PRED_NONZERO;
    case 1: return ORC_PRED_ODD;
    case 2: return ORC_PRED_EVEN;
    case 3: return ORC_PRED_BIT_SET;
    case 4: return ORC_PRED_BIT_CLEAR;
    case 5: return ORC_PRED_MOD_LT;
    case 6: return ORC_PRED_F32_NONZERO;
    case 7: return ORC_PRED_F32_GT;
    case 8: return ORC_PRED_F32_LT;
    case 9: return ORC_PRED_F32_IN;
    default: return -1;
    }
}

/* 1 if the predicate arguments are usable, 0 otherwise. */
int orc_pred_args_ok(int pred, int32_t pa, int32_t pb) {
    (void)pb;
    switch (pred) {
    case ORC_PRED_NONZERO:
    case ORC_PRED_ODD:
    case ORC_PRED_EVEN:
        return 1;
    case ORC_PRED_BIT_SET:
    case ORC_PRED_BIT_CLEAR:
        return pa >= 0 && pa <= 31;
    case ORC_PRED_MOD_LT:
        return pa >= 1;
    default:
        return 0;
    }
}

/* Non-negative residue of x modulo m (m >= 1), by the definition
 * x = q*m + r with 0 <= r < m, computed in 64-bit so no case overflows. */
static int64_t euclid_mod(int32_t x, int32_t m) {
    int64_t r = (int64_t)x % (int64_t)m;
    if (r < 0) r += m;
    return r;
}

/* The predicate, element by element. Returns 0 or 1. */
int orc_pred(int32_t x, int pred, int32_t pa, int32_t pb) {
    uint32_t u = (uint32_t)x;
    switch (pred) {
    case ORC_PRED_NONZERO: return x != 0;
    case ORC_PRED_ODD: return (u & 1u) == 1u;
    case ORC_PRED_EVEN: return (u & 1u) == 0u;
    case ORC_PRED_BIT_SET: return ((u >> pa) & 1u) == 1u;
    case ORC_PRED_BIT_CLEAR: return ((u >> pa) & 1u) == 0u;
    case ORC_PRED_MOD_LT: return euclid_mod(x, pa) < (int64_t)pb;
    default: return 0;
    }
}

/* The fp32 predicate, element by element. Returns 0 or 1. */
int orc_pred_f32(float x, int pred, float a, float b) {
    switch (pred) {
    case ORC_PRED_F32_NONZERO: return x != 0.0f;
    case ORC_PRED_F32_GT: return x > a;
    case ORC_PRED_F32_LT: return x < a;
    case ORC_PRED_F32_IN: return a <= x && x < b;
    default: return 0;
    }
}

/* Order-preserving compaction of fp32 values (as orc_compact_i32). */
int64_t orc_compact_f32(const float *in, float *out, int64_t n, int pred, float a, float b) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (orc_pred_f32(in[i], pred, a, b)) {
            out[m] = in[i];
            ++m;
        }
    }
    return m;
}

/* Stable partition of fp32 values (as orc_partition_i32). */
int64_t orc_partition_f32(const float *in, float *out, int64_t n, int pred, float a, float b) {
    int64_t kept = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (orc_pred_f32(in[i], pred, a, b)) {
            out[kept] = in[i];
            ++kept;
        }
    }
    int64_t pos = kept;
    for (int64_t i = 0; i < n; ++i) {
        if (!orc_pred_f32(in[i], pred, a, b)) {
            out[pos] = in[i];
            ++pos;
        }
    }
    return kept;
}

/* Positions of the fp32 elements for which the predicate holds. */
int64_t orc_select_index_f32(const float *in, int32_t *idx, int64_t n, int pred, float a,
                             float b) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (orc_pred_f32(in[i], pred, a, b)) {
            idx[m] = (int32_t)i;
            ++m;
        }
    }
    return m;
}

/* flags[i] = P(in[i]). */
void orc_flags(const int32_t *in, int32_t *flags, int64_t n, int pred,
               int32_t pa, int32_t pb) {
    for (int64_t i = 0; i < n; ++i) flags[i] = orc_pred(in[i], pred, pa, pb);
}

/* Exclusive scan of int32 values with modulo-2^32 wrap:
 * out[0] = 0, out[i] = out[i-1] + in[i-1]; total = sum of all. */
void orc_exclusive_scan_i32(const int32_t *in, int32_t *out, int64_t n,
                            int32_t *total) {
    uint32_t running = 0;
    for (int64_t i = 0; i < n; ++i) {
        out[i] = (int32_t)running;
        running += (uint32_t)in[i];
    }
    if (total) *total = (int32_t)running;
}

/* Exclusive scan of fp32 values, accumulated in fp64 and kept in fp64:
 * out[i] = sum_{j<i} (double)in[j]. */
void orc_exclusive_scan_f32(const float *in, double *out, int64_t n,
                            double *total) {
    double running = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        out[i] = running;
        running += (double)in[i];
    }
    if (total) *total = running;
}

/* Inclusive scan of int32 values with modulo-2^32 wrap:
 * out[i] = in[0] + ... + in[i]. */
void orc_inclusive_scan_i32(const int32_t *in, int32_t *out, int64_t n) {
    uint32_t running = 0;
    for (int64_t i = 0; i < n; ++i) {
        running += (uint32_t)in[i];
        out[i] = (int32_t)running;
    }
}

/* Inclusive scan of fp32 values, accumulated in fp64 and kept in fp64:
 * out[i] = sum_{j<=i} (double)in[j]. */
void orc_inclusive_scan_f32(const float *in, double *out, int64_t n) {
    double running = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        running += (double)in[i];
        out[i] = running;
    }
}

/* Number of elements for which the predicate holds. */
int64_t orc_count(const int32_t *in, int64_t n, int pred, int32_t pa,
                  int32_t pb) {
    int64_t c = 0;
    for (int64_t i = 0; i < n; ++i) c += orc_pred(in[i], pred, pa, pb);
    return c;
}

/* Order-preserving compaction: the survivors in input order; returns their
 * number. When ranks is not NULL it also receives the exclusive scan of the
 * flags, i.e. the output slot each element would take. */
int64_t orc_compact_i32(const int32_t *in, int32_t *out, int64_t n, int pred,
                        int32_t pa, int32_t pb, int32_t *ranks) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (ranks) ranks[i] = (int32_t)m;
        if (orc_pred(in[i], pred, pa, pb)) {
            out[m] = in[i];
            ++m;
        }
    }
    return m;
}

/* Selection form of compaction ("CUDA Handbook ch. 13": a flag's exclusive-
 * scan value is the element's output index): the positions i of the
 * elements for which the predicate holds, in increasing order; returns their
 * number. */
int64_t orc_select_index_i32(const int32_t *in, int32_t *idx, int64_t n, int pred,
                             int32_t pa, int32_t pb) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (orc_pred(in[i], pred, pa, pb)) {
            idx[m] = (int32_t)i;
            ++m;
        }
    }
    return m;
}

/* Stable two-way partition: every element with P true in input order, then
 * every element with P false in input order. Two passes, one per half.
 * Returns the size of the first half. */
int64_t orc_partition_i32(const int32_t *in, int32_t *out, int64_t n, int pred,
                          int32_t pa, int32_t pb) {
    int64_t kept = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (orc_pred(in[i], pred, pa, pb)) {
            out[kept] = in[i];
            ++kept;
        }
    }
    int64_t pos = kept;
    for (int64_t i = 0; i < n; ++i) {
        if (!orc_pred(in[i], pred, pa, pb)) {
            out[pos] = in[i];
            ++pos;
        }
    }
    return kept;
}

/* Least-significant-bit-first radix sort of uint32 keys as `passes` chained
 * stable partitions, pass b keeping keys whose bit b is clear first. With
 * passes == 32 the result is ascending. in is left unchanged; out receives the
 * result; tmp is n words of workspace. */
void orc_radix_sort_u32(const uint32_t *in, uint32_t *out, uint32_t *tmp,
                        int64_t n, int passes) {
    if (n == 0) return;
    memcpy(out, in, (size_t)n * sizeof(uint32_t));
    for (int b = 0; b < passes; ++b) {
        orc_partition_i32((const int32_t *)out, (int32_t *)tmp, n,
                          ORC_PRED_BIT_CLEAR, b, 0);
        memcpy(out, tmp, (size_t)n * sizeof(uint32_t));
    }
}

/* ---- a caller's predicate as flag bytes ---- */

/* Order-preserving compaction of 32-bit words (int32 or fp32 bits, moved
 * unchanged) whose flag byte is nonzero; returns their number. */
int64_t orc_compact_flags_b32(const uint32_t *in, const uint8_t *flags, uint32_t *out,
                              int64_t n) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (flags[i] != 0) {
            out[m] = in[i];
            ++m;
        }
    }
    return m;
}

/* Positions i whose flag byte is nonzero, in increasing order. */
int64_t orc_select_flags(const uint8_t *flags, int32_t *idx, int64_t n) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (flags[i] != 0) {
            idx[m] = (int32_t)i;
            ++m;
        }
    }
    return m;
}

/* ---- key-value pairs ---- */

/* Pairs (keys[i], vals[i]) whose key satisfies the int32 predicate, in input
 * order; values are 32-bit words moved unchanged. Returns their number. */
int64_t orc_compact_kv_i32(const int32_t *keys, const uint32_t *vals, int32_t *okeys,
                           uint32_t *ovals, int64_t n, int pred, int32_t pa, int32_t pb) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (orc_pred(keys[i], pred, pa, pb)) {
            okeys[m] = keys[i];
            ovals[m] = vals[i];
            ++m;
        }
    }
    return m;
}

/* As orc_compact_kv_i32 with fp32 keys and the fp32 predicates. */
int64_t orc_compact_kv_f32(const float *keys, const uint32_t *vals, float *okeys,
                           uint32_t *ovals, int64_t n, int pred, float a, float b) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (orc_pred_f32(keys[i], pred, a, b)) {
            okeys[m] = keys[i];
            ovals[m] = vals[i];
            ++m;
        }
    }
    return m;
}

/* ---- 64-bit elements ---- */

/* 1 if the predicate and its argument are usable on 64-bit elements. */
int orc_pred_args_ok_i64(int pred, int32_t pa) {
    switch (pred) {
    case ORC_PRED_NONZERO:
    case ORC_PRED_ODD:
    case ORC_PRED_EVEN:
        return 1;
    case ORC_PRED_BIT_SET:
    case ORC_PRED_BIT_CLEAR:
        return pa >= 0 && pa <= 63;
    default:
        return 0;
    }
}

/* The predicate on a 64-bit element, taken on its two's-complement bits. */
int orc_pred_i64(int64_t x, int pred, int32_t pa) {
    uint64_t u = (uint64_t)x;
    switch (pred) {
    case ORC_PRED_NONZERO: return x != 0;
    case ORC_PRED_ODD: return (u & 1u) == 1u;
    case ORC_PRED_EVEN: return (u & 1u) == 0u;
    case ORC_PRED_BIT_SET: return ((u >> pa) & 1u) == 1u;
    case ORC_PRED_BIT_CLEAR: return ((u >> pa) & 1u) == 0u;
    default: return 0;
    }
}

/* Order-preserving compaction of 64-bit elements; returns the survivors'
 * number. */
int64_t orc_compact_i64(const int64_t *in, int64_t *out, int64_t n, int pred, int32_t pa) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (orc_pred_i64(in[i], pred, pa)) {
            out[m] = in[i];
            ++m;
        }
    }
    return m;
}

/* Positions of the 64-bit elements for which the predicate holds. */
int64_t orc_select_index_i64(const int64_t *in, int32_t *idx, int64_t n, int pred,
                             int32_t pa) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (orc_pred_i64(in[i], pred, pa)) {
            idx[m] = (int32_t)i;
            ++m;
        }
    }
    return m;
}
