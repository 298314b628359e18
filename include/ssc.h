/*
 * ssc.h -- single-pass scan, stream compaction and stable partition on
 * AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The method: evaluate a predicate on every element (a 0/1 flag), take the
 * exclusive scan of the flags, and scatter every survivor x[i] to
 * out[rank[i]]. Input order is kept, the survivor count is the top of the
 * scan, and a stable partition addresses its second half with i - rank[i]
 * from the same scan ("Day 33 compaction.cu", header comment and
 * scatterCompact / scatterPartition). The scan runs in one pass over the
 * input with per-tile descriptors and a decoupled look-back over earlier
 * tiles, tile numbers being taken from an atomic counter ("CUDA Handbook
 * ch. 13, Stream Compaction", Listings 13-17 and 13-18).
 *
 * Conventions shared by every call:
 *   - All array, count and scratch pointers are DEVICE pointers (hipMalloc
 *     or equivalent) owned by the caller. The library never allocates and
 *     never frees.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream); it
 *     must belong to the current device. Calls only enqueue work on it and
 *     never synchronise; counts and totals stay in device memory.
 *   - Scratch: a caller-provided device buffer of at least
 *     ssc_scratch_bytes(n) bytes, 8-byte aligned, ZERO-FILLED BEFORE ITS
 *     FIRST USE (ssc_scratch_init, or any memset to 0). The library keeps it
 *     ready for the next call by itself: no clearing between calls, so a
 *     call is a single kernel launch (two for a partition). Pass the same
 *     scratch_bytes every time a buffer is used. One scratch buffer must not
 *     serve two calls that may run at the same time (the calls race).
 *     Diagnostic: a look-back wait that gives up after its bounded spin
 *     (only possible on misuse, such as a scratch that was never zeroed or
 *     one shared by two calls in flight) sets a time-out flag in the
 *     scratch; ssc_scratch_timed_out reads it. Once set, the results of the
 *     calls made with that scratch are invalid and the flag stays set: the
 *     scratch must be re-initialised (ssc_scratch_init) before it is used
 *     again.
 *   - Element pointers must be 4-byte aligned. 16-byte aligned arrays take
 *     the 128-bit load/store path; other arrays take a 32-bit path with the
 *     same results.
 *   - Sizes: n is an element count, 0 <= n <= INT32_MAX (ranks and counts are
 *     int32). n == 0 writes 0 to `count` / `total` and returns SSC_OK; array
 *     pointers may then be NULL (count/total may not be, where required).
 *   - Errors: every call returns an ssc_status; arguments are checked before
 *     anything is enqueued, and on an argument error nothing is enqueued. A
 *     failed launch gives SSC_ERR_HIP (ssc_last_hip_error() has the code).
 *     The library never exits or aborts.
 *   - Only the elements out[0 .. count) of a compaction are written; the rest
 *     of `out` is left as it was.
 */
#ifndef SSC_H
#define SSC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssc_status {
    SSC_OK = 0,
    SSC_ERR_ARG = 1,     /* null pointer, n < 0, bad predicate or predicate argument, misalignment */
    SSC_ERR_SIZE = 2,    /* n > INT32_MAX (the small-tile test build: n > 2^17 x 3840) */
    SSC_ERR_ALIAS = 3,   /* buffers overlap where they must not */
    SSC_ERR_SCRATCH = 4, /* scratch too small or not 8-byte aligned */
    SSC_ERR_HIP = 5,     /* a HIP call or kernel launch failed */
    SSC_ERR_DEVICE = 6   /* current device is not gfx950 with 64-wide wavefronts */
} ssc_status;

/* Predicate kinds. pa/pb are ignored where not listed.
 *   NONZERO    x != 0              zero removal ("Day 33 compaction.cu", markNonZero)
 *   ODD        (x & 1) == 1        ("CUDA Handbook ch. 13", Listing 13-17, isOdd)
 *   EVEN       (x & 1) == 0        ("Day 33 compaction.cu", markEven)
 *   BIT_SET    bit pa of x is 1    0 <= pa <= 31 (one split of an LSD radix sort,
 *   BIT_CLEAR  bit pa of x is 0      "CIS 565 Project 2: Stream Compaction")
 *   MOD_LT     r < pb where r is the non-negative residue of x modulo pa, pa >= 1
 * Bit tests use the two's-complement bits, so -3 is odd.
 * For fp32 arrays (the *_f32 calls; the compaction kernel of "CUDA Handbook
 * ch. 13" is a template over the element type), with thresholds a, b and
 * IEEE comparisons (every comparison with NaN is false, -0.0 == 0.0):
 *   F32_NONZERO  x != 0          (NaN is nonzero, -0.0 is zero)
 *   F32_GT       x > a
 *   F32_LT       x < a
 *   F32_IN       a <= x && x < b
 * The int32 calls take predicates 0..5 only and the fp32 calls 6..9. */
typedef enum ssc_pred {
    SSC_PRED_NONZERO = 0,
    SSC_PRED_ODD = 1,
    SSC_PRED_EVEN = 2,
    SSC_PRED_BIT_SET = 3,
    SSC_PRED_BIT_CLEAR = 4,
    SSC_PRED_MOD_LT = 5,
    SSC_PRED_F32_NONZERO = 6,
    SSC_PRED_F32_GT = 7,
    SSC_PRED_F32_LT = 8,
    SSC_PRED_F32_IN = 9
} ssc_pred;

/* Elements per tile: the share of the single pass behind one tile number
 * claimed from the atomic counter and one look-back descriptor (a workgroup
 * of the compaction kernel processes several tiles in turn). 30720; 3840 in
 * the library's small-tile test build (libssc_stress.so), which otherwise
 * has the same calls and results. */
int64_t ssc_tile_elems(void);

/* Scratch bytes needed by the scan, compaction, partition and counting calls
 * for n elements: a 512-byte header (tile counter and epoch, counting-pass
 * accumulators) plus 16 bytes of look-back descriptors per ssc_tile_elems()
 * elements (one 8-byte descriptor per tile; the fp32 scans use two, the
 * key-value and 64-bit compactions have tiles of half the size). */
size_t ssc_scratch_bytes(int64_t n);

/* Scratch bytes needed by ssc_radix_sort_u32 for n keys. */
size_t ssc_radix_sort_scratch_bytes(int64_t n);

/* Scratch bytes needed by ssc_radix_sort4_u32 for n keys: a scan scratch for
 * a 16 x ceil(n / 8192) table of per-tile digit counts, then the table. */
size_t ssc_radix_sort4_scratch_bytes(int64_t n);

/* Zero-fills a scratch buffer on `stream` (needed once, before first use,
 * and again after a time-out, see below). */
int ssc_scratch_init(void *scratch, size_t scratch_bytes, void *stream);

/* Stream-ordered check of a scratch buffer: writes 1 to *flag (a device
 * int32) if a look-back wait of a call made with this scratch gave up after
 * its bounded spin since the scratch was last initialised, else 0. A set
 * flag means those calls' results are invalid and the scratch needs
 * ssc_scratch_init before further use; it never comes from a correct call.
 * One tiny launch; flag must not lie inside the scratch. */
int ssc_scratch_timed_out(const void *scratch, size_t scratch_bytes, int32_t *flag, void *stream);

/* Exclusive scan of int32 values: out[0] = 0, out[i] = in[0] + ... + in[i-1],
 * with two's-complement wrap (sums taken modulo 2^32). `total` (nullable)
 * receives the sum of all n values. out == in is allowed (in place); any
 * other overlap of in/out/total is SSC_ERR_ALIAS.
 * Source: "Day 32 scan_2.cu" (scanExclusiveCpu) and the exclusive
 * convention of the "CIS 565 Project 2" transcript (0 13 50 ... for 13 37 15 ...). */
int ssc_exclusive_scan_i32(const int32_t *in, int32_t *out, int64_t n, int32_t *total,
                           void *scratch, size_t scratch_bytes, void *stream);

/* Exclusive scan of fp32 values. The prefix inside a tile (at most 30720
 * values) is summed in fp32 in a tiled order; the carries between tiles are
 * fp64, and each output is rounded to fp32 once from the fp64 sum of carry
 * and in-tile prefix, so the error does not grow with the number of tiles
 * (the double accumulation of "Day 32 scan_2.cu", scanExclusiveCpu, for the
 * part that spans tiles). Tested within 1e-6 relative of the exactly
 * accumulated prefix for non-negative values up to n = 2^27. Aliasing rules
 * as above. */
int ssc_exclusive_scan_f32(const float *in, float *out, int64_t n, float *total,
                           void *scratch, size_t scratch_bytes, void *stream);

/* Inclusive scan of int32 values: out[i] = in[0] + ... + in[i], with
 * two's-complement wrap; `total` (nullable) receives out[n-1] (0 for n = 0).
 * Aliasing rules as for the exclusive scan.
 * Source: "Day 31 scan.cu" (scanInclusiveCpu and the inclusive block scans;
 * here over the whole array, not restarted per tile). */
int ssc_inclusive_scan_i32(const int32_t *in, int32_t *out, int64_t n, int32_t *total,
                           void *scratch, size_t scratch_bytes, void *stream);

/* Inclusive scan of fp32 values, accumulated as the exclusive fp32 scan is;
 * same accuracy statement and aliasing rules. Source: "Day 31 scan.cu". */
int ssc_inclusive_scan_f32(const float *in, float *out, int64_t n, float *total,
                           void *scratch, size_t scratch_bytes, void *stream);

/* Order-preserving compaction: out[0 .. count) = the elements x with P(x)
 * true, in input order; *count = their number (the top of the scan of the
 * flags). `ranks` (nullable) receives the exclusive scan of the flags for
 * every i: the output slot of in[i] when it survives. No overlap between
 * in, out, count and ranks is allowed.
 * Source: "Day 33 compaction.cu" (compactCpu, scatterCompact) and
 * "CUDA Handbook ch. 13" (Listing 13-17: survivors scattered to
 * base + index within the tile; the last tile writes the total). */
int ssc_compact_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa,
                    int32_t pb, int32_t *count, int32_t *ranks, void *scratch,
                    size_t scratch_bytes, void *stream);

/* ssc_compact_i32 without a scratch argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results, errors and
 * kernels as ssc_compact_i32; nothing is allocated or freed: the scratch is a
 * library-owned device array of 1,119,232 bytes on each GPU (enough for every
 * n up to INT32_MAX; a larger scratch need would give SSC_ERR_SIZE), held
 * until the process ends. Its address is looked up and the array zero-filled
 * by one clearing kernel on `stream` at the first call on a device; later
 * calls reuse it as left by the previous call, which keeps it ready. All
 * calls on one GPU share that one array, so calls that may run at the same
 * time on one GPU (other streams, other host threads) race and give wrong
 * results: serialise them. */
int ssc_compact_i32_noalloc(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa,
                            int32_t pb, int32_t *count, int32_t *ranks, void *stream);

/* ssc_compact_i32 for fp32 arrays with an fp32 predicate (6..9) and its
 * thresholds a, b; values move bit for bit (-0.0 and NaN payloads kept). */
int ssc_compact_f32(const float *in, float *out, int64_t n, int pred, float a, float b,
                    int32_t *count, int32_t *ranks, void *scratch, size_t scratch_bytes,
                    void *stream);

/* Selection (the index form of compaction): idx[0 .. count) = the
 * positions i, increasing, of the elements with P(in[i]) true; *count =
 * their number. idx[count .. n) is not written. Same single pass as
 * ssc_compact_i32, with each survivor's index scattered instead of its
 * value. No overlap between in, idx and count is allowed.
 * Source: "CUDA Handbook ch. 13, Stream Compaction" (the exclusive scan of
 * the flags gives each kept element its output position). */
int ssc_select_index_i32(const int32_t *in, int32_t *idx, int64_t n, int pred, int32_t pa,
                         int32_t pb, int32_t *count, void *scratch, size_t scratch_bytes,
                         void *stream);

/* ssc_select_index_i32 for fp32 arrays with an fp32 predicate (6..9). */
int ssc_select_index_f32(const float *in, int32_t *idx, int64_t n, int pred, float a, float b,
                         int32_t *count, void *scratch, size_t scratch_bytes, void *stream);

/* Stable partition: out[0 .. K) = the elements with P true, out[K .. n) =
 * the elements with P false, both in input order; *count = K. Kept x[i]
 * goes to out[rank[i]], rejected x[i] to out[K + i - rank[i]], where rank
 * is the exclusive scan of the flags. K is counted first by a reduction
 * pass over the input (written to *count), then one single pass scans and
 * scatters: two launches. No overlap between in, out and count is allowed.
 * Source: "Day 33 compaction.cu" (partitionCpu, scatterPartition). */
int ssc_partition_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa,
                      int32_t pb, int32_t *count, void *scratch, size_t scratch_bytes,
                      void *stream);

/* ssc_partition_i32 for fp32 arrays with an fp32 predicate (6..9). */
int ssc_partition_f32(const float *in, float *out, int64_t n, int pred, float a, float b,
                      int32_t *count, void *scratch, size_t scratch_bytes, void *stream);

/* Compaction by a caller's own predicate, given as one flag byte per
 * element: out[0 .. count) = the 32-bit elements in[i] (int32, fp32 or any
 * 4-byte type, moved bit for bit) whose flags[i] is nonzero, in input
 * order; *count = their number; out[count .. n) is not written. Same single
 * pass as ssc_compact_i32, the flags read in place of a predicate.
 * flags must be 4-byte aligned: the library reads it in 32-bit words,
 * including the whole word that holds flags[n - 1] (never past that word).
 * No overlap between in, flags, out and count is allowed.
 * Source: "Day 33 compaction.cu" (the predicate is the only part that
 * changes; everything after it reads an array of ones and zeros). */
int ssc_compact_flags_b32(const void *in, const uint8_t *flags, void *out, int64_t n,
                          int32_t *count, void *scratch, size_t scratch_bytes, void *stream);

/* Positions of the nonzero flag bytes: idx[0 .. count) = the i, increasing,
 * with flags[i] != 0; *count = their number (the flag-byte form of
 * ssc_select_index_i32; same alignment rule for flags). A 16-byte aligned
 * flag array is read in 128-bit words by a kernel with 61,440-flag tiles
 * (faster: each tile carries twice the bytes per look-back); it too
 * reads nothing past the 32-bit word that holds flags[n - 1]. No overlap
 * between flags, idx and count is allowed. Source: as ssc_compact_flags_b32. */
int ssc_select_flags(const uint8_t *flags, int32_t *idx, int64_t n, int32_t *count,
                     void *scratch, size_t scratch_bytes, void *stream);

/* Key-value compaction: the pairs (keys[i], vals[i]) whose key satisfies the
 * predicate (pred 0..5 with pa, pb as in ssc_compact_i32), in input order:
 * keys_out[0 .. count) and vals_out[0 .. count) hold the same positions;
 * *count = their number. Values are 4-byte words moved bit for bit. One
 * single pass over both arrays (1024 pairs per wavefront and tile). No
 * overlap between any two of keys, vals, keys_out, vals_out and count.
 * Source: the element-type template of "CUDA Handbook ch. 13, Stream
 * Compaction", with a value carried beside each kept key. */
int ssc_compact_kv_i32(const int32_t *keys, const void *vals, int32_t *keys_out, void *vals_out,
                       int64_t n, int pred, int32_t pa, int32_t pb, int32_t *count,
                       void *scratch, size_t scratch_bytes, void *stream);

/* ssc_compact_kv_i32 with fp32 keys and an fp32 predicate (6..9). */
int ssc_compact_kv_f32(const float *keys, const void *vals, float *keys_out, void *vals_out,
                       int64_t n, int pred, float a, float b, int32_t *count, void *scratch,
                       size_t scratch_bytes, void *stream);

/* Compaction of 64-bit elements (int64 or uint64 bits): out[0 .. count) =
 * the elements with P true in input order; *count = their number. P is
 * NONZERO, ODD, EVEN, BIT_SET or BIT_CLEAR on the 64 bits of the value, the
 * bit 0..63 given in `bit`; MOD_LT and the fp32 predicates give
 * SSC_ERR_ARG. in and out must be 8-byte aligned. One single pass (1024
 * elements per wavefront and tile). No overlap between in, out and count.
 * Source: "CUDA Handbook ch. 13, Stream Compaction" (Listing 13-17 is a
 * template over the element type; isOdd is x & 1). */
int ssc_compact_i64(const int64_t *in, int64_t *out, int64_t n, int pred, int32_t bit,
                    int32_t *count, void *scratch, size_t scratch_bytes, void *stream);

/* Selection over 64-bit elements: idx[0 .. count) = the positions i with
 * P(in[i]) true (predicates as ssc_compact_i64). No overlap between in, idx
 * and count. */
int ssc_select_index_i64(const int64_t *in, int32_t *idx, int64_t n, int pred, int32_t bit,
                         int32_t *count, void *scratch, size_t scratch_bytes, void *stream);

/* *count = number of elements with P true (a reduction of the flags; one
 * launch). Needs a scratch buffer of at least ssc_scratch_bytes(0) bytes. */
int ssc_count_if_i32(const int32_t *in, int64_t n, int pred, int32_t pa, int32_t pb,
                     int32_t *count, void *scratch, size_t scratch_bytes, void *stream);

/* Unordered compaction by atomic counter, kept only for comparison (it
 * needs no scratch: its counter is *count itself):
 * out[0 .. count) holds the same multiset as ssc_compact_i32's output, in
 * an order the hardware scheduler decides. variant 0: one atomicAdd per
 * 512-thread workgroup and 8192-element tile (its survivors keep tile
 * order inside the reserved range); variant 1: one atomicAdd per
 * survivor (the form of "Day 33 compaction.cu", compactAtomic). *count is
 * cleared and used as the counter. No overlap between in, out and count. */
int ssc_compact_atomic_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa,
                           int32_t pb, int32_t *count, int variant, void *stream);

/* LSD radix sort of uint32 keys as 32 chained stable 1-bit partitions,
 * pass b keeping keys whose bit b is clear first (bit 0 first), leaving
 * out[] ascending. One counting pass over the input gives the size of the
 * first half for every bit at once (a permutation does not change how many
 * keys have bit b clear). tmp is n words of caller workspace; in is not
 * modified. out == in is allowed; tmp must not overlap in or out.
 * Source: "CIS 565 Project 2: Stream Compaction" (radix sort built on the
 * compaction primitives, checked against std::sort). */
int ssc_radix_sort_u32(const uint32_t *in, uint32_t *out, uint32_t *tmp, int64_t n,
                       void *scratch, size_t scratch_bytes, void *stream);

/* LSD radix sort of uint32 keys with 4-bit digits: `passes` (1..8) stable
 * 16-way splits, pass p by digit (x >> 4p) & 15, so out[] ends stably sorted
 * by the low 4*passes bits of the keys (passes = 8: ascending). One 4-bit
 * split gives the same order as the four 1-bit splits of those bits in
 * ssc_radix_sort_u32, each a stable partition by a bit-test predicate. Each
 * pass: per-tile digit counts (tiles of 8192 keys), one exclusive scan of
 * the digit-major count table (the single-pass scan), then a stable scatter
 * in 16 contiguous runs per tile. tmp is n words of caller workspace; in is
 * not modified. out == in is allowed when passes is even; tmp must not
 * overlap in or out. passes outside 1..8 is SSC_ERR_ARG.
 * Source: "CIS 565 Project 2: Stream Compaction" (radix sort built on
 * split, LSD bit order); the digit width is this library's. */
int ssc_radix_sort4_u32(const uint32_t *in, uint32_t *out, uint32_t *tmp, int64_t n, int passes,
                        void *scratch, size_t scratch_bytes, void *stream);

/* Comparison only: the multi-launch structure of the pages, ported so that
 * the single pass can be measured against it on this hardware. A scan is a
 * tree of tile scans (8192-element tiles; each level writes its tiles'
 * exclusive prefixes and one sum per tile, and the next level scans the
 * sums) with the carries added back level by level: 3 launches up to
 * 8192^2 elements ("Day 32 scan_2.cu": tile scan, scan of the tile sums,
 * add the offsets). A compaction marks the flags into `ranks`, scans them
 * there with that tree and scatters the survivors to out[rank], recomputing
 * the predicate: 7 launches at 2^28 elements ("Day 33 compaction.cu": mark,
 * scan, scatter). `ranks` (required, n words) ends as the exclusive scan of
 * the flags. Results equal those of ssc_exclusive_scan_i32 and
 * ssc_compact_i32; scratch (16-byte aligned, ssc_multipass_scratch_bytes
 * bytes) holds the tile sums; no overlap of the arrays is allowed, except
 * in == out for the scan. */
size_t ssc_multipass_scratch_bytes(int64_t n);
int ssc_exclusive_scan_multipass_i32(const int32_t *in, int32_t *out, int64_t n, int32_t *total,
                                     void *scratch, size_t scratch_bytes, void *stream);
int ssc_compact_multipass_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa,
                              int32_t pb, int32_t *count, int32_t *ranks, void *scratch,
                              size_t scratch_bytes, void *stream);

/* Comparison only, the separate steps of that multi-launch compaction, so
 * that each can be timed alone ("Day 33 compaction.cu", markNonZero /
 * markEven and scatterCompact, and its table of where the time goes):
 * ssc_mark_i32 writes flags[i] = P(in[i]) (0 or 1) for every i;
 * ssc_scatter_i32 writes out[ranks[i]] = in[i] for every i with P(in[i])
 * (the predicate evaluated again, not read back) given the exclusive scan
 * of the flags in `ranks`, and *count = ranks[n-1] + P(in[n-1]). A rank
 * outside [0, n) is skipped. No overlap of the arrays is allowed. */
int ssc_mark_i32(const int32_t *in, int32_t *flags, int64_t n, int pred, int32_t pa, int32_t pb,
                 void *stream);
int ssc_scatter_i32(const int32_t *in, const int32_t *ranks, int32_t *out, int64_t n, int pred,
                    int32_t pa, int32_t pb, int32_t *count, void *stream);

/* out[i] = in[i] with 128-bit nontemporal loads and stores (32-bit ones when
 * either array is not 16-byte aligned), one 256-thread workgroup per 4096
 * elements: the bandwidth reference the single pass is compared with ("Day
 * 33 compaction.cu", copyInts; "Day 32 scan_2.cu", copyFloats). No overlap
 * allowed. */
int ssc_copy_i32(const int32_t *in, int32_t *out, int64_t n, void *stream);

/* Human-readable name of a status code (static storage). */
const char *ssc_status_str(int status);

/* The hipError_t of the last SSC_ERR_HIP on the calling thread (0 if none). */
int ssc_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SSC_H */
