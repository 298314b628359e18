// Device-side building blocks for the single-pass kernels on gfx950 (CDNA4):
// wave64 lane helpers, ballot/mbcnt ranks, DPP wave scans, predicates, the
// packed tile descriptor and the decoupled look-back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssc {

constexpr int kWave = 64;

// ---------------------------------------------------------------- lanes ---

__device__ __forceinline__ int lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t mbcnt64(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ uint32_t uniform(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(x)));
}

// ------------------------------------------------------------ value ops ---
// Sum over uint32 (wraps modulo 2^32, which also serves int32 scans) and
// over fp32. `bits`/`from_bits` move values through 32-bit descriptors.

struct SumU32 {
    using T = uint32_t;
    __device__ static T zero() { return 0u; }
    __device__ static T add(T a, T b) { return a + b; }
    __device__ static uint32_t bits(T a) { return a; }
    __device__ static T from_bits(uint32_t b) { return b; }
};

struct SumF32 {
    using T = float;
    __device__ static T zero() { return 0.0f; }
    __device__ static T add(T a, T b) { return a + b; }
    __device__ static uint32_t bits(T a) { return __float_as_uint(a); }
    __device__ static T from_bits(uint32_t b) { return __uint_as_float(b); }
};

// DPP move with the identity (all-zero bits) written where the source lane
// is outside the pattern or the row is masked off.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_move(uint32_t x) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROW_MASK, 0xf, true));
}

// Inclusive scan across the 64 lanes of a wavefront: a Hillis-Steele scan
// inside each 16-lane row (row_shr 1, 2, 4, 8), then row 15's total is carried
// into the next row (row_bcast:15) and lane 31's into rows 2-3 (row_bcast:31).
template <class Op>
__device__ __forceinline__ typename Op::T wave_inclusive_scan(typename Op::T v) {
    uint32_t x = Op::bits(v);
    x = Op::bits(Op::add(Op::from_bits(x), Op::from_bits(dpp_move<0x111, 0xf>(x))));
    x = Op::bits(Op::add(Op::from_bits(x), Op::from_bits(dpp_move<0x112, 0xf>(x))));
    x = Op::bits(Op::add(Op::from_bits(x), Op::from_bits(dpp_move<0x114, 0xf>(x))));
    x = Op::bits(Op::add(Op::from_bits(x), Op::from_bits(dpp_move<0x118, 0xf>(x))));
    x = Op::bits(Op::add(Op::from_bits(x), Op::from_bits(dpp_move<0x142, 0xa>(x))));
    x = Op::bits(Op::add(Op::from_bits(x), Op::from_bits(dpp_move<0x143, 0xc>(x))));
    return Op::from_bits(x);
}

// Sum over all 64 lanes, result in every lane (butterfly through ds_swizzle-free
// lane shuffles; used only on the look-back path).
template <class Op>
__device__ __forceinline__ typename Op::T wave_sum(typename Op::T v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = Op::add(v, __shfl_xor(v, off));
    return v;
}

// ----------------------------------------------------------- predicates ---
// Numbering matches ssc_pred in ssc.h. PredArgs carries a predicate's
// arguments: `a` is the bit of BIT_SET/BIT_CLEAR and the modulus of MOD_LT,
// `b` the bound of MOD_LT (keep iff mod(x, a) < b, residue in [0, a)). The
// F32 predicates (6..9) read the 32-bit element and a, b as fp32 bits and
// compare with IEEE semantics (NaN compares false, -0.0 == 0.0).
//
// MOD_LT reads the residue off a fractional part, with constants the host
// computes once per call (make_pred_args): inv = 1/a rounded once, half =
// inv/2 and thr = b/a rounded once. t = fma(x, inv, half) is (x + 1/2)/a to
// within 2^-21/a for every int32 x, and (x + 1/2)/a = floor(x/a) + (r + 1/2)/a
// with r the non-negative residue, whose fractional part lies in [1/(2a),
// 1 - 1/(2a)]. The error is far inside that margin, so floor(t) = floor(x/a)
// and t - floor(t) (v_fract_f64, exact) is (r + 1/2)/a to within 2^-21/a,
// which is below b/a iff r < b, with 1/(2a) to spare on either side (b <= 0
// keeps nothing, b >= a everything). Four full-rate fp64 operations: convert,
// fma, fract, compare.
struct PredArgs {
    int32_t a, b;
    double inv, half, thr;  // MOD_LT: 1/a, 1/(2a), b/a
};

template <int P>
__device__ __forceinline__ bool pred_eval(int32_t x, const PredArgs &pr) {
    const uint32_t u = static_cast<uint32_t>(x);
    if constexpr (P == 0) {
        return x != 0;
    } else if constexpr (P == 1) {
        return (u & 1u) != 0u;
    } else if constexpr (P == 2) {
        return (u & 1u) == 0u;
    } else if constexpr (P == 3) {
        return ((u >> pr.a) & 1u) != 0u;
    } else if constexpr (P == 4) {
        return ((u >> pr.a) & 1u) == 0u;
    } else if constexpr (P == 6) {
        return __int_as_float(x) != 0.0f;
    } else if constexpr (P == 7) {
        return __int_as_float(x) > __int_as_float(pr.a);
    } else if constexpr (P == 8) {
        return __int_as_float(x) < __int_as_float(pr.a);
    } else if constexpr (P == 9) {
        const float f = __int_as_float(x);
        return __int_as_float(pr.a) <= f && f < __int_as_float(pr.b);
    } else {
        static_assert(P == 5, "predicate numbering");
        const double t = __builtin_fma(static_cast<double>(x), pr.inv, pr.half);
        return __builtin_amdgcn_fract(t) < pr.thr;
    }
}

// ------------------------------------------------------ tile descriptors ---
// One 64-bit word per tile: the low half holds a 32-bit value (a count, an
// int sum or fp32 bits); the high half holds (tag << 2) | status, where tag
// is the call's epoch modulo 2^30. Status and value are written and read as
// a single agent-scope atomic, so they always travel together. A word whose
// tag is not the current call's, or whose status is 0 (all-zero memory
// included), means "nothing published yet": descriptors never need clearing
// between calls.

constexpr uint32_t kStatusAggregate = 1;  // value = this tile's own total
constexpr uint32_t kStatusInclusive = 2;  // value = total of tiles 0..t
constexpr uint32_t kTagMask = 0x3FFFFFFFu;

__device__ __forceinline__ uint64_t descriptor(uint32_t tag, uint32_t status, uint32_t value) {
    return (static_cast<uint64_t>((tag << 2) | status) << 32) | value;
}

__device__ __forceinline__ void perturb(uint32_t key, uint32_t site);

__device__ __forceinline__ void publish(uint64_t *desc, uint32_t tag, uint32_t status,
                                        uint32_t value) {
    perturb(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(desc) >> 3), 2 + status);
    __hip_atomic_store(desc, descriptor(tag, status, value), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t peek(uint64_t *desc) {
    return __hip_atomic_load(desc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Decoupled look-back, run by one whole wavefront of the tile's workgroup.
//
// Waiting: first the wavefront polls only the immediate predecessor's
// descriptor (one lane, one 8-byte agent-scope load), sleeping SLEEP x 64
// clocks between polls, until it has published. Measured on MI355X: with
// one workgroup per tile (hundreds of tiles waiting at once), frequent
// coherent polling costs more throughput than it saves latency, and about
// 3.4 us (s_sleep 127) is best; the persistent compaction kernel, whose
// control wavefronts wait on tiles published earlier, polls at s_sleep 16.
//
// With PRED_FIRST false the wavefront skips that first wait and polls the
// window itself: for a caller whose predecessor has almost always published
// already, the lone poll is one coherent round trip spent for nothing.
//
// Walking: then each step reads the descriptors of the 64 tiles just below
// the window end at once (one load, 512 contiguous bytes). The window is
// usable once the nearest tile with an {inclusive} value is nearer than every
// tile that has published nothing in this call: the result is that value plus
// the aggregates above it. Unpublished tiles below it are never waited for
// (descriptor stores to different words need not become visible in order, so
// they do occur, and waiting on them measured 3% slower). With no inclusive
// value and no unpublished tile in the window, all aggregates are added and
// the window moves down; otherwise the window is polled again. Tiles below 0
// count as inclusive with value 0. Returns the exclusive prefix of `tile`
// (the total of tiles 0..tile-1) in every lane.
//
// Forward progress: a tile only waits on lower-numbered tiles, whose numbers
// were claimed earlier by workgroups that are already running and whose
// aggregates are published without waiting on anything; tile 0 never waits.
//
// The wait is bounded: after kSpinLimit polls without progress (far beyond
// any legitimate wait) the walk stops, *timed_out is set to 1 and the
// partial prefix is returned, so a fault elsewhere can corrupt results but
// can never leave the kernel spinning.
constexpr uint32_t kSpinLimit = 1u << 20;

// Timing perturbation for race testing, compiled in only with -DSSC_PERTURB
// (a separate test build; the library proper compiles it out). perturb(key,
// site) pauses the wavefront for 0 to 7 x 1024 clocks, chosen by a hash of a
// uniform key (a tile, a descriptor address, a workgroup) and the call site:
// before every tile claim, descriptor publication and data-wavefront
// arrival, and after every look-back poll. Tiles then publish, arrive and
// claim in orders the normal build rarely shows, with every wait still
// bounded.
#ifdef SSC_PERTURB
__device__ __forceinline__ void perturb(uint32_t key, uint32_t site) {
    uint32_t h = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(key)));
    h = h * 0x9E3779B1u ^ site * 0x85EBCA77u;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    for (uint32_t i = 0; i < (h & 7u); ++i) __builtin_amdgcn_s_sleep(16);
}
#else
__device__ __forceinline__ void perturb(uint32_t, uint32_t) {}
#endif

// One pause between look-back polls; key (the tile and the poll count) only
// feeds the perturbation.
template <int SLEEP>
__device__ __forceinline__ void poll_pause(uint32_t key) {
    __builtin_amdgcn_s_sleep(SLEEP);
    perturb(key, 1);
}

// Descriptor of tile idx (>= 0) read as base + 32-bit byte offset, so the
// address needs one VGPR; tiles below 0 read as inclusive with value 0.
__device__ __forceinline__ uint64_t peek_tile(uint64_t *desc, int32_t idx, uint32_t tag) {
    const uint32_t off = static_cast<uint32_t>(idx < 0 ? 0 : idx) * 8u;
    const uint64_t w = peek(reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(desc) + off));
    return idx < 0 ? descriptor(tag, kStatusInclusive, 0u) : w;
}

__device__ __forceinline__ uint32_t status_of(uint64_t word, uint32_t tag) {
    const uint32_t hi = static_cast<uint32_t>(word >> 32);
    return (hi >> 2) == tag ? (hi & 3u) : 0u;
}

// Windows of 64 descriptors read per step. Wider reads (2-4 windows) measured
// slower on MI355X: the extra coherent traffic costs more than the steps saved.
constexpr int kLookBackWindows = 1;

template <class Op, int SLEEP, bool PRED_FIRST = true>
__device__ typename Op::T look_back(uint64_t *desc, uint32_t tile, uint32_t tag,
                                    uint32_t *timed_out) {
    using T = typename Op::T;
    const int lane = lane_id();
    T prefix = Op::zero();
    uint32_t spins = 0;
    // wait on the immediate predecessor alone
    while (PRED_FIRST) {
        uint64_t w1 = 0;
        if (lane == 0) w1 = peek_tile(desc, static_cast<int32_t>(tile) - 1, tag);
        if (status_of(w1, tag) != 0u && lane == 0) spins |= 0x80000000u;
        if (uniform(spins) & 0x80000000u) break;
        if (++spins > kSpinLimit) {
            if (lane == 0)
                __hip_atomic_store(timed_out, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return prefix;
        }
        poll_pause<SLEEP>(tile * 64u + spins);
    }
    spins &= 0x7FFFFFFFu;
    int32_t end = static_cast<int32_t>(tile);
    while (true) {
        uint64_t word[kLookBackWindows];
        int stop_r = -1, top = -1;  // window and lane of the nearest inclusive tile
        while (true) {
#pragma unroll
            for (int r = 0; r < kLookBackWindows; ++r)
                word[r] = peek_tile(desc, end - (r + 1) * kWave + lane, tag);
            // nearest first (window 0, lane 63 = tile end-1): usable while the
            // nearest inclusive tile comes before any unpublished one
            bool ready = true;
            stop_r = -1;
            top = -1;
#pragma unroll
            for (int r = 0; r < kLookBackWindows; ++r) {
                if (stop_r < 0 && ready) {
                    const uint32_t st = status_of(word[r], tag);
                    const uint64_t unpublished = ballot(st == 0u);
                    const uint64_t inclusive = ballot(st == kStatusInclusive);
                    const int ti = inclusive ? 63 - __builtin_clzll(inclusive) : -1;
                    const int tx = unpublished ? 63 - __builtin_clzll(unpublished) : -1;
                    if (tx > ti) {
                        ready = false;
                    } else if (ti >= 0) {
                        stop_r = r;
                        top = ti;
                    }
                }
            }
            if (ready) break;
            if (++spins > kSpinLimit) {
                if (lane == 0)
                    __hip_atomic_store(timed_out, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return prefix;
            }
            poll_pause<SLEEP>(tile * 64u + spins);
        }
        // add the values from the nearest inclusive tile up (everything read
        // when there is none)
        T acc = Op::zero();
#pragma unroll
        for (int r = 0; r < kLookBackWindows; ++r) {
            const bool take = stop_r < 0 || r < stop_r || (r == stop_r && lane >= top);
            if (take) acc = Op::add(acc, Op::from_bits(static_cast<uint32_t>(word[r])));
        }
        const T all = wave_inclusive_scan<Op>(acc);
        prefix = Op::add(prefix, Op::from_bits(static_cast<uint32_t>(__builtin_amdgcn_readlane(
                                     static_cast<int>(Op::bits(all)), kWave - 1))));
        if (stop_r >= 0) return prefix;
        end -= kLookBackWindows * kWave;
    }
}

// ------------------------------------------------- wide (fp64) descriptors ---
// For fp32 scans with fp64 carries a tile's descriptor is two 64-bit words,
// each laid out as a narrow descriptor ((tag << 2) | status in the high
// half). Word 0 decides the status:
//   {aggregate}: word 0 alone, its low half the fp32 bits of the tile's sum
//     (a tile aggregate is an fp32 sum, so 32 bits hold it exactly);
//   {inclusive}: word 0 the high 32 bits of the fp64 prefix, word 1 (also
//     marked inclusive) the low 32 bits; word 1 is stored first.
// A reader whose word 0 says inclusive but whose word 1 does not yet carry
// this call's tag and the inclusive status reads the tile as unpublished and
// polls again; word 1 is written by the inclusive store alone, so that wait
// ends. The aggregate (a data wavefront) and the inclusive stores (the
// control wavefront, a barrier later) are not ordered by a fence: should the
// aggregate's word 0 land last, the tile reads as {aggregate} with its
// correct value from then on and readers walk past it. No interleaving of
// the stores leaves a tile unreadable.
__device__ __forceinline__ void publish_wide(uint64_t *desc, uint32_t tile, uint32_t tag,
                                             uint32_t status, double value) {
    uint64_t *p = desc + 2 * static_cast<uint64_t>(tile);
    perturb(tile, 5 + status);
    if (status == kStatusAggregate) {
        __hip_atomic_store(p, descriptor(tag, status, __float_as_uint(static_cast<float>(value))),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(value));
    __hip_atomic_store(p + 1, descriptor(tag, status, static_cast<uint32_t>(b)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p, descriptor(tag, status, static_cast<uint32_t>(b >> 32)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Status and value of tile idx's wide descriptor; tiles below 0 read as
// inclusive with value 0.
__device__ __forceinline__ uint32_t peek_wide(uint64_t *desc, int32_t idx, uint32_t tag,
                                              double &value) {
    const uint32_t off = static_cast<uint32_t>(idx < 0 ? 0 : idx) * 16u;
    uint64_t *p = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(desc) + off);
    const uint64_t hi = peek(p);
    const uint64_t lo = peek(p + 1);
    if (idx < 0) {
        value = 0.0;
        return kStatusInclusive;
    }
    const uint32_t sh = status_of(hi, tag);
    if (sh == kStatusAggregate) {
        value = static_cast<double>(__uint_as_float(static_cast<uint32_t>(hi)));
        return sh;
    }
    value = __longlong_as_double(static_cast<long long>((hi << 32) | (lo & 0xFFFFFFFFull)));
    return sh == kStatusInclusive && status_of(lo, tag) == kStatusInclusive ? sh : 0u;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// The look-back of `look_back` over wide descriptors: the same waiting,
// windows, stopping rule and time-out, summing the values in fp64. Returns
// the exclusive prefix of `tile` in every lane. PRED_FIRST as for
// look_back (the persistent scan, whose look-back has a whole tile period,
// goes straight to the window: 2^28 fp32 370.1 -> 362.7 us).
template <int SLEEP, bool PRED_FIRST = true>
__device__ double look_back_wide(uint64_t *desc, uint32_t tile, uint32_t tag,
                                 uint32_t *timed_out) {
    const int lane = lane_id();
    double prefix = 0.0;
    uint32_t spins = 0;
    while (PRED_FIRST) {
        uint32_t st = 0;
        if (lane == 0) {
            double unused;
            st = peek_wide(desc, static_cast<int32_t>(tile) - 1, tag, unused);
        }
        if (uniform(st) != 0u) break;
        if (++spins > kSpinLimit) {
            if (lane == 0)
                __hip_atomic_store(timed_out, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return prefix;
        }
        poll_pause<SLEEP>(tile * 64u + spins);
    }
    int32_t end = static_cast<int32_t>(tile);
    while (true) {
        double val = 0.0;
        int top = -1;  // lane of the nearest inclusive tile
        while (true) {
            const uint32_t st = peek_wide(desc, end - kWave + lane, tag, val);
            const uint64_t unpublished = ballot(st == 0u);
            const uint64_t inclusive = ballot(st == kStatusInclusive);
            const int ti = inclusive ? 63 - __builtin_clzll(inclusive) : -1;
            const int tx = unpublished ? 63 - __builtin_clzll(unpublished) : -1;
            if (tx <= ti) {
                top = ti;
                break;
            }
            if (++spins > kSpinLimit) {
                if (lane == 0)
                    __hip_atomic_store(timed_out, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return prefix;
            }
            poll_pause<SLEEP>(tile * 64u + spins);
        }
        prefix += wave_sum_f64(lane >= top ? val : 0.0);
        if (top >= 0) return prefix;
        end -= kWave;
    }
}

}  // namespace ssc
